"""Pins of the multi-query (extend) attention oracle: causal attention of each sequence's new
query tokens over its cached tokens. Pinned to torch SDPA in float64 with an explicit causal
mask over the generator's logical rows (never paged); one new token per sequence reduces to
the decode oracle; planted mistakes (causal boundary off by one, no causal mask, queries read
from the wrong sequence) fail the SDPA pin."""
import numpy as np
import pytest
import torch

import oracle
import oracle.attention as A
import workloads as W


def _sdpa(b, q, start):
    """Row (start[s] + t, h): softmax over positions <= L_s - n_s + t of sequence s."""
    T, Hq, d = q.shape
    G = Hq // b.num_kv_heads
    out = np.zeros((T, Hq, d))
    for s in range(len(start) - 1):
        n = int(start[s + 1] - start[s])
        if n == 0:
            continue
        L = int(b.lengths[s])
        K = b.k_logical[s].double()                  # [Hkv][L][d]
        V = b.v_logical[s].double()
        Q = q[start[s]:start[s + 1]].double()         # [n][Hq][d]
        pos = torch.arange(L - n, L)                  # positions of the new tokens
        mask = torch.arange(L)[None, :] <= pos[:, None]          # [n][L]
        for h in range(Hq):
            z = (Q[:, h] @ K[h // G].T) / np.sqrt(d)
            z = z.masked_fill(~mask, float("-inf"))
            out[start[s]:start[s + 1], h] = (torch.softmax(z, -1) @ V[h // G]).numpy()
    return out


CASES = [
    # lengths (including the new tokens), new tokens per sequence, Hq, Hkv, d, B, dtype
    ([40, 17, 64, 5], [3, 1, 16, 5], 8, 2, 16, 16, torch.float32),
    ([100, 33], [33, 0], 4, 4, 8, 32, torch.float32),
    ([31, 70, 9], [8, 70, 2], 6, 3, 16, 16, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{len(c[0])}-G{c[2] // c[3]}-B{c[5]}")
def test_matches_causal_sdpa(case):
    lens, new, hq, hkv, d, B, dt = case
    b = W.small_batch(lens, hq, hkv, d, B, dt, seed=31, poison=True)
    q, start = W.extend_queries(b, new, seed=32)
    got = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    assert np.allclose(got, _sdpa(b, q, start), rtol=0, atol=1e-12)


def test_one_new_token_is_the_decode():
    b = W.small_batch([12, 50, 1, 33], 8, 2, 16, 16, torch.float32, seed=5)
    q, start = W.extend_queries(b, [1, 1, 1, 1], seed=6)
    got = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    ref = oracle.paged_decode(q, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_row_with_nothing_to_attend_is_zero():
    b = W.small_batch([3], 2, 1, 8, 16, torch.float32, seed=7)
    q, start = W.extend_queries(b, [5], seed=8)       # 5 new tokens but only 3 stored
    got = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    assert np.all(got[:2] == 0) and np.all(np.isfinite(got))
    # rows 2..4 see positions 0..0, 0..1, 0..2
    ref = _sdpa_rows(b, q, 3)
    assert np.allclose(got[2:], ref, rtol=0, atol=1e-12)


def _sdpa_rows(b, q, L):
    K = b.k_logical[0].double()[0]
    V = b.v_logical[0].double()[0]
    out = []
    for t, upto in zip(range(2, 5), (1, 2, 3)):
        rows = []
        for h in range(2):
            z = (K[:upto] @ q[t, h].double()) / np.sqrt(8)
            rows.append((torch.softmax(z, 0) @ V[:upto]).numpy())
        out.append(rows)
    return np.array(out)


def _with_planted(monkeypatch, bad_attend_len):
    b = W.small_batch([40, 17, 64], 8, 2, 16, 16, torch.float32, seed=41)
    q, start = W.extend_queries(b, [3, 2, 9], seed=42)
    orig = A.gather_kv

    def gather(k_pool, v_pool, table_row, length, kv_head, block_size):
        return orig(k_pool, v_pool, table_row, bad_attend_len(length), kv_head, block_size)
    monkeypatch.setattr(A, "gather_kv", gather)
    got = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    return np.allclose(got, _sdpa(b, q, start), rtol=0, atol=1e-12)


def test_causal_off_by_one_is_caught(monkeypatch):
    assert not _with_planted(monkeypatch, lambda n: max(n - 1, 1))


def test_missing_causal_mask_is_caught(monkeypatch):
    b = W.small_batch([40, 17, 64], 8, 2, 16, 16, torch.float32, seed=41)
    q, start = W.extend_queries(b, [3, 2, 9], seed=42)
    orig = A.gather_kv

    def whole_context(k_pool, v_pool, table_row, length, kv_head, block_size):
        s = next(i for i in range(b.num_seqs) if np.array_equal(b.tables[i], table_row))
        return orig(k_pool, v_pool, table_row, int(b.lengths[s]), kv_head, block_size)
    monkeypatch.setattr(A, "gather_kv", whole_context)
    got = oracle.extend_attention(q, start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    assert not np.allclose(got, _sdpa(b, q, start), rtol=0, atol=1e-12)


def test_queries_of_wrong_sequence_are_caught():
    b = W.small_batch([40, 17, 64], 8, 2, 16, 16, torch.float32, seed=41)
    q, start = W.extend_queries(b, [3, 2, 9], seed=42)
    bad_start = start.copy()
    bad_start[1] += 1                                   # rows shifted between sequences
    got = oracle.extend_attention(q, bad_start, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    assert not np.allclose(got, _sdpa(b, q, start), rtol=0, atol=1e-12)
