"""Each plausible mistake planted in the attention oracle (on the CPU) must be caught by the
pins: torch SDPA in float64, the generator's logical rows, or the exact-merge check."""
import math

import numpy as np
import pytest
import torch

import oracle.attention as A
import workloads as W
from tests.test_oracle_attention import sdpa_decode


def _batch():
    # d == B so that a transposed read of the value block does not fail on shape alone
    return W.small_batch([7, 33, 50], 8, 2, 16, 16, torch.float32, seed=123, poison=True)


def _agrees_with_sdpa(b):
    got = A.paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, b.block_size)
    return np.allclose(got, sdpa_decode(b), rtol=0, atol=1e-12)


def test_unmodified_oracle_passes():
    assert _agrees_with_sdpa(_batch())


def test_dropped_scale_is_caught(monkeypatch):
    orig = A.attend
    monkeypatch.setattr(A, "attend", lambda q, K, V, s: orig(q, K, V, 1.0))
    assert not _agrees_with_sdpa(_batch())


def test_wrong_sign_is_caught(monkeypatch):
    def bad(q, K, V, s):
        z = -(A._f64(K) @ A._f64(q)) * s
        w = np.exp(z - z.max())
        return (w @ A._f64(V)) / w.sum()
    monkeypatch.setattr(A, "attend", bad)
    assert not _agrees_with_sdpa(_batch())


def test_transposed_value_block_is_caught(monkeypatch):
    def bad_gather(k_pool, v_pool, table_row, length, kv_head, block_size):
        pos = np.arange(int(length))
        phys = np.asarray(table_row, dtype=np.int64)[pos // block_size]
        off = pos % block_size
        # value block read as if stored [d][B] (head-dim rows and token slots swapped)
        return A._index(k_pool, phys, kv_head, off), \
            A._index(v_pool.transpose(2, 3), phys, kv_head, off)
    monkeypatch.setattr(A, "gather_kv", bad_gather)
    assert not _agrees_with_sdpa(_batch())


def test_wrong_head_grouping_is_caught(monkeypatch):
    b = _batch()
    G = b.num_q_heads // b.num_kv_heads

    def bad_decode(q, k_pool, v_pool, tables, lengths, block_size, scale=None, seqs=None):
        S, Hq, d = q.shape
        out = np.zeros((S, Hq, d))
        for s in range(S):
            for h in range(Hq):
                K, V = A.gather_kv(k_pool, v_pool, tables[s], int(lengths[s]),
                                   h % k_pool.shape[1], block_size)
                out[s, h] = A.attend(A._f64(q)[s, h], K, V, 1 / math.sqrt(d))
        return out
    assert G > 1
    monkeypatch.setattr(A, "paged_decode", bad_decode)
    assert not _agrees_with_sdpa(b)


def test_reading_padding_slots_is_caught(monkeypatch):
    orig = A.gather_kv

    def bad_gather(k_pool, v_pool, table_row, length, kv_head, block_size):
        whole = -(-int(length) // block_size) * block_size     # every slot of the last block
        return orig(k_pool, v_pool, table_row, whole, kv_head, block_size)
    monkeypatch.setattr(A, "gather_kv", bad_gather)
    assert not _agrees_with_sdpa(_batch())


def test_wrong_merge_weight_is_caught(monkeypatch):
    def bad_merge(states):
        ms = np.array([s[0] for s in states])
        m_star = ms.max()
        num = sum(math.exp(m_star - m) * acc for m, l, acc in states)
        den = sum(math.exp(m_star - m) * l for m, l, acc in states)
        return num / den
    b = W.small_batch([100, 300], 4, 4, 16, 16, torch.float32, seed=4)
    ref = sdpa_decode(b)
    good = A.paged_decode_split(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16, 64)
    assert np.allclose(good, ref, atol=1e-12)
    monkeypatch.setattr(A, "merge_states", bad_merge)
    bad = A.paged_decode_split(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16, 64)
    assert not np.allclose(bad, ref, atol=1e-6)
