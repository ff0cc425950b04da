"""Pins of the shared-prefix decode oracle: it must reach the plain definition (torch SDPA in
float64 over the generator's logical rows, which never went through a block table) to 1e-12,
since a prefix/suffix split merged with the log-sum-exp rule is exact; planted mistakes (a
suffix off by one token, a dropped prefix state, the prefix read through the wrong KV head)
must fail that pin."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as A
import workloads as W


def _sdpa(b):
    """softmax(q K^T / sqrt(d)) V per sequence and head, float64, from the logical rows."""
    S, Hq, d = b.q.shape
    G = Hq // b.num_kv_heads
    out = np.zeros((S, Hq, d))
    for s in range(S):
        K = b.k_logical[s].double()
        V = b.v_logical[s].double()
        q = b.q[s].double()
        for h in range(Hq):
            z = (K[h // G] @ q[h]) / np.sqrt(d)
            out[s, h] = (torch.softmax(z, 0) @ V[h // G]).numpy()
    return out


def _run(b, P):
    return oracle.shared_prefix_decode(b.q, b.k_pool, b.v_pool, b.tables[0][:P // b.block_size],
                                       P, b.tables, b.lengths, b.block_size)


CASES = [
    # suffix lengths, prefix, Hq, Hkv, d, B, dtype
    ([5, 40, 1, 17], 64, 8, 2, 16, 16, torch.float32),
    ([0, 33, 2], 96, 4, 1, 8, 32, torch.float32),
    ([31, 32, 0, 100, 7], 32, 6, 3, 16, 16, torch.bfloat16),
    ([12], 16, 2, 2, 8, 16, torch.float16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"P{c[1]}-G{c[2] // c[3]}-B{c[5]}")
def test_matches_sdpa_on_logical_rows(case):
    suf, P, hq, hkv, d, B, dt = case
    seed = zlib.crc32(repr(case).encode()) % 1000
    b = W.shared_prefix_batch(suf, P, hq, hkv, d, B, dt, seed=seed, poison=True)
    got = _run(b, P)
    assert np.allclose(got, _sdpa(b), rtol=0, atol=1e-12)
    # and the plain paged oracle over the full tables agrees
    ref = oracle.paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_shared_prefix_config_sample():
    """Six sequences of the shared-prefix workload's recipe with an 800-token prefix."""
    b = W.config4a(num_seqs=6, prefix_len=800)
    assert np.allclose(_run(b, 800), _sdpa(b), rtol=0, atol=1e-12)


def test_contract_violations_raise():
    b = W.shared_prefix_batch([4, 9], 32, 4, 2, 8, 16, torch.float32, seed=3)
    with pytest.raises(ValueError):
        oracle.shared_prefix_decode(b.q, b.k_pool, b.v_pool, b.tables[0][:2], 24, b.tables,
                                    b.lengths, 16)
    short = b.lengths.copy()
    short[1] = 20
    with pytest.raises(ValueError):
        oracle.shared_prefix_decode(b.q, b.k_pool, b.v_pool, b.tables[0][:2], 32, b.tables,
                                    short, 16)


def _planted(monkeypatch, make_bad):
    b = W.shared_prefix_batch([5, 40, 17], 64, 8, 2, 16, 16, torch.float32, seed=9)
    orig = A.partial_state
    calls = {"n": 0}

    def bad(q, K, V, scale):
        calls["n"] += 1
        return make_bad(orig, calls["n"], q, K, V, scale)
    monkeypatch.setattr(A, "partial_state", bad)
    got = _run(b, 64)
    return np.allclose(got, _sdpa(b), rtol=0, atol=1e-12)


def test_dropped_prefix_state_is_caught(monkeypatch):
    # odd calls are prefix states (prefix first, then suffix, per row)
    assert not _planted(monkeypatch, lambda o, n, q, K, V, s:
                        (-np.inf, 0.0, np.zeros(V.shape[1])) if n % 2 else o(q, K, V, s))


def test_suffix_off_by_one_is_caught(monkeypatch):
    assert not _planted(monkeypatch, lambda o, n, q, K, V, s:
                        o(q, K[1:], V[1:], s) if n % 2 == 0 and len(K) > 1 else o(q, K, V, s))


def test_prefix_from_wrong_kv_head_is_caught(monkeypatch):
    b = W.shared_prefix_batch([5, 40, 17], 64, 8, 2, 16, 16, torch.float32, seed=9)
    orig = A._index

    def bad(pool, phys, kv_head, offset):
        if len(phys) == 64:                           # the prefix gather
            return orig(pool, phys, (kv_head + 1) % 2, offset)
        return orig(pool, phys, kv_head, offset)
    monkeypatch.setattr(A, "_index", bad)
    assert not np.allclose(_run(b, 64), _sdpa(b), rtol=0, atol=1e-12)
