"""Pins of the attention oracle to things other than itself: torch's scaled-dot-product
attention in float64 (a library routine, with its own GQA head grouping), closed forms,
the pages' exactness and invariance statements, and the generator's logical data."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import workloads as W
from oracle import (attend, contiguous_decode, gather_kv, merge_states, paged_decode,
                    paged_decode_split, partial_state, token_address)


def sdpa_decode(batch):
    """Reference by torch SDPA (float64, CPU): one query per head over the logical K/V."""
    out = []
    for s in range(batch.num_seqs):
        q = batch.q[s].to(torch.float64)[None, :, None, :]          # [1][Hq][1][d]
        k = batch.k_logical[s].to(torch.float64)[None]               # [1][Hkv][L][d]
        v = batch.v_logical[s].to(torch.float64)[None]
        o = F.scaled_dot_product_attention(q, k, v, enable_gqa=True)  # scale 1/sqrt(d)
        out.append(o[0, :, 0, :].numpy())
    return np.stack(out)


CASES = [
    # lengths, Hq, Hkv, d, B, dtype
    ([1, 17, 70, 16, 33], 4, 4, 64, 16, torch.float32),
    ([5, 64, 31], 8, 2, 16, 32, torch.float16),
    ([40, 2, 48], 16, 2, 8, 16, torch.bfloat16),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_matches_sdpa(case):
    lengths, hq, hkv, d, B, dt = CASES[case]
    b = W.small_batch(lengths, hq, hkv, d, B, dt, seed=11 + case, poison=True)
    ref = sdpa_decode(b)
    got = paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, B)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    cont = contiguous_decode(b.q, b.k_logical, b.v_logical)
    assert np.allclose(cont, ref, rtol=0, atol=1e-12)


def test_gather_returns_logical_rows():
    b = W.small_batch([3, 16, 45, 77], 4, 2, 32, 16, torch.bfloat16, seed=5, poison=True)
    for s in range(b.num_seqs):
        for g in range(2):
            K, V = gather_kv(b.k_pool, b.v_pool, b.tables[s], int(b.lengths[s]), g, 16)
            assert np.array_equal(K, b.k_logical[s][g].double().numpy())
            assert np.array_equal(V, b.v_logical[s][g].double().numpy())
            # and the vectorised rule agrees with the scalar one, token by token
            for p in range(int(b.lengths[s])):
                blk, r = token_address(p, b.tables[s], 16)
                assert np.array_equal(K[p], b.k_pool[blk, g, r].double().numpy())
                assert np.array_equal(V[p], b.v_pool[blk, g, r].double().numpy())


def test_closed_forms():
    rng = np.random.default_rng(3)
    d = 8
    q = rng.standard_normal(d)
    V = rng.standard_normal((5, d))
    K = rng.standard_normal((5, d))
    s = 1 / math.sqrt(d)
    # one token: the output is that token's value, exactly
    assert np.array_equal(attend(q, K[:1], V[:1], s), V[0])
    # zero query or identical keys: the plain mean of the values
    assert np.allclose(attend(np.zeros(d), K, V, s), V.mean(0), atol=1e-15)
    assert np.allclose(attend(q, np.repeat(K[:1], 5, 0), V, s), V.mean(0), atol=1e-15)
    # two tokens: a logistic blend
    z0, z1 = K[0] @ q * s, K[1] @ q * s
    w1 = 1.0 / (1.0 + math.exp(z0 - z1))
    assert np.allclose(attend(q, K[:2], V[:2], s), V[0] + w1 * (V[1] - V[0]), atol=1e-15)
    # shifting all scores leaves the output unchanged; scaling q changes it
    assert np.allclose(attend(q, K + 0.0, V, s), attend(q, K, V, s), atol=0)
    assert not np.allclose(attend(2 * q, K, V, s), attend(q, K, V, s))
    # empty context
    assert np.array_equal(attend(q, K[:0], V[:0], s), np.zeros(d))


def test_spike_selects_the_addressed_slot():
    """Config-1 shape: making key 37 of the 47-token request a large multiple of the query
    drives its softmax weight to 1, so the output is the value stored at block 9, offset 5."""
    b = W.config1()
    s, h = 1, 2
    blk, off = token_address(37, b.tables[s], 16)
    assert (blk, off) == (9, 5)
    kp = b.k_pool.clone()
    kp[blk, h, off] = 40.0 * b.q[s, h]
    out = paged_decode(b.q, kp, b.v_pool, b.tables, b.lengths, 16, seqs=[s])
    assert np.allclose(out[s, h], b.v_pool[blk, h, off].double().numpy(), atol=1e-12)


def test_split_merge_is_exact():
    b = W.small_batch([1, 16, 100, 257, 512, 513], 8, 2, 32, 16, torch.bfloat16, seed=9)
    ref = paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    for part in (16, 32, 64, 512):
        got = paged_decode_split(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16, part)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_merge_of_partials():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(4)
    K = rng.standard_normal((9, 4)) * 3
    V = rng.standard_normal((9, 4))
    s = 0.5
    states = [partial_state(q, K[i:i + 2], V[i:i + 2], s) for i in range(0, 9, 2)]
    states.append(partial_state(q, K[:0], V[:0], s))          # an empty partition
    assert np.allclose(merge_states(states), attend(q, K, V, s), atol=1e-14)
    m, l, acc = partial_state(q, K, V, s)
    z = K @ q * s
    assert m == z.max() and np.isclose(l, np.exp(z - m).sum())
    assert np.array_equal(merge_states([partial_state(q, K[:0], V[:0], s)]), np.zeros(4))


def test_placement_invariance():
    b = W.small_batch([30, 64, 5], 4, 4, 16, 16, torch.float16, seed=21)
    r = W.relabel(b, 77)
    assert not np.array_equal(r.tables, b.tables)
    o1 = paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, 16)
    o2 = paged_decode(r.q, r.k_pool, r.v_pool, r.tables, r.lengths, 16)
    assert np.array_equal(o1, o2)


def test_shared_prefix_equals_private_copies():
    shared = W.config4a(num_seqs=4, prefix_len=64)
    private = W.config4a_private(shared)
    assert len(set(shared.tables[:, 0])) == 1 and len(set(private.tables[:, 0])) == 4
    o1 = paged_decode(shared.q, shared.k_pool, shared.v_pool, shared.tables, shared.lengths, 16)
    o2 = paged_decode(private.q, private.k_pool, private.v_pool, private.tables,
                      private.lengths, 16)
    assert np.array_equal(o1, o2)
    assert np.allclose(o1, sdpa_decode(shared), atol=1e-12)



@settings(max_examples=60, deadline=None)
@given(lengths=st.lists(st.integers(0, 70), min_size=1, max_size=4),
       block_size=st.sampled_from([16, 32]), group=st.sampled_from([1, 2, 8]),
       hkv=st.sampled_from([1, 2]), d=st.sampled_from([8, 16]),
       dtype=st.sampled_from([torch.float32, torch.bfloat16]), seed=st.integers(0, 10_000))
def test_random_small_cases_match_sdpa(lengths, block_size, group, hkv, d, dtype, seed):
    """Random small batches (S <= 4, L <= 70, empty contexts included, both block sizes,
    G in {1, 2, 8}): the paged oracle equals torch SDPA on the logical rows (zero rows for
    empty contexts), with poisoned unused slots and random placement."""
    b = W.small_batch(lengths, hkv * group, hkv, d, block_size, dtype, seed=seed, poison=True)
    got = paged_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lengths, block_size)
    for s, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(got[s], np.zeros_like(got[s]))
        else:
            q = b.q[s].to(torch.float64)[None, :, None, :]
            k = b.k_logical[s].to(torch.float64)[None]
            v = b.v_logical[s].to(torch.float64)[None]
            ref = F.scaled_dot_product_attention(q, k, v, enable_gqa=True)[0, :, 0, :].numpy()
            assert np.allclose(got[s], ref, rtol=0, atol=1e-12)
