"""Pins of the swap part of the bookkeeping oracle ("Paged Attention and vLLM", section
"Continuous Batching and Scheduler": a preempted sequence's blocks go to CPU memory a block at a
time and come back when it resumes). The pages print no worked swap example, so the pins are
brute force over flat element offsets, the generator's logical rows (independent of the oracle),
the attention value before and after a preempt/resume cycle, and reference-count invariants."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import BlockPool, PagedKVModel, copy_blocks


def _flat_copy(dst, src, src_ids, dst_ids):
    """Element by element over flat offsets ((blk * H + g) * B + r) * d + c."""
    N_src, H, B, d = src.shape
    out = dst.reshape(-1).copy()
    flat = src.reshape(-1)
    for s, t in zip(src_ids, dst_ids):
        if not (0 <= s < N_src and 0 <= t < dst.shape[0]):
            continue
        for g in range(H):
            for r in range(B):
                for c in range(d):
                    out[((t * H + g) * B + r) * d + c] = flat[((s * H + g) * B + r) * d + c]
    return out.reshape(dst.shape)


@pytest.mark.parametrize("src_ids,dst_ids", [
    ([3, 0, 5], [1, 4, 0]),
    ([2, 9, 1, 7], [0, 2, -1, 3]),      # out-of-range ids on either side are skipped
    ([], []),
])
def test_copy_blocks_matches_flat_offsets(src_ids, dst_ids):
    rng = np.random.default_rng(5)
    sk = rng.standard_normal((6, 2, 4, 3))
    sv = rng.standard_normal((6, 2, 4, 3))
    dk = rng.standard_normal((5, 2, 4, 3))
    dv = rng.standard_normal((5, 2, 4, 3))
    want_k, want_v = _flat_copy(dk, sk, src_ids, dst_ids), _flat_copy(dv, sv, src_ids, dst_ids)
    n = copy_blocks(dk, dv, sk, sv, src_ids, dst_ids)
    assert n == sum(0 <= s < 6 and 0 <= t < 5 for s, t in zip(src_ids, dst_ids))
    assert np.array_equal(dk, want_k) and np.array_equal(dv, want_v)


def _model_from_batch(b, extra_blocks=0):
    """The batch's pools as numpy (values only copied), a pool with its blocks referenced."""
    k = b.k_pool.numpy().copy()
    v = b.v_pool.numpy().copy()
    if extra_blocks:
        pad = np.zeros((extra_blocks,) + k.shape[1:], k.dtype)
        k, v = np.concatenate([k, pad]), np.concatenate([v, pad])
    pool = BlockPool(k.shape[0])
    m = PagedKVModel(pool, k, v, b.block_size)
    for s in range(b.num_seqs):
        row = [int(x) for x in b.tables[s] if x >= 0]
        for blk in row:
            pool.claim(blk)
        m.add_sequence(s, row, int(b.lengths[s]))
    return m


def _decode(m, b, q, seqs):
    tables = m.table_array(seqs, b.max_blocks_per_seq)
    lens = np.array([m.lengths[s] for s in seqs], np.int32)
    return oracle.paged_decode(q[seqs], m.k, m.v, tables, lens, b.block_size)


def test_preempt_and_resume_restores_every_row():
    b = W.small_batch([40, 17, 64, 5], 8, 2, 16, 16, torch.float32, seed=11)
    m = _model_from_batch(b, extra_blocks=8)
    before = _decode(m, b, b.q, [0, 1, 2, 3])
    free0 = m.pool.num_free()
    group = [1, 2]
    nblk = sum(len(m.tables[s]) for s in group)
    host = BlockPool(nblk + 2)
    hk = np.full((nblk + 2,) + m.k.shape[1:], np.nan)
    hv = np.full_like(hk, np.nan)
    out_pairs = m.swap_out(group, host, hk, hv)
    # the cost is the evicted blocks: one copy per distinct block of the group
    assert len(out_pairs) == nblk == m.pool.num_free() - free0
    assert host.num_free() == 2
    # another request reuses the freed device blocks and overwrites them
    for dev, _ in out_pairs:
        m.pool.claim(dev)
        m.k[dev] = 1e3
        m.v[dev] = -1e3
        m.pool.decref(dev)
    # resume into the highest free blocks, so every block lands somewhere new
    free = sorted((x for x in range(m.k.shape[0]) if m.pool.refcount(x) == 0), reverse=True)
    in_pairs = m.swap_in(group, host, hk, hv, claims=free[:nblk])
    assert host.num_free() == nblk + 2
    assert [h for h, _ in in_pairs] == [h for _, h in out_pairs]
    assert all(dev not in {d for d, _ in out_pairs} for _, dev in in_pairs)
    # every token of the resumed sequences reads its generator row through the new table
    for s in group:
        for g in range(b.num_kv_heads):
            K, V = oracle.gather_kv(m.k, m.v, m.tables[s], m.lengths[s], g, b.block_size)
            assert np.array_equal(K, b.k_logical[s][g].numpy())
            assert np.array_equal(V, b.v_logical[s][g].numpy())
    after = _decode(m, b, b.q, [0, 1, 2, 3])
    assert np.array_equal(before, after)


def test_group_sharing_a_block_copies_it_once():
    """Two forks that share every block are swapped out together: each shared block moves
    once, and its host block carries both references; a third sharer outside the group keeps
    the device block alive."""
    pool = BlockPool(10)
    k = np.arange(10 * 1 * 4 * 2, dtype=np.float64).reshape(10, 1, 4, 2)
    v = -k
    m = PagedKVModel(pool, k, v, 4)
    m.add_sequence("a", [pool.alloc(), pool.alloc()], 6)   # blocks 0, 1
    m.fork("a", "b")
    m.fork("a", "c")
    m.append("b", np.full((1, 2), 7.0), np.full((1, 2), -7.0))   # copy-on-write of block 1
    assert m.tables["b"] == [0, 2] and m.copies == [(1, 2, 2)]
    host = BlockPool(4)
    hk, hv = np.zeros((4, 1, 4, 2)), np.zeros((4, 1, 4, 2))
    pairs = m.swap_out(["a", "b"], host, hk, hv)
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert [host.refcount(x) for x in range(3)] == [2, 1, 1]
    # blocks 0 and 1 stay resident for "c" (one reference left), block 2 is free again
    assert [pool.refcount(x) for x in range(3)] == [1, 1, 0]
    assert np.array_equal(hk[:3], k[:3]) and np.array_equal(hv[:3], v[:3])
    back = m.swap_in(["a", "b"], host, hk, hv, claims=[7, 8, 9])
    assert back == [(0, 7), (1, 8), (2, 9)]
    assert m.tables["a"] == [7, 8] and m.tables["b"] == [7, 9] and m.tables["c"] == [0, 1]
    assert [pool.refcount(x) for x in (7, 8, 9)] == [2, 1, 1]
    assert host.num_free() == 4
    assert np.array_equal(k[7], k[0]) and np.array_equal(k[9, 0, 2], [7.0, 7.0])
    with pytest.raises(ValueError):
        m.swap_in(["a"], host, hk, hv)


def test_swap_out_twice_is_rejected():
    pool = BlockPool(4)
    m = PagedKVModel(pool, np.zeros((4, 1, 4, 1)), np.zeros((4, 1, 4, 1)), 4)
    m.add_sequence(0, [pool.alloc()], 3)
    host = BlockPool(2)
    hk, hv = np.zeros((2, 1, 4, 1)), np.zeros((2, 1, 4, 1))
    m.swap_out([0], host, hk, hv)
    with pytest.raises(ValueError):
        m.swap_out([0], host, hk, hv)


def test_planted_mistakes_are_caught(monkeypatch):
    """A swap that copies keys only, or indexes the destination with the source id, fails the
    flat-offset pin; a swap-in that forgets the second reference of a shared block fails the
    reference-count pin."""
    import oracle.bookkeeping as BK
    rng = np.random.default_rng(1)
    sk, sv = rng.standard_normal((4, 1, 2, 2)), rng.standard_normal((4, 1, 2, 2))

    def keys_only(dk, dv, sk_, sv_, si, di):
        for s, d in zip(si, di):
            dk[d] = sk_[s]
        return len(si)

    def wrong_index(dk, dv, sk_, sv_, si, di):
        for s, d in zip(si, di):
            dk[s], dv[s] = sk_[s], sv_[s]
        return len(si)

    for bad in (keys_only, wrong_index):
        dk, dv = np.zeros((4, 1, 2, 2)), np.zeros((4, 1, 2, 2))
        bad(dk, dv, sk, sv, [0, 2], [3, 1])
        assert not (np.array_equal(dk, _flat_copy(np.zeros_like(dk), sk, [0, 2], [3, 1])) and
                    np.array_equal(dv, _flat_copy(np.zeros_like(dv), sv, [0, 2], [3, 1])))

    orig_incref = BK.BlockPool.incref
    pool = BlockPool(6)
    m = PagedKVModel(pool, np.zeros((6, 1, 2, 1)), np.zeros((6, 1, 2, 1)), 2)
    m.add_sequence("a", [pool.alloc()], 2)
    m.fork("a", "b")
    host = BlockPool(2)
    hk, hv = np.zeros((2, 1, 2, 1)), np.zeros((2, 1, 2, 1))
    m.swap_out(["a", "b"], host, hk, hv)
    monkeypatch.setattr(BK.BlockPool, "incref", lambda self, blk: None)
    m.swap_in(["a", "b"], host, hk, hv)
    monkeypatch.setattr(BK.BlockPool, "incref", orig_incref)
    assert pool.refcount(m.tables["a"][0]) != 2      # the pin that would catch it
