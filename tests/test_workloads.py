"""The seeded generators: determinism, shapes and the structure each workload promises."""
import numpy as np
import torch

import workloads as W


def test_config1_structure():
    b = W.config1()
    assert list(b.lengths) == [25, 47, 12]
    assert b.tables.tolist() == [[3, 7, -1, -1], [0, 5, 9, -1], [4, -1, -1, -1]]
    assert b.num_blocks == 64 and b.k_pool.shape == (64, 4, 16, 64)
    assert b.v_pool.shape == (64, 4, 16, 64) and b.q.dtype == torch.float32


def test_determinism():
    a = W.small_batch([10, 20], 4, 2, 16, 16, torch.bfloat16, seed=5)
    b = W.small_batch([10, 20], 4, 2, 16, 16, torch.bfloat16, seed=5)
    assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
    assert np.array_equal(a.tables, b.tables)


def test_config3_lengths_and_shared_logical_data():
    L = W.config3_lengths()
    assert L.shape == (256,) and L.min() >= 16 and L.max() <= 4096
    assert 300 < np.median(L) < 800
    a = W.config3(16, batch=8)
    b = W.config3(32, batch=8)
    assert np.array_equal(a.lengths, b.lengths) and torch.equal(a.q, b.q)
    assert all(torch.equal(x, y) for x, y in zip(a.k_logical, b.k_logical))
    assert a.tables.shape[1] == 2 * b.tables.shape[1] or a.tables.shape[1] >= b.tables.shape[1]


def test_placement_uses_distinct_blocks():
    b = W.config2(batch=8)
    used = b.tables[b.tables >= 0]
    assert len(set(used.tolist())) == used.size
    need = sum(-(-int(x) // 16) for x in b.lengths)
    assert b.num_blocks == int(np.ceil(1.25 * need))


def test_config4_structure():
    a = W.config4a(num_seqs=6, prefix_len=800)
    assert (a.lengths > 800).all() and (a.lengths <= 1312).all()
    assert (a.tables[:, :50] == a.tables[0, :50]).all()
    priv = a.tables[:, 50:]
    priv = priv[priv >= 0]
    assert len(set(priv.tolist())) == priv.size and not set(priv.tolist()) & set(a.tables[0, :50].tolist())
    b = W.config4b(num_pairs=3)
    assert list(b.lengths) == [24] * 6
    for i in range(3):
        assert b.tables[2 * i].tolist() == b.tables[2 * i + 1].tolist()
    assert len(W.config4b_free_blocks(b)) == b.num_blocks - 6


def test_config5_room_to_grow():
    b = W.config5(batch=2, steps=8)
    assert (b.lengths >= 16384).all() and (b.lengths <= 32768).all()
    assert b.tables.shape[1] * 16 >= int(b.lengths.max()) + 8
