"""Pins of the bookkeeping oracle to the values the pages print (tests/golden/*.json)."""
import numpy as np
import pytest

from oracle import (BlockPool, PagedKVModel, PoolExhausted, RefcountError, blocks_for,
                    capacity_report, reserved_slots, shareable_prefix_blocks, token_address)
from tests.conftest import load_golden


def test_allocation_example():
    g = load_golden("p1_allocation_example.json")
    B = g["block_size"]
    assert sum(g["lengths"]) == g["total_tokens"]
    assert [blocks_for(n, B) for n in g["lengths"]] == g["blocks"]
    slots = sum(reserved_slots(n, B) for n in g["lengths"])
    assert slots == g["paged_slots"]
    assert slots - g["total_tokens"] == g["padding_slots"]
    naive = g["reservation_per_request"] * len(g["lengths"])
    assert naive == g["naive_slots"]
    num, den = g["paged_over_naive"]
    assert slots * den == naive * num
    # waste per request is below one block
    assert all(reserved_slots(n, B) - n < B for n in g["lengths"])


def test_address_example():
    g = load_golden("p1_address_example.json")
    blk, off = token_address(g["position"], g["table"], g["block_size"])
    assert (blk, off) == (g["physical_block"], g["offset"])
    assert divmod(g["position"], g["block_size"])[0] == g["logical_block"]


def test_growth_example():
    g = load_golden("p1_growth_example.json")
    B = g["block_size"]
    pool = BlockPool(g["pool_blocks"])
    for t in g["tables"]:
        for b in t:
            pool.claim(b)
    assert pool.num_free() == g["free_after_allocation"]
    assert g["pool_blocks"] * B == g["pool_slots"]
    assert g["pool_slots"] < 6144          # the per-request reservation would not fit
    k = np.zeros((g["pool_blocks"], 1, B, 2), np.float32)
    v = np.zeros((g["pool_blocks"], 1, B, 2), np.float32)
    model = PagedKVModel(pool, k, v, B)
    for s, (t, L) in enumerate(zip(g["tables"], g["lengths"])):
        model.add_sequence(s, t, L)
    s = g["grow_request"]
    before = {b: list(model.tables[b]) for b in model.tables}
    for i in range(g["grow_by"]):
        # the page's engine takes physical block 11 for the new logical block
        model.append(s, np.full((1, 2), i), np.full((1, 2), -i), claim=g["new_block"])
    assert model.lengths[s] == g["grown_length"]
    assert blocks_for(model.lengths[s], B) == g["grown_blocks"]
    assert model.tables[s] == g["grown_table"]
    # existing entries stay where they are; other requests untouched
    assert model.tables[s][:3] == before[s]
    for o in (0, 2):
        assert model.tables[o] == before[o]
    assert blocks_for(g["lengths"][s] + g["alt_grow_by"], B) == g["alt_grown_blocks"]
    # the first appended token went to the last slot of block 9, the rest into block 11
    assert k[9, 0, 15, 0] == 0 and v[9, 0, 15, 0] == 0
    assert k[11, 0, 0, 0] == 1 and k[11, 0, 8, 0] == 9 and v[11, 0, 8, 0] == -9
    assert pool.num_free() == g["free_after_allocation"] - 1


def test_full_prefix_needs_no_copy():
    g = load_golden("p1_sharing_example.json")
    B = g["block_size"]
    n = g["full_prefix_tokens"]
    assert shareable_prefix_blocks(n, B) == g["full_prefix_blocks"] == blocks_for(n, B)
    pool = BlockPool(64)
    k = np.zeros((64, 1, B, 1), np.float32)
    v = np.zeros((64, 1, B, 1), np.float32)
    model = PagedKVModel(pool, k, v, B)
    table = [pool.alloc() for _ in range(g["full_prefix_blocks"])]
    model.add_sequence("a", table, n)
    model.fork("a", "b")
    blk, off = model.append("b", np.ones((1, 1)), np.ones((1, 1)))
    assert off == 0 and blk not in table
    assert model.copies == []
    assert model.tables["a"] == table and model.tables["b"][:-1] == table


def test_copy_on_write_example():
    g = load_golden("p1_sharing_example.json")["cow"]
    B = 16
    H, d = 2, 3
    pool = BlockPool(8)
    rng = np.random.default_rng(0)
    k = rng.standard_normal((8, H, B, d)).astype(np.float32)
    v = rng.standard_normal((8, H, B, d)).astype(np.float32)
    k0, v0 = k.copy(), v.copy()
    model = PagedKVModel(pool, k, v, B)
    names = {"P0": pool.alloc(), "P1": pool.alloc()}
    assert names == {"P0": 0, "P1": 1}
    model.add_sequence("A", [names["P0"], names["P1"]], sum(g["tokens_in_shared_blocks"]))
    model.fork("A", "B")
    for nm, r in g["refcounts_before"].items():
        assert pool.refcount(names[nm]) == r
    kr, vr = np.full((H, d), 7.0), np.full((H, d), -7.0)
    blk, off = model.append(g["writer"], kr, vr)
    names["P2"] = blk
    assert blk == 2 and off == g["writer_new_entry_offset"]
    assert model.copies == [(names["P1"], names["P2"], g["entries_copied"])]
    assert model.tables["B"] == [names[x] for x in g["writer_table_after"]]
    assert model.tables["A"] == [names[x] for x in g["other_table_after"]]
    for nm, r in g["refcounts_after"].items():
        assert pool.refcount(names[nm]) == r
    n = g["entries_copied"]
    # copied entries equal the originals bit for bit; A's block is untouched
    assert np.array_equal(k[2, :, :n], k0[1, :, :n]) and np.array_equal(v[2, :, :n], v0[1, :, :n])
    assert np.array_equal(k[1], k0[1]) and np.array_equal(v[1], v0[1])
    assert np.array_equal(k[2, :, n], kr) and np.array_equal(v[2, :, n], vr)
    # slots past the new entry of the copy keep what the fresh block held
    assert np.array_equal(k[2, :, n + 1:], k0[2, :, n + 1:])
    # A then appends in place: P1 now has one reference, so no copy
    model.append("A", kr, vr)
    assert len(model.copies) == 1 and model.tables["A"] == [0, 1]


def test_capacity_examples():
    g = load_golden("p3_capacity_examples.json")
    for key in ("worked_example_1", "a2"):
        e = g[key]
        r = capacity_report(e["lengths"], e["block_size"], e["max_len"])
        assert [blocks_for(x, e["block_size"]) for x in e["lengths"]] == e["blocks_each"]
        assert r["blocks"] == e["blocks"]
        assert r["actual_tokens"] == e["actual_tokens"]
        assert r["paged_slots"] == e["paged_slots"] and r["naive_slots"] == e["naive_slots"]
        assert round(r["paged_waste_pct"], 2) == e["paged_waste_pct"]
        assert round(r["naive_waste_pct"], 2) == e["naive_waste_pct"]
        assert round(r["reduction"], 2) == e["reduction"]
    a3 = g["a3"]
    r = capacity_report(a3["lengths"], a3["block_size"], a3["max_len"])
    assert [blocks_for(x, 64) for x in a3["lengths"]] == a3["blocks_each"]
    assert r["blocks"] == a3["blocks"] == a3["table_entries_b64"]
    assert r["paged_slots"] == a3["paged_slots"]
    assert round(r["paged_waste_pct"], 2) == a3["paged_waste_pct"]
    assert capacity_report(a3["lengths"], 16, 512)["blocks"] == a3["table_entries_b16"]
    assert shareable_prefix_blocks(a3["shared_prompt_tokens"], 16) == a3["shareable_blocks_b16"]
    assert shareable_prefix_blocks(a3["shared_prompt_tokens"], 16) * 16 == a3["shareable_tokens_b16"]
    assert shareable_prefix_blocks(a3["shared_prompt_tokens"], 64) == a3["shareable_blocks_b64"]
    assert shareable_prefix_blocks(a3["shared_prompt_tokens"], 64) * 64 == a3["shareable_tokens_b64"]
    a5 = g["a5"]
    pb = blocks_for(a5["prefix_tokens"], a5["block_size"])
    sb = blocks_for(a5["suffix_tokens"], a5["block_size"])
    assert (pb, sb) == (a5["prefix_blocks"], a5["suffix_blocks"])
    assert (pb + sb) * a5["requests"] == a5["blocks_unshared"]
    assert pb + sb * a5["requests"] == a5["blocks_shared"]
    assert round(a5["blocks_unshared"] / a5["blocks_shared"], 2) == a5["reduction"]


def test_release_only_at_zero():
    a6 = load_golden("p3_capacity_examples.json")["a6"]
    pool = BlockPool(4)
    k = np.zeros((4, 1, 16, 1)); v = np.zeros((4, 1, 16, 1))
    model = PagedKVModel(pool, k, v, 16)
    p0 = pool.alloc()
    model.add_sequence("A", [p0], 16)
    model.fork("A", "B")
    assert pool.refcount(p0) == a6["refcount_before"]
    freed = model.release("A")
    assert pool.refcount(p0) == a6["refcount_after_one_release"]
    assert (p0 in freed) == a6["returned_to_free_pool"]
    assert pool.num_free() == 3
    assert model.release("B") == [p0] and pool.num_free() == 4


def test_pool_errors():
    pool = BlockPool(2)
    pool.alloc(); pool.alloc()
    with pytest.raises(PoolExhausted):
        pool.alloc()
    p = BlockPool(1)
    with pytest.raises(RefcountError):
        p.decref(0)
    b = p.alloc()
    with pytest.raises(RefcountError):
        p.claim(b)
    assert p.decref(b) is True
    with pytest.raises(RefcountError):
        p.incref(b)
