"""Pins of the prefix-index model (oracle/prefix_index.py): the shareable whole blocks of the
380-token system prompt of "KV Cache Optimization and Management" (Worked Example 2 and
answer A3: 23 blocks of 16, 5 blocks of 64), brute-force longest common whole-block prefixes
against the inserted sequences themselves, least-recently-used order, leaf-first eviction and
the protection of blocks a running request still references."""
import numpy as np
import pytest

from oracle import BlockPool
from oracle.prefix_index import PrefixCache
from tests.conftest import load_golden


def _alloc(pool, n):
    return [pool.alloc() for _ in range(n)]


@pytest.mark.parametrize("B,key", [(16, "b16"), (64, "b64")])
def test_shared_system_prompt(B, key):
    g = load_golden("p3_capacity_examples.json")["a3"]
    rng = np.random.default_rng(1)
    prompt = rng.integers(0, 50000, g["shared_prompt_tokens"]).tolist()
    q1 = rng.integers(0, 50000, 90).tolist()
    q2 = rng.integers(0, 50000, 90).tolist()
    pool = BlockPool(256)
    idx = PrefixCache(pool, B)
    r1 = prompt + q1
    blocks1 = _alloc(pool, -(-len(r1) // B))
    assert idx.insert(r1, blocks1) == len(r1) // B
    got = idx.match(prompt + q2)
    assert len(got) == g[f"shareable_blocks_{key}"]
    assert len(got) * B == g[f"shareable_tokens_{key}"]
    assert got == blocks1[:len(got)]
    # the matched blocks carry the caller's reference besides the first request's and the
    # index's
    assert all(pool.refcount(b) == 3 for b in got)


def _lcp_blocks(a, b, B):
    n = 0
    while (n + 1) * B <= min(len(a), len(b)) and a[n * B:(n + 1) * B] == b[n * B:(n + 1) * B]:
        n += 1
    return n


def test_match_is_longest_common_whole_block_prefix():
    """Sequences over a 3-symbol vocabulary share prefixes often; the match of each query is
    the longest whole-block common prefix with any inserted sequence, and the blocks are those
    of the first sequence that brought each prefix in."""
    B = 4
    rng = np.random.default_rng(2)
    pool = BlockPool(4096)
    idx = PrefixCache(pool, B)
    inserted = []
    for _ in range(60):
        seq = rng.integers(0, 3, rng.integers(1, 30)).tolist()
        blocks = _alloc(pool, -(-len(seq) // B))
        idx.insert(seq, blocks)
        inserted.append((seq, blocks))
    for _ in range(200):
        qry = rng.integers(0, 3, rng.integers(0, 30)).tolist()
        want = max([_lcp_blocks(qry, s, B) for s, _ in inserted] + [0])
        got = idx.match(qry)
        assert len(got) == want
        for j, b in enumerate(got):
            first = next(bl for s, bl in inserted if _lcp_blocks(qry, s, B) > j)
            assert b == first[j]


def test_lru_order_and_leaf_first():
    B = 2
    pool = BlockPool(64)
    idx = PrefixCache(pool, B)
    a, b, c = [1, 1, 5, 5], [2, 2, 6, 6], [3, 3, 7, 7]
    blocks = {}
    for name, seq in (("a", a), ("b", b), ("c", c)):
        blocks[name] = _alloc(pool, 2)
        idx.insert(seq, blocks[name])
        for blk in blocks[name]:           # the requests finish: only the index holds them
            pool.decref(blk)
    for blk in idx.match(a):               # a is used again, then released
        pool.decref(blk)
    # oldest first: b's leaf, then b's first block (now a leaf), then c's
    assert idx.evict(3) == [blocks["b"][1], blocks["b"][0], blocks["c"][1]]
    assert idx.size() == 3
    assert pool.refcount(blocks["b"][0]) == 0


def test_referenced_blocks_are_not_evicted():
    B = 2
    pool = BlockPool(64)
    idx = PrefixCache(pool, B)
    seq = [9, 9, 8, 8, 7, 7]
    mine = _alloc(pool, 3)
    idx.insert(seq, mine)                  # the request still runs: its blocks have count 2
    assert idx.evict(10) == []
    for blk in mine:
        pool.decref(blk)
    held = idx.match([9, 9, 8, 8, 1, 1])   # another request takes the first two blocks
    assert held == mine[:2]
    assert idx.evict(10) == [mine[2]]      # only the unreferenced leaf goes
    for blk in held:
        pool.decref(blk)
    assert idx.evict(10) == [mine[1], mine[0]]
    assert idx.size() == 0 and pool.num_free() == 64


def test_duplicate_prefix_keeps_the_cached_block():
    B = 2
    pool = BlockPool(16)
    idx = PrefixCache(pool, B)
    first = _alloc(pool, 2)
    second = _alloc(pool, 3)
    assert idx.insert([1, 2, 3, 4], first) == 2
    assert idx.insert([1, 2, 3, 4, 5, 6], second) == 1      # only the third block is new
    assert idx.match([1, 2, 3, 4, 5, 6]) == [first[0], first[1], second[2]]
    assert pool.refcount(second[0]) == 1                   # still only the caller's
