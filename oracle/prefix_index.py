"""Reference model of a prefix index over refcounted KV blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "KV Cache Optimization and Management", section "RadixAttention: caching, not just
packing, the prefix" -- cached token sequences are organised so that sequences sharing a prefix
share it; a new request is matched against them and every matched token's K/V is reused, only
the tokens past the divergence need a fresh prefill; when memory runs low the least recently
used leaves go first, and a branch that a running request still references is never evicted
(reference counting, as in "PagedAttention: Virtual Memory for the KV Cache", section
"Sharing a prefix and copying a partial block").

This model is written as a plain map, not a tree: a cached entry is a whole-block prefix
(the tuple of its first k * B tokens, k >= 1) and maps to the physical block holding tokens
[(k - 1) B, k B). Readings (the pages leave the granularity open):
  * sharing is by whole blocks (a partially filled block is not shared), so a match is the
    longest cached prefix of whole blocks;
  * the index holds one pool reference per cached block; ``match`` takes one more per matched
    block for the caller (released by the caller like any table entry);
  * a cached prefix is never replaced: inserting a prefix that is already cached keeps the
    cached block (the caller's own block stays the caller's);
  * "recently used" is a logical clock that advances once per match or insert; every entry on
    the matched or inserted path gets the new time;
  * eviction removes one block at a time: among entries that nothing cached extends (leaves)
    and that only the index references (pool count 1), the one with the oldest time (ties: the
    lower block id), until enough blocks are freed or none qualifies.
"""
from __future__ import annotations


class PrefixCache:
    def __init__(self, pool, block_size: int):
        self.pool = pool
        self.B = int(block_size)
        self.entries: dict = {}     # tuple(tokens[:k B]) -> physical block
        self.stamp: dict = {}       # tuple(tokens[:k B]) -> last use
        self.clock = 0

    def _keys(self, tokens):
        toks = tuple(int(t) for t in tokens)
        return [toks[:j * self.B] for j in range(1, len(toks) // self.B + 1)]

    def match(self, tokens) -> list:
        """Blocks of the longest cached whole-block prefix of ``tokens`` (one new reference
        each, for the caller)."""
        self.clock += 1
        out = []
        for key in self._keys(tokens):
            if key not in self.entries:
                break
            out.append(self.entries[key])
            self.stamp[key] = self.clock
        for b in out:
            self.pool.incref(b)
        return out

    def insert(self, tokens, blocks) -> int:
        """Cache the whole blocks of a computed sequence; ``blocks[j]`` holds its tokens
        [j B, (j + 1) B). Returns how many blocks became cached."""
        self.clock += 1
        added = 0
        for j, key in enumerate(self._keys(tokens)):
            if key not in self.entries:
                self.entries[key] = int(blocks[j])
                self.pool.incref(int(blocks[j]))
                added += 1
            self.stamp[key] = self.clock
        return added

    def _is_leaf(self, key) -> bool:
        n = len(key) + self.B
        return not any(len(k) == n and k[:len(key)] == key for k in self.entries)

    def evict(self, want: int) -> list:
        """Free up to ``want`` blocks, least recently used leaves first; returns their ids in
        eviction order."""
        freed = []
        while len(freed) < want:
            cand = [k for k in self.entries
                    if self._is_leaf(k) and self.pool.refcount(self.entries[k]) == 1]
            if not cand:
                break
            k = min(cand, key=lambda k: (self.stamp[k], self.entries[k]))
            b = self.entries.pop(k)
            del self.stamp[k]
            self.pool.decref(b)
            freed.append(b)
        return freed

    def size(self) -> int:
        return len(self.entries)
