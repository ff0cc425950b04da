"""Float-free bookkeeping model of a paged KV cache: block counts, a refcounted block pool,
per-sequence block tables, appends that grow the table, prefix sharing and copy-on-write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * "PagedAttention: Virtual Memory for the KV Cache": ceil(T/B) blocks per request and the
    25/47/12-token example (section "Where contiguous allocation wastes space"); tables,
    free count and growth by one block ("Growing a request"); shared full blocks and the
    copy of a partially filled shared block ("Sharing a prefix and copying a partial block").
  * "Paged Attention and vLLM", section "Continuous Batching and Scheduler": a write into a
    shared block allocates a fresh block, copies, and redirects the writer's table entry.
  * "KV Cache Optimization and Management": blocks are allocated one at a time as a sequence
    grows; a reference count tracks sharers and a block returns to the free pool only at zero
    (section "PagedAttention: borrowing virtual memory", answer A6); capacity examples.
  * "Paged Attention and vLLM", section "Continuous Batching and Scheduler": a preempted
    sequence's physical blocks are evicted to CPU memory a block at a time and swapped back
    when it resumes, so the cost is the evicted blocks only.

Readings: the pages name no allocation order (the example takes block 11 while lower ones are
free), so ``BlockPool.alloc`` hands out the lowest free block and ``claim`` takes a named one.
A copy-on-write copies the valid slots [0, n) of every KV head of K and V, where n is the
writer's offset inside the shared block.

Swap (the pages give the mechanism, not its bookkeeping): host memory holds a second pool of
blocks with the device pools' block shape, managed by its own ``BlockPool``. Swapping out a
group of sequences gives each distinct device block they reference one host block, copies it
whole (every head, every slot, K and V), moves the group's references from the device block to
the host block and rewrites the group's tables with host ids. A device block that a sequence
outside the group also references stays resident for it. Swapping in is the mirror image, with
fresh device blocks. A whole block moves even when only some of its slots are valid.
"""
from __future__ import annotations

import numpy as np


class PoolExhausted(RuntimeError):
    """No free block: the pages leave the recovery policy to the scheduler."""


class RefcountError(RuntimeError):
    """A reference count would go below zero, or a free block was referenced."""


def blocks_for(tokens: int, block_size: int) -> int:
    """Blocks needed to hold ``tokens`` tokens: the smallest n with n*B >= tokens."""
    n = tokens // block_size
    if n * block_size < tokens:
        n += 1
    return n


def reserved_slots(tokens: int, block_size: int) -> int:
    """Token slots a request of ``tokens`` tokens holds under paging (whole blocks)."""
    return blocks_for(tokens, block_size) * block_size


def shareable_prefix_blocks(prefix_tokens: int, block_size: int) -> int:
    """Blocks of a shared prefix that are complete and so can be shared without a copy."""
    return prefix_tokens // block_size


def capacity_report(lengths, block_size: int, max_len: int) -> dict:
    """Slots reserved by paging vs by a per-request ``max_len`` reservation, the wasted share
    of each (in percent) and the ratio of reserved slots."""
    actual = sum(int(x) for x in lengths)
    blocks = sum(blocks_for(int(x), block_size) for x in lengths)
    paged = blocks * block_size
    naive = max_len * len(lengths)
    return {
        "blocks": blocks,
        "actual_tokens": actual,
        "paged_slots": paged,
        "naive_slots": naive,
        "paged_waste_pct": 100.0 * (paged - actual) / paged,
        "naive_waste_pct": 100.0 * (naive - actual) / naive,
        "reduction": naive / paged,
    }


class BlockPool:
    """Fixed pool of ``num_blocks`` physical block ids with reference counts."""

    def __init__(self, num_blocks: int):
        self.num_blocks = int(num_blocks)
        self.ref = [0] * self.num_blocks

    def num_free(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def alloc(self) -> int:
        for b, r in enumerate(self.ref):
            if r == 0:
                self.ref[b] = 1
                return b
        raise PoolExhausted("no free block")

    def claim(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise IndexError(block)
        if self.ref[block] != 0:
            raise RefcountError(f"block {block} is in use")
        self.ref[block] = 1
        return block

    def incref(self, block: int) -> None:
        if self.ref[block] == 0:
            raise RefcountError(f"block {block} is free")
        self.ref[block] += 1

    def decref(self, block: int) -> bool:
        """Drop one reference; returns True when the block went back to the free pool."""
        if self.ref[block] == 0:
            raise RefcountError(f"block {block} is already free")
        self.ref[block] -= 1
        return self.ref[block] == 0

    def refcount(self, block: int) -> int:
        return self.ref[block]


def copy_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                src_ids, dst_ids) -> int:
    """Batched whole-block copy between two pools of one block shape ``[H_kv][B][d]``:
    block ``src_ids[i]`` of (src_k, src_v) goes to block ``dst_ids[i]`` of (dst_k, dst_v).
    A pair whose id falls outside its pool is skipped. Returns the number of pairs copied."""
    done = 0
    for s, d in zip(src_ids, dst_ids):
        s, d = int(s), int(d)
        if not (0 <= s < src_k.shape[0] and 0 <= d < dst_k.shape[0]):
            continue
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
        done += 1
    return done


class PagedKVModel:
    """Pools of raw K/V values plus per-sequence tables and lengths.

    ``k_pool`` and ``v_pool`` are ``[N][H_kv][B][d]`` (numpy arrays of any
    dtype; values are only copied, never combined).
    """

    def __init__(self, pool: BlockPool, k_pool: np.ndarray, v_pool: np.ndarray,
                 block_size: int):
        self.pool = pool
        self.k = k_pool
        self.v = v_pool
        self.B = int(block_size)
        self.tables: dict = {}
        self.lengths: dict = {}
        self.copies: list = []        # (src, dst, n) copy-on-write records, in order
        self.swapped: set = set()     # sequences whose tables hold host block ids

    # -- sequence lifetime --------------------------------------------------------------
    def add_sequence(self, s, table, length: int) -> None:
        """Register a sequence whose blocks are already referenced in ``pool``."""
        self.tables[s] = [int(b) for b in table]
        self.lengths[s] = int(length)

    def fork(self, parent, child) -> None:
        """``child`` shares every block of ``parent`` (one more reference each)."""
        for b in self.tables[parent]:
            self.pool.incref(b)
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]

    def release(self, s) -> list:
        """Drop the sequence; returns the blocks that went back to the free pool."""
        freed = [b for b in self.tables[s] if self.pool.decref(b)]
        del self.tables[s]
        del self.lengths[s]
        return freed

    # -- preemption ---------------------------------------------------------------------
    def swap_out(self, group, host: BlockPool, host_k: np.ndarray, host_v: np.ndarray) -> list:
        """Evict the blocks of the sequences in ``group`` to the host pool.

        Each distinct device block gets one host block (the lowest free); the block is copied
        whole, the group's references move to the host block and the device block loses them
        (it returns to the free pool at zero). Returns the (device block, host block) pairs
        in the order of first reference.
        """
        mapping: dict = {}
        for s in group:
            if s in self.swapped:
                raise ValueError(f"sequence {s} is already swapped out")
            for b in self.tables[s]:
                if b in mapping:
                    host.incref(mapping[b])
                else:
                    mapping[b] = host.alloc()
        pairs = list(mapping.items())
        copy_blocks(host_k, host_v, self.k, self.v, [p[0] for p in pairs], [p[1] for p in pairs])
        for s in group:
            t = self.tables[s]
            for j, b in enumerate(t):
                self.pool.decref(b)
                t[j] = mapping[b]
            self.swapped.add(s)
        return pairs

    def swap_in(self, group, host: BlockPool, host_k: np.ndarray, host_v: np.ndarray,
                claims=None) -> list:
        """Bring a swapped-out group back: each distinct host block gets a device block
        (``claims`` names them in order of first reference, else the lowest free), is copied
        whole, and the group's references move back. Returns the (host block, device block)
        pairs."""
        mapping: dict = {}
        claims = iter(claims) if claims is not None else None
        for s in group:
            if s not in self.swapped:
                raise ValueError(f"sequence {s} is not swapped out")
            for b in self.tables[s]:
                if b in mapping:
                    self.pool.incref(mapping[b])
                else:
                    mapping[b] = self.pool.claim(next(claims)) if claims else self.pool.alloc()
        pairs = list(mapping.items())
        copy_blocks(self.k, self.v, host_k, host_v, [p[0] for p in pairs], [p[1] for p in pairs])
        for s in group:
            t = self.tables[s]
            for j, b in enumerate(t):
                host.decref(b)
                t[j] = mapping[b]
            self.swapped.discard(s)
        return pairs

    # -- writes -------------------------------------------------------------------------
    def prepare_write(self, s, claim=None):
        """Make the slot of token ``lengths[s]`` writable by ``s`` alone.

        A new logical block gets a fresh physical block (``claim`` names one, else the lowest
        free). A shared partially filled block is first copied to a fresh block: slots
        [0, offset) of every head, K and V; the table entry is redirected and the old block
        loses one reference. Returns (physical block, offset).
        """
        pos = self.lengths[s]
        j, r = divmod(pos, self.B)
        table = self.tables[s]
        if j == len(table):
            blk = self.pool.claim(claim) if claim is not None else self.pool.alloc()
            table.append(blk)
        elif j > len(table):
            raise IndexError("table has a gap")
        else:
            old = table[j]
            if self.pool.refcount(old) > 1:
                new = self.pool.claim(claim) if claim is not None else self.pool.alloc()
                self.k[new, :, :r, :] = self.k[old, :, :r, :]
                self.v[new, :, :r, :] = self.v[old, :, :r, :]
                table[j] = new
                self.pool.decref(old)
                self.copies.append((old, new, r))
        return table[j], r

    def append(self, s, k_row, v_row, claim=None):
        """Store one token's K and V rows (``[H_kv][d]`` each) after the last stored token."""
        blk, r = self.prepare_write(s, claim)
        self.k[blk, :, r, :] = k_row
        self.v[blk, :, r, :] = v_row
        self.lengths[s] += 1
        return blk, r

    def table_array(self, order, width: int) -> np.ndarray:
        out = np.full((len(order), width), -1, dtype=np.int32)
        for i, s in enumerate(order):
            t = self.tables[s]
            out[i, :len(t)] = t
        return out
