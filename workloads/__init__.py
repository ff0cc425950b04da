"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out in the cache layout that the
library's entry points take. It holds none of the attention arithmetic, so the CPU oracle
(``oracle/``) and the HIP path can both take their inputs from here without sharing any
of the method.

Cache layout (one layer; K and V in separate pools):
  * ``k_pool``  ``[num_blocks][H_kv][B][d]``  -- a block holds B key rows per KV head;
  * ``v_pool``  ``[num_blocks][H_kv][B][d]``  -- and B value rows, in the same order.
The pages leave the in-block layout to the kernel ("PagedAttention: Virtual Memory for the KV
Cache", section "Block size is a kernel choice too").

Random streams: every draw comes from ``numpy.random.default_rng([seed, stream])`` with a
fixed stream id per kind of draw (lengths, placement, queries, keys/values, appended tokens),
so the same logical data can be re-placed (other block size, other permutation) unchanged.
Values are N(0, 1) drawn in float32 and rounded to the storage dtype by ``torch.Tensor.to``
(round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

SEED_BASE = 127000

# stream ids for numpy.random.default_rng([seed, stream])
_LEN, _PLACE, _Q, _KV, _NEW, _SUFFIX, _EXTQ = 0, 1, 2, 3, 4, 5, 6

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def rng_for(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) in float32, rounded to ``dtype`` (RNE)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class Batch:
    """One decode batch: queries, a paged cache and the per-sequence block tables."""

    dtype: torch.dtype
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: np.ndarray            # int32 [S]  stored tokens per sequence
    tables: np.ndarray             # int32 [S][max_blocks]; -1 marks an unused entry
    num_blocks: int                # physical blocks in the pool
    q: torch.Tensor                # [S][H_q][d]
    k_pool: torch.Tensor           # [N][H_kv][B][d]
    v_pool: torch.Tensor           # [N][H_kv][B][d]
    k_logical: list                # per sequence [H_kv][L_s][d], in token order
    v_logical: list                # per sequence [H_kv][L_s][d]
    seed: int = 0
    note: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.tables.shape[1])

    @property
    def kv_bytes(self) -> int:
        """Bytes of valid K and V rows one decode pass must read (each KV head once)."""
        es = torch.tensor([], dtype=self.dtype).element_size()
        return int(2 * int(self.lengths.sum()) * self.num_kv_heads * self.head_dim * es)


def empty_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                dtype: torch.dtype, poison: bool = False):
    fill = float("nan") if poison else 0.0
    k_pool = torch.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=dtype)
    v_pool = torch.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=dtype)
    return k_pool, v_pool


def write_rows(k_pool, v_pool, table_row, k_seq, v_seq, start: int = 0):
    """Store logical rows ``[start, start + n)`` of one sequence into the pools.

    ``k_seq`` / ``v_seq`` are ``[H_kv][n][d]``; ``table_row`` lists the physical block of each
    logical block. Copies whole block-sized slices (a layout step, not a per-token gather).
    """
    bsz = k_pool.shape[2]
    n = k_seq.shape[1]
    pos = start
    end = start + n
    while pos < end:
        j = pos // bsz
        lo = pos - j * bsz
        hi = min(bsz, end - j * bsz)
        blk = int(table_row[j])
        a, b = pos - start, pos - start + (hi - lo)
        k_pool[blk, :, lo:hi, :] = k_seq[:, a:b, :]
        v_pool[blk, :, lo:hi, :] = v_seq[:, a:b, :]
        pos += hi - lo


def place_blocks(lengths: Sequence[int], block_size: int, rng: np.random.Generator,
                 pool_factor: float = 1.25, max_blocks: Optional[int] = None,
                 num_blocks: Optional[int] = None):
    """Random physical placement: sequence s takes the next ceil(L_s/B) entries of a seeded
    permutation of a pool sized ``pool_factor`` times the total need."""
    nbs = [_ceil_div(int(L), block_size) for L in lengths]
    need = sum(nbs)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    if max_blocks is None:
        max_blocks = max(1, max(nbs) if nbs else 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(lengths), max_blocks), -1, dtype=np.int32)
    cur = 0
    for s, nb in enumerate(nbs):
        tables[s, :nb] = perm[cur:cur + nb]
        cur += nb
    return tables, num_blocks, perm[cur:]


def make_batch(lengths, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
               dtype: torch.dtype, seed: int, tables: Optional[np.ndarray] = None,
               num_blocks: Optional[int] = None, max_blocks: Optional[int] = None,
               pool_factor: float = 1.25, poison: bool = False, note: str = "") -> Batch:
    lengths = np.asarray(lengths, dtype=np.int32)
    S = int(lengths.shape[0])
    if tables is None:
        tables, num_blocks, _ = place_blocks(lengths, block_size, rng_for(seed, _PLACE),
                                             pool_factor, max_blocks, num_blocks)
    else:
        tables = np.asarray(tables, dtype=np.int32)
        assert num_blocks is not None
    q = normal(rng_for(seed, _Q), (S, num_q_heads, head_dim), dtype)
    rkv = rng_for(seed, _KV)
    k_log, v_log = [], []
    for s in range(S):
        L = int(lengths[s])
        k_log.append(normal(rkv, (num_kv_heads, L, head_dim), dtype))
        v_log.append(normal(rkv, (num_kv_heads, L, head_dim), dtype))
    k_pool, v_pool = empty_pools(num_blocks, num_kv_heads, block_size, head_dim, dtype, poison)
    for s in range(S):
        write_rows(k_pool, v_pool, tables[s], k_log[s], v_log[s])
    return Batch(dtype, block_size, num_q_heads, num_kv_heads, head_dim, lengths, tables,
                 int(num_blocks), q, k_pool, v_pool, k_log, v_log, seed, note)


def new_queries(batch: Batch, step: int) -> torch.Tensor:
    """Fresh queries for decode step ``step`` (step 0 is ``batch.q``)."""
    if step == 0:
        return batch.q
    rng = rng_for(batch.seed + 1000 * step, _Q)
    return normal(rng, tuple(batch.q.shape), batch.dtype)


def new_tokens(seed: int, step: int, n: int, num_kv_heads: int, head_dim: int, dtype):
    """K and V rows ``[n][H_kv][d]`` of tokens appended at decode step ``step``."""
    rng = rng_for(seed + 1000 * step, _NEW)
    return (normal(rng, (n, num_kv_heads, head_dim), dtype),
            normal(rng, (n, num_kv_heads, head_dim), dtype))


# ----------------------------------------------------------------------------------------
# The five workloads. Shapes follow the pages' examples: the 25/47/12-token requests with
# tables [3,7], [0,5,9], [4] in a 64-block pool; a 7B-like MHA batch; a GQA batch with
# log-normal lengths; an 800-token shared prefix and a 24-token prefix that needs a
# copy-on-write; long contexts split into 512-token partitions.
# ----------------------------------------------------------------------------------------

def config1(poison: bool = False) -> Batch:
    """3 requests of 25, 47 and 12 tokens, B=16, tables [3,7], [0,5,9], [4] in a 64-block pool,
    4/4 heads, d=64, fp32. The table row has room for a fourth block (the growth step)."""
    tables = np.full((3, 4), -1, dtype=np.int32)
    tables[0, :2] = [3, 7]
    tables[1, :3] = [0, 5, 9]
    tables[2, :1] = [4]
    return make_batch([25, 47, 12], 4, 4, 64, 16, torch.float32, SEED_BASE + 1,
                      tables=tables, num_blocks=64, poison=poison, note="config1")


def config2_lengths(seed: int = SEED_BASE + 2, batch: int = 64):
    return rng_for(seed, _LEN).integers(128, 2048, size=batch, endpoint=True).astype(np.int32)


def config2(batch: int = 64, poison: bool = False) -> Batch:
    """MHA decode, 32/32 heads, d=128, fp16, B=16, L ~ U{128..2048}, 1.25x pool."""
    seed = SEED_BASE + 2
    return make_batch(config2_lengths(seed, batch), 32, 32, 128, 16, torch.float16, seed,
                      poison=poison, note="config2")


def config3_lengths(seed: int = SEED_BASE + 3, batch: int = 256):
    """log-normal, median 512 (mu = ln 512), sigma 1.0, rounded, clipped to [16, 4096]."""
    x = rng_for(seed, _LEN).lognormal(mean=math.log(512.0), sigma=1.0, size=batch)
    return np.clip(np.rint(x), 16, 4096).astype(np.int32)


def config3(block_size: int = 16, batch: int = 256, poison: bool = False,
            lengths=None) -> Batch:
    """GQA decode, 64 query / 8 KV heads, d=128, bf16, log-normal lengths; B = 16 or 32 share
    lengths, queries and logical K/V, each with its own pool and placement."""
    seed = SEED_BASE + 3
    if lengths is None:
        lengths = config3_lengths(seed, batch)
    lengths = np.asarray(lengths, dtype=np.int32)
    place_seed = seed + 17 * block_size
    tables, nblk, _ = place_blocks(lengths, block_size, rng_for(place_seed, _PLACE))
    return make_batch(lengths, 64, 8, 128, block_size, torch.bfloat16, seed, tables=tables,
                      num_blocks=nblk, poison=poison, note=f"config3_B{block_size}")


def config4a(num_seqs: int = 128, prefix_len: int = 800, poison: bool = False) -> Batch:
    """``num_seqs`` sequences share one ``prefix_len``-token prefix (its full blocks appear in
    every table) plus private suffixes of U{1..512} tokens; 64/8 heads, d=128, bf16, B=16."""
    seed = SEED_BASE + 4
    B, Hq, Hkv, d, dt = 16, 64, 8, 128, torch.bfloat16
    assert prefix_len % B == 0
    suffix = rng_for(seed, _LEN).integers(1, 512, size=num_seqs, endpoint=True).astype(np.int32)
    lengths = (prefix_len + suffix).astype(np.int32)
    npre = prefix_len // B
    nsuf = [_ceil_div(int(x), B) for x in suffix]
    need = npre + sum(nsuf)
    nblk = math.ceil(1.25 * need)
    perm = rng_for(seed, _PLACE).permutation(nblk).astype(np.int32)
    max_blocks = npre + max(nsuf)
    tables = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
    tables[:, :npre] = perm[:npre]
    cur = npre
    for s in range(num_seqs):
        tables[s, npre:npre + nsuf[s]] = perm[cur:cur + nsuf[s]]
        cur += nsuf[s]
    q = normal(rng_for(seed, _Q), (num_seqs, Hq, d), dt)
    rkv = rng_for(seed, _KV)
    kp = normal(rkv, (Hkv, prefix_len, d), dt)
    vp = normal(rkv, (Hkv, prefix_len, d), dt)
    rs = rng_for(seed, _SUFFIX)
    k_log, v_log = [], []
    k_pool, v_pool = empty_pools(nblk, Hkv, B, d, dt, poison)
    write_rows(k_pool, v_pool, tables[0], kp, vp)
    for s in range(num_seqs):
        ks = normal(rs, (Hkv, int(suffix[s]), d), dt)
        vs = normal(rs, (Hkv, int(suffix[s]), d), dt)
        write_rows(k_pool, v_pool, tables[s], ks, vs, start=prefix_len)
        k_log.append(torch.cat([kp, ks], dim=1))
        v_log.append(torch.cat([vp, vs], dim=1))
    return Batch(dt, B, Hq, Hkv, d, lengths, tables, nblk, q, k_pool, v_pool, k_log, v_log,
                 seed, "config4a")


def shared_prefix_batch(suffix_lens, prefix_len: int, num_q_heads: int, num_kv_heads: int,
                        head_dim: int, block_size: int, dtype: torch.dtype, seed: int,
                        poison: bool = False) -> Batch:
    """Sequences that all begin with one ``prefix_len``-token prefix held in shared whole
    blocks (the first ``prefix_len / B`` entries of every table), followed by private suffixes
    of ``suffix_lens`` tokens (0 allowed); random placement in a 1.25x pool. Same draw order as
    :func:`config4a`: suffix lengths are given, then placement, Q, prefix K/V, suffix K/V."""
    B, Hkv, d = block_size, num_kv_heads, head_dim
    assert prefix_len % B == 0
    suffix = np.asarray(suffix_lens, dtype=np.int32)
    S = len(suffix)
    lengths = (prefix_len + suffix).astype(np.int32)
    npre = prefix_len // B
    nsuf = [_ceil_div(int(x), B) for x in suffix]
    need = npre + sum(nsuf)
    nblk = max(1, math.ceil(1.25 * need))
    perm = rng_for(seed, _PLACE).permutation(nblk).astype(np.int32)
    max_blocks = max(1, npre + max(nsuf, default=0))
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    tables[:, :npre] = perm[:npre]
    cur = npre
    for s in range(S):
        tables[s, npre:npre + nsuf[s]] = perm[cur:cur + nsuf[s]]
        cur += nsuf[s]
    q = normal(rng_for(seed, _Q), (S, num_q_heads, d), dtype)
    rkv = rng_for(seed, _KV)
    kp = normal(rkv, (Hkv, prefix_len, d), dtype)
    vp = normal(rkv, (Hkv, prefix_len, d), dtype)
    rs = rng_for(seed, _SUFFIX)
    k_log, v_log = [], []
    k_pool, v_pool = empty_pools(nblk, Hkv, B, d, dtype, poison)
    if S:
        write_rows(k_pool, v_pool, tables[0], kp, vp)
    for s in range(S):
        ks = normal(rs, (Hkv, int(suffix[s]), d), dtype)
        vs = normal(rs, (Hkv, int(suffix[s]), d), dtype)
        write_rows(k_pool, v_pool, tables[s], ks, vs, start=prefix_len)
        k_log.append(torch.cat([kp, ks], dim=1))
        v_log.append(torch.cat([vp, vs], dim=1))
    return Batch(dtype, B, num_q_heads, Hkv, d, lengths, tables, nblk, q, k_pool, v_pool, k_log,
                 v_log, seed, "shared_prefix")


def extend_queries(batch: Batch, new_tokens, seed: int):
    """Query rows for the last ``new_tokens[s]`` stored tokens of each sequence of ``batch``
    (their keys and values are already in the cache): ``(q [T][H_q][d], query_start [S + 1])``
    with T = sum of new_tokens, drawn N(0, 1) and rounded to the batch's dtype."""
    n = np.asarray(new_tokens, dtype=np.int64)
    start = np.zeros(len(n) + 1, dtype=np.int32)
    start[1:] = np.cumsum(n)
    q = normal(rng_for(seed, _EXTQ), (int(start[-1]), batch.num_q_heads, batch.head_dim),
               batch.dtype)
    return q, start


def config4a_private(shared: Batch) -> Batch:
    """The same logical data as :func:`config4a` with every sequence holding private copies of
    the prefix blocks (no sharing)."""
    lengths = shared.lengths
    B = shared.block_size
    seed = shared.seed
    tables, nblk, _ = place_blocks(lengths, B, rng_for(seed + 99, _PLACE))
    k_pool, v_pool = empty_pools(nblk, shared.num_kv_heads, B, shared.head_dim, shared.dtype)
    for s in range(shared.num_seqs):
        write_rows(k_pool, v_pool, tables[s], shared.k_logical[s], shared.v_logical[s])
    return Batch(shared.dtype, B, shared.num_q_heads, shared.num_kv_heads, shared.head_dim,
                 lengths, tables, nblk, shared.q, k_pool, v_pool, shared.k_logical,
                 shared.v_logical, seed, "config4a_private")


def config4b(num_pairs: int = 64, poison: bool = False) -> Batch:
    """``num_pairs`` pairs (A, B) that share a 24-token prefix: one full block P0 and one block
    P1 holding 8 tokens. Sequence 2i is A and 2i+1 is B of pair i; both tables are [P0, P1]
    with room for one more entry. Before decoding, B appends one token, which needs a private
    copy of P1 first."""
    seed = SEED_BASE + 5
    B, Hq, Hkv, d, dt = 16, 64, 8, 128, torch.bfloat16
    S = 2 * num_pairs
    lengths = np.full(S, 24, dtype=np.int32)
    nblk = math.ceil(1.25 * 3 * num_pairs)   # P0, P1 and the copy target per pair
    perm = rng_for(seed, _PLACE).permutation(nblk).astype(np.int32)
    tables = np.full((S, 3), -1, dtype=np.int32)
    for i in range(num_pairs):
        tables[2 * i, :2] = perm[2 * i:2 * i + 2]
        tables[2 * i + 1, :2] = perm[2 * i:2 * i + 2]
    q = normal(rng_for(seed, _Q), (S, Hq, d), dt)
    rkv = rng_for(seed, _KV)
    k_pool, v_pool = empty_pools(nblk, Hkv, B, d, dt, poison)
    k_log, v_log = [], []
    for i in range(num_pairs):
        kk = normal(rkv, (Hkv, 24, d), dt)
        vv = normal(rkv, (Hkv, 24, d), dt)
        write_rows(k_pool, v_pool, tables[2 * i], kk, vv)
        k_log += [kk, kk]
        v_log += [vv, vv]
    return Batch(dt, B, Hq, Hkv, d, lengths, tables, nblk, q, k_pool, v_pool, k_log, v_log,
                 seed, "config4b")


def config4b_free_blocks(batch: Batch) -> list:
    """Pool blocks not referenced by any table of :func:`config4b`, in ascending order."""
    used = set(int(x) for x in batch.tables.ravel() if x >= 0)
    return [b for b in range(batch.num_blocks) if b not in used]


def config5(batch: int = 8, steps: int = 64, poison: bool = False,
            lengths=None) -> Batch:
    """Long contexts: L ~ U{16384..32768}, 64/8 heads, d=128, bf16, B=16; the tables have room
    for ``steps`` appended tokens per sequence and the pool is 1.25x the final need."""
    seed = SEED_BASE + 6
    B = 16
    if lengths is None:
        lengths = rng_for(seed, _LEN).integers(16384, 32768, size=batch,
                                               endpoint=True).astype(np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    final = lengths + steps
    need = sum(_ceil_div(int(x), B) for x in final)
    nblk = math.ceil(1.25 * need)
    max_blocks = max(_ceil_div(int(x), B) for x in final)
    tables, nblk, _ = place_blocks(lengths, B, rng_for(seed, _PLACE), num_blocks=nblk,
                                   max_blocks=max_blocks)
    return make_batch(lengths, 64, 8, 128, B, torch.bfloat16, seed, tables=tables,
                      num_blocks=nblk, poison=poison, note="config5")


def small_batch(lengths, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                dtype: torch.dtype, seed: int, poison: bool = False,
                pool_factor: float = 1.25) -> Batch:
    """A small random batch for parity cases (ragged lengths, several tiles, random placement)."""
    return make_batch(lengths, num_q_heads, num_kv_heads, head_dim, block_size, dtype, seed,
                      poison=poison, pool_factor=pool_factor, note="small")


def relabel(batch: Batch, seed: int) -> Batch:
    """Move every physical block to a new random slot and rewrite the tables to match."""
    rng = rng_for(seed, _PLACE)
    perm = rng.permutation(batch.num_blocks)
    # block b moves to slot perm[b]
    k_pool = torch.empty_like(batch.k_pool)
    v_pool = torch.empty_like(batch.v_pool)
    k_pool[torch.from_numpy(perm.astype(np.int64))] = batch.k_pool
    v_pool[torch.from_numpy(perm.astype(np.int64))] = batch.v_pool
    tables = batch.tables.copy()
    m = tables >= 0
    tables[m] = perm[tables[m]]
    return dataclasses.replace(batch, tables=tables.astype(np.int32), k_pool=k_pool,
                               v_pool=v_pool, note=batch.note + "_relabel")
