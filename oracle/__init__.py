"""CPU oracle for paged decode attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 statement of what the
decode path computes. It exists so that tests can check the HIP library against it. Only
``tests/``, the smoke check in ``__graft_entry__.py`` and the CPU-baseline leg of
``bench.py`` may import it; the library under ``paged_kv_cache_127_amd/`` never does, and
this package imports nothing from there.

Sources (web pages; cited by title and section):
  * "PagedAttention: Virtual Memory for the KV Cache" -- block counts, the block table and
    its indexing rule, growth, prefix sharing and copy-on-write of a partial block.
  * "Paged Attention and vLLM" -- the attention equation over table-gathered keys, the
    per-block partial softmax and its log-sum-exp merge, the copy-on-write rule, block swap of
    a preempted sequence to CPU memory and back.
  * "KV Cache Optimization and Management" -- reference counting, release at count zero,
    worked capacity examples, the prefix index (match, insert, least-recently-used eviction of
    unreferenced leaves) in ``oracle.prefix_index``.

Every function here is pinned by ``tests/test_oracle_*.py`` to values the pages print,
closed forms, library routines or brute force, not to itself. No function is "parity
unpinned".
"""
from .attention import (attend, contiguous_decode, extend_attention, gather_kv, merge_states,
                        paged_decode, paged_decode_split, partial_state, shared_prefix_decode,
                        token_address)
from .bookkeeping import (BlockPool, PagedKVModel, RefcountError, PoolExhausted,
                          blocks_for, copy_blocks, capacity_report, reserved_slots, shareable_prefix_blocks)

__all__ = [
    "attend", "contiguous_decode", "extend_attention", "gather_kv", "merge_states",
    "paged_decode", "paged_decode_split", "partial_state", "shared_prefix_decode",
    "token_address", "BlockPool",
    "PagedKVModel", "RefcountError", "PoolExhausted", "blocks_for", "copy_blocks", "capacity_report",
    "reserved_slots", "shareable_prefix_blocks",
]
