/*
 * pagedkv.h -- C ABI of the paged KV-cache decode library for AMD Instinct MI355X (gfx950).
 *
 * Single-query decode attention over a KV cache that lives in fixed-size physical blocks and
 * is addressed through a per-sequence block table, plus the two calls that mutate the cache
 * (append of new tokens, copy-on-write of a shared block) and a host-side refcounted block
 * pool. Around that path: decode of sequences that share a prefix (the shared blocks read once
 * for all sharers), extend attention (several new query tokens per sequence, causal), block
 * swap between the pools and pinned host memory, and a host prefix index (radix tree with
 * least-recently-used eviction) over the block pool.
 *
 * Sources, cited by page title and section:
 *   [P1] "PagedAttention: Virtual Memory for the KV Cache"
 *   [P2] "Paged Attention and vLLM"
 *   [P3] "KV Cache Optimization and Management"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: "device" pointers address GPU memory that the caller allocated (hipMalloc or a
 *   framework allocator); "host" pointers address CPU memory. The library never allocates,
 *   frees or retains device memory: the caller owns every buffer, including the decode
 *   workspace, whose size it queries first.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream). Every device
 *   call only enqueues work on that stream, in call order, and never synchronizes; ordering
 *   between calls (append, then decode) comes from the stream.
 * Errors: every int-returning call returns PKV_OK (0) or a negative PKV_ERR_* code and then
 *   pkv_last_error() describes the failure. On an error nothing has been enqueued.
 *   Host-side checks cover pointers, sizes, supported shapes and workspace size. Device-
 *   resident contents (table entries, lengths, positions) are the caller's contract; the
 *   kernels never access memory outside the pools for out-of-range contents (an attention row
 *   whose table holds an out-of-range entry comes out as NaN; an append or copy with an
 *   out-of-range target is skipped). Setting the environment variable PAGEDKV_VALIDATE=1
 *   makes each call copy those contents to the host first (a synchronizing debug mode) and
 *   return PKV_ERR_VALIDATION when they break the contract (pkv_set_validate switches the mode
 *   at run time).
 *
 * Cache layout (the pages leave it to the kernel, [P1] "Block size is a kernel choice too"):
 *   k_pool  [num_blocks][num_kv_heads][block_size][head_dim]   key rows of a block
 *   v_pool  [num_blocks][num_kv_heads][block_size][head_dim]   value rows, same order
 *   Both pools hold one layer and share the element type `kv_dtype`.
 * Token p of sequence s sits in physical block block_tables[s][p / block_size] at offset
 * p % block_size ([P1] "A block table preserves token order"; [P2] "Block Table and
 * Logical-to-Physical Mapping", tau_s).
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {16, 32}; kv_dtype PKV_F32, PKV_F16
 * or PKV_BF16; G = num_q_heads / num_kv_heads any integer for the decode calls (query heads
 * that one kernel segment cannot take -- more than 16 for 16-bit caches, a G outside
 * {1, 2, 4, 8} for PKV_F32 -- run as several equal groups over the same KV head, each group
 * reading its keys and values).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,          /* null pointer, negative size, inconsistent sizes   */
  PKV_ERR_UNSUPPORTED = -2,          /* head_dim / block_size / dtype / G not supported    */
  PKV_ERR_WORKSPACE_TOO_SMALL = -3,  /* decode workspace smaller than the queried size     */
  PKV_ERR_LAUNCH = -4,               /* the HIP runtime rejected a launch                  */
  PKV_ERR_POOL_EXHAUSTED = -5,       /* no free block in a pkv_pool                        */
  PKV_ERR_REFCOUNT = -6,             /* refcount would drop below zero / block not free    */
  PKV_ERR_VALIDATION = -7            /* PAGEDKV_VALIDATE=1 found a contract violation      */
};

/* Message for the last error on the calling thread ("" if none). Owned by the library. */
const char* pkv_last_error(void);

/* ---------------------------------------------------------------------------------------
 * Decode attention
 *
 * For every sequence s < num_seqs and query head h < num_q_heads, with g = h / G:
 *   out[s][h][:] = softmax( q[s][h] . K_s^T * scale ) . V_s
 * where K_s, V_s are the first context_lens[s] key and value rows of sequence s, read
 * through its block table: [P2] "Block Table and Logical-to-Physical Mapping" (the equation
 * for a_t, with V applied) -- the gather is fused, no contiguous copy is made. Keys and values
 * of KV head g serve the G query heads g*G .. g*G+G-1 (grouped-query attention, [P1] "Where
 * contiguous allocation wastes space" notes that GQA stores fewer KV heads).
 * Work split: the 32-token steps of all (sequence, KV head) pairs form one line, cut into one
 * contiguous range per wavefront ("worker") of equal weight, where a step weighs one unit and
 * the start of a pair about one more; so all workers finish close together whatever the
 * length mix (a KV head whose query heads one kernel segment cannot take counts as the
 * fewest equal groups that it can: of at most 16 query heads for 16-bit caches, of 1, 2, 4
 * or 8 for fp32 caches). A pair finished inside one range is written directly; a pair split
 * across ranges leaves one partial (m, l, acc) per range and a second kernel merges them with the
 * log-sum-exp rule of [P2] "Paged Attention CUDA Kernel" (exact up to rounding). The split
 * depends only on the lengths and num_workers, so a call is deterministic.
 * context_lens[s] == 0 gives a zero row.
 *
 *   out           device [num_seqs][num_q_heads][head_dim], element type out_dtype
 *                 (PKV_F32, or the same 16-bit type as kv_dtype: round to nearest even)
 *   q             device [num_seqs][num_q_heads][head_dim], element type kv_dtype
 *   k_pool,v_pool device, layout above
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(context_lens[s] / block_size) are never read
 *   context_lens  device int32 [num_seqs], each in [0, max_context_len] (values outside are
 *                 clamped to that range)
 *   max_context_len  host int, an upper bound of context_lens, at most
 *                 max_blocks_per_seq * block_size
 *   num_seqs      any number: a launch's schedule holds at most 4096 sequences, so a larger
 *                 batch runs as consecutive launches of at most 4096 on `stream`, each reusing
 *                 the workspace (sized for the whole batch); the results do not depend on the
 *                 split. paged_attn_decode_shared_prefix takes at most 4096.
 *   scale         softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   num_workers   0 = automatic (as many wavefronts as the chosen kernel keeps resident on
 *                 the current device, at most 8 per compute unit, and no more than
 *                 num_kv_heads * num_seqs * ceil(max_context_len / 32), the most 32-token
 *                 steps the call can have), else 1 .. 2^20 (any count gives the same result
 *                 up to rounding)
 *   workspace     device scratch, 256-byte aligned, of at least
 *                 pkv_decode_workspace_size(...) bytes for the same num_workers; no contents
 *                 are assumed between calls. Calls that overlap in time need separate
 *                 workspaces.
 * --------------------------------------------------------------------------------------- */
size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int num_workers);

/* The worker count that num_workers = 0 selects on the current device for a call with at
 * least that many 32-token steps (an upper bound on what it uses; it sizes the workspace). */
int pkv_decode_auto_workers(void);

int paged_attn_decode(void* out, int out_dtype, const void* q, const void* k_pool,
                      const void* v_pool, int kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, int num_workers,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * paged_attn_decode without a caller workspace, for callers that cannot allocate device
 * memory at the call site: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The same kernels and the same result, bit for bit, as paged_attn_decode
 * with the same arguments and num_workers; the decode's scratch (schedule prefixes and split
 * partial states) lives in a static device array of the library, PKV_DECODE_STATIC_SCRATCH
 * bytes on each GPU, held from the first call on that GPU until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine). A call whose
 * scratch need, pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
 * num_workers), exceeds that size fails with PKV_ERR_WORKSPACE_TOO_SMALL before enqueuing
 * anything. Every call on one GPU shares that GPU's array and leaves its contents behind:
 * calls that overlap in time on one GPU (other streams, other host threads) race and must be
 * serialized by the caller.
 * --------------------------------------------------------------------------------------- */
#define PKV_DECODE_STATIC_SCRATCH ((size_t)32 << 20)
int paged_attn_decode_noalloc(void* out, int out_dtype, const void* q, const void* k_pool,
                              const void* v_pool, int kv_dtype, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* context_lens,
                              int max_context_len, int num_seqs, int num_q_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              float scale, int num_workers, void* stream);

/* ---------------------------------------------------------------------------------------
 * Decode step with the step's append fused in: the same result, in the pools and in `out`,
 * as kv_cache_append of one token per sequence -- k_new[s] / v_new[s] at position
 * context_lens[s] - 1, for every s with context_lens[s] >= 1 -- followed by
 * paged_attn_decode, in one launch less ([P1] "Growing a request": a generated token's keys and
 * values join the cache and the next query attends to them). The worker that computes the
 * step holding that position reads the row from k_new / v_new; the rows are stored into their
 * slots by the same kernel. The table must already map position context_lens[s] - 1 (the host
 * grows it first, as for kv_cache_append); a slot whose table entry is out of range is not
 * written and, as in paged_attn_decode, that sequence's row comes out NaN.
 *   k_new, v_new  device [num_seqs][num_kv_heads][head_dim], element type kv_dtype
 *   other arguments as for paged_attn_decode; k_pool and v_pool are written.
 * --------------------------------------------------------------------------------------- */
int paged_attn_decode_append(void* out, int out_dtype, const void* q, void* k_pool, void* v_pool,
                             int kv_dtype, const void* k_new, const void* v_new,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int num_seqs,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int num_blocks, float scale, int num_workers, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Decode step of sequences that all begin with one shared prefix: the same result as
 * paged_attn_decode on the same arguments (up to rounding order), with the prefix's keys and
 * values read once per step for all sharers instead of once per sequence ([P1] "Sharing a
 * prefix and copying a partial block": sharers' tables point at the same full blocks; [P3]
 * "RadixAttention: caching, not just packing, the prefix": requests that begin with the same
 * prompt hold it once and differ only in their own suffixes). The softmax state of every
 * query row over the prefix and its state over the sequence's own suffix merge exactly by the
 * log-sum-exp rule ([P2] "Paged Attention CUDA Kernel"): one matrix-core kernel takes the
 * states of all S * G rows of each KV head over the prefix, the decode kernel runs over each
 * suffix, and a third kernel merges the two per row.
 *   prefix_blocks  device int32 [prefix_len / block_size]: the shared blocks, in token order
 *   prefix_len     tokens of the prefix: a positive multiple of block_size (only whole blocks
 *                  are shared), at most max_context_len
 *   block_tables   as for paged_attn_decode; entries [0, prefix_len / block_size) of every row
 *                  equal prefix_blocks and are not read
 *   context_lens   every context_lens[s] >= prefix_len (the suffix may be empty)
 *   workspace      device, 256-byte aligned, at least pkv_shared_prefix_workspace_size(...)
 *                  bytes for the same sizes, num_workers and prefix_len
 * 16-bit caches (PKV_ERR_UNSUPPORTED otherwise), any number of query heads per KV head; one call
 * per group of sequences that share a prefix. Under PAGEDKV_VALIDATE the shared table entries,
 * the lengths and the prefix ids are checked first.
 * --------------------------------------------------------------------------------------- */
size_t pkv_shared_prefix_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                        int head_dim, int num_workers, int prefix_len);
int paged_attn_decode_shared_prefix(void* out, int out_dtype, const void* q, const void* k_pool,
                                    const void* v_pool, int kv_dtype,
                                    const int32_t* prefix_blocks, int prefix_len,
                                    const int32_t* block_tables, int max_blocks_per_seq,
                                    const int32_t* context_lens, int max_context_len,
                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks, float scale,
                                    int num_workers, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------------------
 * Extend (multi-query) attention: several new query tokens per sequence -- a prefill chunk
 * past a cached prefix, or speculated tokens to verify -- attend causally to the paged cache
 * ([P3] "RadixAttention: caching, not just packing, the prefix": a request whose prefix is
 * already cached runs a fresh prefill pass over its new tokens only; [P1] "Sharing a prefix
 * and copying a partial block"). The new tokens' keys and values are already stored
 * (kv_cache_append first). Sequence s owns query rows query_start[s] .. query_start[s+1] - 1
 * (n_s rows); its cache holds context_lens[s] = L_s tokens, the last n_s of them the new ones,
 * and new token t attends to positions 0 .. L_s - n_s + t:
 *   out[query_start[s] + t][h] = softmax(q[..][h] . K_s[0 .. L_s - n_s + t]^T * scale) . V_s[..]
 *   out, q         device [num_query_tokens][num_q_heads][head_dim]; q in kv_dtype, out fp32
 *                  or kv_dtype
 *   query_start    device int32 [num_seqs + 1], from 0 to num_query_tokens, nondecreasing
 *   max_query_len  host: the largest n_s (sizes the launch and the workspace)
 *   workspace      device, 256-byte aligned, pkv_extend_workspace_size(...) bytes for the same
 *                  sizes
 * Other arguments as for paged_attn_decode. 16-bit caches only (PKV_ERR_UNSUPPORTED otherwise).
 * Each tile of 32 query rows (32 / G new tokens of one KV head) reads its keys and values once
 * when max_query_len * G < 128 (speculative verification); longer runs (prefill chunks) share
 * each step's keys and values among a workgroup's four 32-row tiles. Starts outside
 * [0, num_query_tokens] are clamped (never read outside q or out); PAGEDKV_VALIDATE checks the
 * starts, n_s <= max_query_len, n_s <= L_s and the table entries.
 * --------------------------------------------------------------------------------------- */
size_t pkv_extend_workspace_size(int num_seqs, int num_query_tokens, int num_q_heads,
                                 int num_kv_heads, int head_dim, int max_query_len,
                                 int max_context_len);
int paged_attn_extend(void* out, int out_dtype, const void* q, const int32_t* query_start,
                      int num_query_tokens, int max_query_len, const void* k_pool,
                      const void* v_pool, int kv_dtype, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Append: store the keys and values of new tokens into their slots
 * ([P1] "Growing a request"; [P2] "KV Cache Fundamentals": the cache grows by one row per
 * head per generated token). For every i < num_tokens and KV head g:
 *   slot = (block_tables[seq_ids[i]][positions[i] / block_size], positions[i] % block_size)
 *   k_pool[slot.block][g][slot.offset][:] = k_new[i][g][:]
 *   v_pool[slot.block][g][slot.offset][:] = v_new[i][g][:]
 * The caller has already grown the table (and made shared blocks private, see
 * cow_block_copy). Slots must be distinct; a bitwise copy, no rounding.
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_dim], element type kv_dtype;
 *                 num_tokens * num_kv_heads * head_dim < 2^31 per call
 *   seq_ids, positions  device int32 [num_tokens]
 * --------------------------------------------------------------------------------------- */
int kv_cache_append(void* k_pool, void* v_pool, int kv_dtype, const void* k_new,
                    const void* v_new, const int32_t* seq_ids, const int32_t* positions,
                    int num_tokens, const int32_t* block_tables, int max_blocks_per_seq,
                    int num_seqs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    void* stream);

/* ---------------------------------------------------------------------------------------
 * Copy-on-write: copy the first n token slots of block src into block dst, for every KV
 * head, keys and values ([P1] "Sharing a prefix and copying a partial block"; [P2]
 * "Continuous Batching and Scheduler", the copy-on-write rule). Slots >= n of dst are left as
 * they are. The host redirects the table entry and adjusts reference counts (pkv_pool_*).
 *   src_blocks, dst_blocks  device int32 [num_pairs]; src != dst, all destinations distinct
 *   num_tokens  device int32 [num_pairs] in [0, block_size], or NULL = whole blocks
 * --------------------------------------------------------------------------------------- */
int cow_block_copy(void* k_pool, void* v_pool, int kv_dtype, const int32_t* src_blocks,
                   const int32_t* dst_blocks, const int32_t* num_tokens, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int num_blocks, void* stream);

/* ---------------------------------------------------------------------------------------
 * Block swap between the device pools and a pool of blocks in host memory ([P2] "Continuous
 * Batching and Scheduler": a preempted sequence's physical blocks are evicted to CPU memory a
 * block at a time and swapped back when it resumes, so resuming costs only those blocks).
 *   host_k, host_v  host [num_host_blocks][num_kv_heads][block_size][head_dim], element type
 *                   kv_dtype: the device pools' block shape. They must be pinned host memory
 *                   that the device can address (hipHostMalloc, or a framework's pinned
 *                   allocator); anything else is rejected with PKV_ERR_INVALID_ARG before a
 *                   launch. The caller owns them and sizes them for num_host_blocks blocks.
 *   device_blocks, host_blocks  int32 [num_pairs], device memory or pinned host memory.
 * kv_swap_out copies device block device_blocks[i] (every head, every slot, keys and values)
 * to host block host_blocks[i]; kv_swap_in copies host block host_blocks[i] to device block
 * device_blocks[i]. Destinations must be distinct; a pair with an id outside its pool is
 * skipped. One launch moves the whole list, reading or writing host memory directly across
 * the host link. The copy is complete when the stream reaches it: synchronize (or wait on an
 * event) before the host reads host_k / host_v, and before it reuses evicted device blocks
 * from another stream. Which blocks to evict, and the table and reference-count bookkeeping
 * (pkv_pool_* on a second pool of host block ids), are the caller's.
 * --------------------------------------------------------------------------------------- */
int kv_swap_out(const void* k_pool, const void* v_pool, int kv_dtype, void* host_k,
                void* host_v, int num_host_blocks, const int32_t* device_blocks,
                const int32_t* host_blocks, int num_pairs, int num_kv_heads, int head_dim,
                int block_size, int num_blocks, void* stream);
int kv_swap_in(void* k_pool, void* v_pool, int kv_dtype, const void* host_k, const void* host_v,
               int num_host_blocks, const int32_t* host_blocks, const int32_t* device_blocks,
               int num_pairs, int num_kv_heads, int head_dim, int block_size, int num_blocks,
               void* stream);

/* Block swap through the copy engines (the same section of "Paged Attention and vLLM"). The
 * same transfer as kv_swap_out / kv_swap_in for a contiguous run of host blocks
 * [host_block0, host_block0 + num_pairs): the device side goes through a caller-owned staging
 * buffer (one launch gathers device_blocks[i] into staging block i, or scatters staging block
 * i to device_blocks[i]; keys first, then values, each num_pairs blocks), and the host side is
 * one DMA copy per pool between the staging buffer and the host run (hipMemcpyAsync on
 * `stream`). The host link is then carried by the copy engines instead of compute units, so a
 * decode running on another stream meanwhile keeps its CUs for all but the short gather or
 * scatter launch.
 *   staging         device memory of at least pkv_swap_staging_size(...) bytes, 16-byte
 *                   aligned, caller-owned; its contents are scratch.
 *   host_k, host_v  as for kv_swap_out: pinned host memory of num_host_blocks blocks
 *                   (PKV_ERR_INVALID_ARG otherwise, before anything is enqueued).
 *   device_blocks   int32 [num_pairs], device memory. kv_swap_in_dma's must be distinct. An
 *                   id outside [0, num_blocks) is skipped on the device side: kv_swap_in_dma
 *                   writes no device block for it, and kv_swap_out_dma's host block for it
 *                   receives whatever its staging block held (PAGEDKV_VALIDATE=1 rejects both).
 * Errors: PKV_ERR_INVALID_ARG (sizes, null or misaligned pointers, a host run outside
 * [0, num_host_blocks)), PKV_ERR_WORKSPACE_TOO_SMALL (staging), PKV_ERR_LAUNCH. Asynchronous:
 * the copy is complete when the stream reaches it. */
size_t pkv_swap_staging_size(int num_pairs, int num_kv_heads, int head_dim, int block_size,
                             int kv_dtype);
int kv_swap_out_dma(const void* k_pool, const void* v_pool, int kv_dtype, void* host_k,
                    void* host_v, int num_host_blocks, const int32_t* device_blocks,
                    int host_block0, int num_pairs, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, void* staging, size_t staging_bytes,
                    void* stream);
int kv_swap_in_dma(void* k_pool, void* v_pool, int kv_dtype, const void* host_k,
                   const void* host_v, int num_host_blocks, int host_block0,
                   const int32_t* device_blocks, int num_pairs, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, void* staging, size_t staging_bytes,
                   void* stream);

/* ---------------------------------------------------------------------------------------
 * Host block pool: free list and reference counts of `num_blocks` physical block ids. No
 * device memory. A block returns to the free list only when its count reaches zero
 * ([P3] "PagedAttention: borrowing virtual memory", answer A6); a full pool is reported, not
 * overwritten ([P1] "Growing a request": the scheduler needs an explicit policy).
 * A pkv_pool is not thread-safe.
 * --------------------------------------------------------------------------------------- */
typedef struct pkv_pool pkv_pool;

pkv_pool* pkv_pool_create(int num_blocks);            /* NULL on bad size / no memory      */
void pkv_pool_destroy(pkv_pool* pool);
int pkv_pool_alloc(pkv_pool* pool, int32_t* out_block);  /* lowest free id, count 1         */
int pkv_pool_claim(pkv_pool* pool, int32_t block);       /* take a named free block         */
int pkv_pool_incref(pkv_pool* pool, int32_t block);      /* +1 on a live block              */
int pkv_pool_decref(pkv_pool* pool, int32_t block, int* freed);  /* -1; *freed = 1 at zero  */
int pkv_pool_refcount(const pkv_pool* pool, int32_t block);      /* count, or <0 on error   */
int pkv_pool_num_free(const pkv_pool* pool);

/* ---------------------------------------------------------------------------------------
 * Host prefix index over a pkv_pool: a radix tree of cached token sequences whose edges own
 * runs of whole blocks ([P3] "RadixAttention: caching, not just packing, the prefix": requests
 * that share a prefix share its path; a new request reuses every matched token's blocks and
 * prefills only the rest; the least recently used leaves are trimmed first and a branch still
 * referenced by a running request is never evicted). Sharing is by whole blocks of block_size
 * tokens. The index holds one pool reference per cached block. No device memory; not
 * thread-safe; destroy the index before its pool.
 *
 * pkv_prefix_index_match: the physical blocks of the longest cached whole-block prefix of
 *   tokens[0, num_tokens) (at most max_blocks of them) into out_blocks, their count into
 *   *matched_blocks; each gets one pool reference for the caller, which releases it with the
 *   sequence (pkv_seq_release / pkv_pool_decref). Marks the matched path as just used.
 * pkv_prefix_index_insert: cache the whole blocks of a computed sequence; blocks[j] holds its
 *   tokens [j * block_size, (j + 1) * block_size) and must be live in the pool
 *   (PKV_ERR_REFCOUNT otherwise, nothing changed). A prefix that is already cached keeps its
 *   cached block. *inserted_blocks = blocks that became cached (one index reference each).
 * pkv_prefix_index_evict: free up to max_blocks blocks, one at a time, each the least recently
 *   used last block of a leaf that only the index references (ties: lower id); their ids go
 *   to freed_ids (may be NULL) in that order, their count to *freed_blocks.
 * pkv_prefix_index_size: blocks the index holds.
 * --------------------------------------------------------------------------------------- */
typedef struct pkv_prefix_index pkv_prefix_index;

pkv_prefix_index* pkv_prefix_index_create(pkv_pool* pool, int block_size);  /* NULL on error */
void pkv_prefix_index_destroy(pkv_prefix_index* index);      /* drops the index's references */
int pkv_prefix_index_match(pkv_prefix_index* index, const int32_t* tokens, int num_tokens,
                           int32_t* out_blocks, int max_blocks, int* matched_blocks);
int pkv_prefix_index_insert(pkv_prefix_index* index, const int32_t* tokens, int num_tokens,
                            const int32_t* blocks, int* inserted_blocks);
int pkv_prefix_index_evict(pkv_prefix_index* index, int max_blocks, int32_t* freed_ids,
                           int* freed_blocks);
int pkv_prefix_index_size(const pkv_prefix_index* index);

/* Table helpers on one host table row (int32 [max_blocks]) of a sequence that currently
 * holds `length` tokens.
 *
 * pkv_seq_prepare_write: make the slot of token `length` writable by this sequence alone.
 *   If it starts a new logical block, a block is allocated and appended to the row
 *   (*cow_n = -1). If it falls in a block whose count is > 1 (shared, partially filled), a
 *   fresh block is allocated, the row entry is redirected to it, the old block loses one
 *   reference, and (*cow_src, *cow_dst, *cow_n) name the copy the caller must enqueue with
 *   cow_block_copy before writing (n = length % block_size). Otherwise nothing changes
 *   (*cow_n = -1). *block and *offset receive the slot of token `length`.
 * pkv_seq_fork: dst_row = src_row[0:num_blocks_used], one more reference on each block.
 * pkv_seq_release: drop one reference on each of the first num_blocks_used entries; returns
 *   the number of blocks that went back to the free list (or an error code).
 */
int pkv_seq_prepare_write(pkv_pool* pool, int32_t* table_row, int max_blocks, int length,
                          int block_size, int32_t* block, int32_t* offset, int32_t* cow_src,
                          int32_t* cow_dst, int32_t* cow_n);
int pkv_seq_fork(pkv_pool* pool, const int32_t* src_row, int32_t* dst_row, int num_blocks_used);
int pkv_seq_release(pkv_pool* pool, const int32_t* table_row, int num_blocks_used);

/* ---------------------------------------------------------------------------------------
 * Kernel timing (for tests and benchmarks). pkv_timing_enable(k) with k > 0 brackets every
 * k-th launch of each kernel this library launches by a pair of hipEvents recorded on its
 * launch stream (k = 1: every launch; a larger k keeps the events' own cost out of most
 * launches); k = 0 switches timing off. pkv_timing_query waits for the recorded events of
 * kernels whose name contains `name` ("decode_partial", "splitk_reduce", "append", "cow", or
 * "" for all) and returns their summed duration and the number of timed launches. Enabling
 * clears earlier records.
 * --------------------------------------------------------------------------------------- */
int pkv_timing_enable(int on);
int pkv_timing_query(const char* name, double* total_ms, int64_t* launches);

/* Streaming-read probe (measurement only): one kernel that reads `bytes` of device memory at
 * `src` once with 16-byte loads, so that a benchmark can report the decode bandwidth as a
 * fraction of what plain reads reach on the same device as well as of the vendor peak.
 *   src    device, 16-byte aligned; bytes a positive multiple of 16
 *   sink   device uint32, written only in a case that does not occur (keeps the loads alive)
 * Asynchronous on `stream`; time it with events or pkv_timing_query("stream_read").
 * PKV_ERR_INVALID_ARG for null pointers, misalignment or a bad size. */
int pkv_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Matrix-core probe (measurement only): `workgroups` workgroups of 4 wavefronts, each issuing
 * `iters` rounds of 8 independent 16x16x32 bf16 MFMAs (16,384 flops each, no memory traffic),
 * so that a benchmark can compare MFMA-bound kernels with what the matrix cores sustain.
 *   sink   device float, written only in a case that does not occur
 * Asynchronous on `stream`; time it with pkv_timing_query("mfma_rate").
 * PKV_ERR_INVALID_ARG for a null sink or non-positive counts. */
int pkv_mfma_rate_probe(int workgroups, int iters, float* sink, void* stream);

/* Contract validation on (1) or off (0) for this process, overriding PAGEDKV_VALIDATE. */
int pkv_set_validate(int on);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
