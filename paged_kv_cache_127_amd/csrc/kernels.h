// Internal launch interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "schedule.h"

namespace pkv {

// Kernel launches. When the library's timing layer has armed a pair of events for the calling
// thread, the next launch goes through hipExtLaunchKernelGGL, which stamps those events with the
// kernel's own start and end (the dispatch's timestamps, as a kernel-trace profiler reports
// them) instead of separate event packets around the launch; otherwise a plain launch.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool used = false;
};
LaunchEvents& launch_events();   // per host thread (api.hip)

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                          hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start && !ev.used) {
    ev.used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, ev.start, ev.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

// Decode over the balanced step schedule (schedule.h). kv_dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int head_dim, int block_size,
                              int waves, hipStream_t st);
hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, int head_dim, int block_size,
                              int group, int waves, hipStream_t st);
// Wavefronts of the decode kernel that fit on one compute unit at once (0 if unknown).
int decode_mfma_resident_waves(int kv_dtype, int head_dim, int block_size, int group, int waves,
                               int num_seqs);

// Dynamic LDS of the matrix-core decode kernel, after the schedule arrays: per wavefront a
// value staging tile (32 token rows of D 16-bit elements, re-read transposed as MFMA operands)
// and an output ring of ring_capacity staged piece results (G rows x D floats plus 2 G floats,
// each with a 16-byte header). The ring takes what the workgroup's LDS has left, at most
// kRingBudgetBytes and 16 entries per wavefront, at least one entry.
constexpr size_t kLdsPerWorkgroup = 160 * 1024;   // gfx950
constexpr size_t kRingBudgetBytes = 32 * 1024;    // per wavefront
inline size_t value_stage_bytes(int head_dim) { return (size_t)32 * head_dim * 2; }
inline size_t ring_entry_bytes(int group, int head_dim) {
  return 16 + 4 * ((size_t)group * head_dim + 2 * (size_t)group);
}
inline int ring_capacity(int num_seqs, int group, int head_dim, int waves) {
  const size_t per = ring_entry_bytes(group, head_dim);
  const size_t fixed = ring_offset(num_seqs) + (size_t)waves * value_stage_bytes(head_dim);
  size_t r = kRingBudgetBytes / per;
  const size_t fit = fixed < kLdsPerWorkgroup ? (kLdsPerWorkgroup - fixed) / ((size_t)waves * per) : 0;
  if (fit < r) r = fit;
  return r < 1 ? 1 : (r > 16 ? 16 : (int)r);
}
inline size_t mfma_lds_bytes(int num_seqs, int group, int head_dim, int waves) {
  return ring_offset(num_seqs) +
         (size_t)waves * (value_stage_bytes(head_dim) +
                          ring_capacity(num_seqs, group, head_dim, waves) *
                              ring_entry_bytes(group, head_dim));
}
int decode_valu_resident_waves(int kv_dtype, int head_dim, int block_size, int group, int waves,
                               int num_seqs);
hipError_t launch_splitk_reduce(const DecodeParams& p, int kv_dtype, int head_dim,
                                hipStream_t st);

// Softmax states of many query rows over one block list (row_states.hip): the shared-prefix
// pass (all sharers' rows over the shared blocks; the merge kernel folds them with the suffix
// decode's results) and extend attention (each sequence's new-token rows over its own blocks,
// causal; extend_finish folds and normalises).
struct RowStateParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* lens;            // [S] context lengths
  // prefix mode (query_start null)
  const int32_t* prefix_blocks;   // [prefix_len / block_size]
  int32_t* suffix_lens;           // [S] out: max(lens - prefix_len, 0)
  int prefix_len;                 // tokens, a multiple of the block size
  // extend mode (query_start set)
  const int32_t* query_start;     // [S + 1] first query row of each sequence
  const int32_t* tables;          // [S][max_blocks]
  int max_blocks;
  int max_row_groups;             // row groups of the longest query run
  int num_query_tokens;           // T
  float* st_m;                    // [chunk_groups][state_rows]
  float* st_l;                    // [chunk_groups][state_rows]
  float* st_acc;                  // [chunk_groups][state_rows][D]
  void* out;                      // extend mode with one chunk group: the normalised rows
                                  // [T * Hq][D] go here directly (states unused); else null
  int out_f32;                    // out is fp32 (else the cache's 16-bit type)
  size_t state_rows;              // S * Hq (prefix mode) or T * Hq (extend mode)
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int num_blocks;
  int chunk_groups;
  int steps_per_chunk;            // planned 32-token steps per wavefront (the kernel splits each
                                  // row group's own steps evenly)
  float scale_log2;
};
struct ExtendFinishParams {
  void* out;                      // [rows][D], fp32 or the cache's 16-bit type
  const float* st_m;
  const float* st_l;
  const float* st_acc;
  size_t rows;                    // T * Hq
  int chunk_groups;
  int out_f32;
};
// Chunk groups and steps per wavefront for `base_workgroups` workgroups per chunk group over
// up to max_tokens tokens: at least one workgroup per CU, at most 32 steps per wavefront and
// 16 groups.
void row_state_plan(int64_t base_workgroups, int max_tokens, int num_cus, int* chunk_groups,
                    int* steps_per_chunk);
int64_t row_groups(int64_t rows);   // row groups (of one wavefront's rows) covering `rows`
hipError_t launch_row_states(const RowStateParams& p, int kv_dtype, int head_dim,
                             int block_size, hipStream_t st);
hipError_t launch_extend_finish(const ExtendFinishParams& p, int kv_dtype, int head_dim,
                                hipStream_t st);
// Extend attention with workgroup-shared key/value tiles (runs of new tokens whose rows per KV
// head reach 128): 128-row groups covering `rows`, and the chunk groups for `base_workgroups`
// workgroups per chunk group over up to max_tokens tokens (one whenever they fill the CUs).
int64_t wide_row_groups(int64_t rows);
void wide_row_plan(int64_t base_workgroups, int max_tokens, int num_cus, int* chunk_groups);
hipError_t launch_extend_rows_shared(const RowStateParams& p, int kv_dtype, int head_dim,
                                     int block_size, hipStream_t st);
// Prefix states (prefix mode of RowStateParams) on the same kernel: grid = KV heads x 128-row
// groups of the S * G rows x chunk groups.
hipError_t launch_wide_prefix_states(const RowStateParams& p, int kv_dtype, int head_dim,
                                     int block_size, hipStream_t st);

struct AppendParams {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_ids;
  const int32_t* positions;
  const int32_t* tables;
  int num_tokens;
  int max_blocks;
  int num_seqs;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int num_blocks;
};
hipError_t launch_append(const AppendParams& p, int elem_bytes, hipStream_t st);

struct CowParams {
  void* k_pool;
  void* v_pool;
  const int32_t* src;
  const int32_t* dst;
  const int32_t* ntok;   // may be null: whole blocks
  int num_pairs;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int num_blocks;
};
hipError_t launch_cow(const CowParams& p, int elem_bytes, hipStream_t st);

// Whole-block copy between two pools of one block shape (swap.hip): block src_ids[i] of
// (src_k, src_v) to block dst_ids[i] of (dst_k, dst_v). `units` = 16-byte units per block of
// one pool; every base pointer is 16-byte aligned. One side may be mapped host memory.
struct SwapParams {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* src_ids;         // null: pair i reads block i (a staging buffer)
  const int32_t* dst_ids;         // null: pair i writes block i
  int num_pairs;
  int src_count;   // blocks in the source pool
  int dst_count;   // blocks in the destination pool
  int units;
};
hipError_t launch_block_copy(const SwapParams& p, int num_cus, hipStream_t st);

// Streaming-read probe (probe.hip): reads `bytes` (multiple of 16) of src once.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int num_cus,
                              hipStream_t st);
// Matrix-core probe (probe.hip): 4 wavefronts per workgroup, each `iters` x 8 independent
// 16x16x32 bf16 MFMAs (16,384 flops each).
hipError_t launch_mfma_rate(int workgroups, int iters, float* sink, hipStream_t st);

}  // namespace pkv
