// Balanced streaming schedule for the decode kernels.
//
// The decode work is the set of 32-token "steps" of every (sequence, KV head) segment: segment
// (s, g) holds ns(s) = ceil(L_s / 32) steps, and segments are ordered (s, g). All steps are laid
// out in one line of N = H_kv * sum_s ns(s) steps, and worker w (one wavefront) streams the
// contiguous range [w*N/n, (w+1)*N/n) -- every worker reads the same number of K/V bytes to
// within one step, whatever the length mix. A worker's range crosses segment boundaries; each
// maximal run of one segment inside a range is a "piece". A piece that is a whole segment
// writes the normalised output directly. Only a worker's first and last piece can be part of a
// longer segment; those write a partial softmax state (m, l, acc) -- per-block partials of
// "Paged Attention and vLLM", section "Paged Attention CUDA Kernel" -- to slot 2w (first
// piece) or 2w+1 (last piece, when it is not also the first), and the merge kernel combines the
// partials of each split segment with the log-sum-exp rule of the same section.
//
// A worker computes its whole step schedule up front, 32 steps at a time: lane j of a chunk
// holds segment, step-in-segment and the physical block ids of step j (lane j + 32 holds the
// second block at block size 16), and the next chunk is prepared while the current one
// streams, so no dependent table load sits between two steps.
#pragma once

#include "device_common.h"

namespace pkv {

constexpr int kStepTokens = 32;
constexpr int kMaxSeqsPerCall = 4096;   // LDS holds the per-sequence step prefix

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Workgroup-wide exclusive prefix of ns(s) over s into sm_prefix[0..S] (sm_prefix[S] = total).
// All threads of the workgroup must call it.
__device__ inline void build_step_prefix(const int32_t* lens, int S, int cap, int64_t* sm_prefix,
                                         int64_t* sm_wave) {
  const int nthr = blockDim.x;
  const int t = threadIdx.x;
  const int per = (S + nthr - 1) / nthr;
  const int lo = t * per;
  const int hi = min(lo + per, S);
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += ceil_div(clamp_len(lens[i], cap), kStepTokens);
  // inclusive scan of the per-thread sums inside the wavefront
  const int lane = t & 63;
  int64_t inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  const int wave = t >> 6;
  if (lane == 63) sm_wave[wave] = inc;
  __syncthreads();
  int64_t base = 0;
  for (int w = 0; w < wave; ++w) base += sm_wave[w];
  int64_t run = base + inc - sum;   // exclusive prefix of this thread's first element
  for (int i = lo; i < hi; ++i) {
    sm_prefix[i] = run;
    run += ceil_div(clamp_len(lens[i], cap), kStepTokens);
  }
  if (t == nthr - 1) sm_prefix[S] = base + inc;
  __syncthreads();
}

// Largest s in [0, S) with Hkv * prefix[s] <= r (r < Hkv * prefix[S]).
__device__ __forceinline__ int find_seq(const int64_t* sm_prefix, int S, int Hkv, int64_t r) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)Hkv * sm_prefix[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// First step of worker w's range. The host guarantees N * n < 2^62.
__device__ __forceinline__ int64_t range_begin(int64_t N, int n, int w) {
  return (int64_t)(((uint64_t)N * (uint64_t)w) / (uint64_t)n);
}

// Worker that owns global step r < N: the largest w with range_begin(w) <= r.
__device__ __forceinline__ int worker_of(int64_t N, int n, int64_t r) {
  return (int)((((uint64_t)r + 1) * (uint64_t)n - 1) / (uint64_t)N);
}

// Dynamic LDS of a decode workgroup: the step prefix (S+1 int64), the per-wavefront partial
// sums (16 int64) and the clamped lengths (S int32).
inline size_t decode_lds_bytes(int num_seqs) {
  return ((size_t)num_seqs + 1 + 16) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

// Store the clamped lengths next to the prefix (all threads of the workgroup call it; a
// barrier follows in build_step_prefix's caller before use).
__device__ inline void stage_lengths(const int32_t* lens, int S, int cap, int32_t* sm_len) {
  for (int i = threadIdx.x; i < S; i += blockDim.x) sm_len[i] = clamp_len(lens[i], cap);
}

// Wave-uniform position in the step line: segment (s, g), step k of ns, sequence length L.
struct Cursor {
  int s, g, k, ns, L;
};

__device__ inline Cursor cursor_at(const int64_t* sm_prefix, const int32_t* sm_len, int S,
                                   int Hkv, int64_t r) {
  Cursor c;
  c.s = find_seq(sm_prefix, S, Hkv, r);
  const int64_t rem = r - (int64_t)Hkv * sm_prefix[c.s];
  c.ns = (int)(sm_prefix[c.s + 1] - sm_prefix[c.s]);
  c.g = (int)(rem / c.ns);
  c.k = (int)(rem - (int64_t)c.g * c.ns);
  c.L = sm_len[c.s];
  return c;
}

// Next step of the line (the caller knows one exists).
__device__ inline void cursor_next(Cursor& c, const int64_t* sm_prefix, const int32_t* sm_len,
                                   int Hkv) {
  if (++c.k < c.ns) return;
  c.k = 0;
  if (++c.g < Hkv) return;
  c.g = 0;
  do {
    ++c.s;
    c.ns = (int)(sm_prefix[c.s + 1] - sm_prefix[c.s]);
  } while (c.ns == 0);
  c.L = sm_len[c.s];
}

// Physical block of this lane's slot in a 32-step chunk starting at step r0 of the line: lane j
// holds the first block of step r0 + (j & 31), lane j + 32 the second (block size 16). -1 marks an
// out-of-range table entry, 0 a slot past the sequence (never used).
template <int B>
__device__ inline int chunk_blocks(const int64_t* sm_prefix, const int32_t* sm_len,
                                   const int32_t* tables, int S, int Hkv, int max_blocks,
                                   int num_blocks, int64_t r0, int64_t r1, int lane) {
  const int64_t r = r0 + (lane & 31);
  if (r >= r1) return 0;
  const Cursor c = cursor_at(sm_prefix, sm_len, S, Hkv, r);
  const int jb = (B == 16) ? 2 * c.k + (lane >> 5) : c.k;
  if (jb >= ceil_div(c.L, B)) return 0;
  const int b = tables[(size_t)c.s * max_blocks + jb];
  return ((unsigned)b < (unsigned)num_blocks) ? b : -1;
}

// Uniform description of one step of a worker's range.
struct StepInfo {
  int s, g, k, ns, L, b0, b1;
};

// Per-lane schedule of one 32-step chunk of a worker's range.
struct ChunkMeta {
  int s;      // sequence
  int g;      // KV head
  int k;      // step inside the segment
  int ns;     // steps in the segment
  int L;      // tokens of the sequence (clamped)
  int blk;    // physical block of this lane's block slot, -1 = out-of-range table entry
};

template <int B>
__device__ inline ChunkMeta make_chunk_meta(const int64_t* sm_prefix, const int32_t* lens,
                                            const int32_t* tables, int S, int Hkv, int cap,
                                            int max_blocks, int num_blocks, int64_t r0,
                                            int64_t r1, int lane) {
  ChunkMeta m{0, 0, 0, 1, 0, 0};
  const int64_t r = r0 + (lane & 31);
  if (r < r1) {
    const int s = find_seq(sm_prefix, S, Hkv, r);
    const int64_t base = (int64_t)Hkv * sm_prefix[s];
    const int ns = (int)(sm_prefix[s + 1] - sm_prefix[s]);
    const int64_t rem = r - base;
    m.s = s;
    m.ns = ns;
    m.g = (int)(rem / ns);
    m.k = (int)(rem - (int64_t)m.g * ns);
    m.L = clamp_len(lens[s], cap);
    const int jb = (B == 16) ? 2 * m.k + (lane >> 5) : m.k;
    const int nb = ceil_div(m.L, B);
    if (jb < nb) {
      const int b = tables[(size_t)s * max_blocks + jb];
      m.blk = ((unsigned)b < (unsigned)num_blocks) ? b : -1;
    }
  }
  return m;
}

}  // namespace pkv
