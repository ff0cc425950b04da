// Balanced static streaming schedule for the decode kernels.
//
// The decode work is the set of 32-token "steps" of every (sequence, KV head) segment: segment
// (s, g) holds ns(s) = ceil(L_s / 32) steps, and segments are ordered (s, g), so all steps form
// one line of N = H_kv * sum_s ns(s) steps. Each worker (one wavefront) takes one contiguous
// range of that line, so every worker reads about the same number of K/V bytes whatever the
// length mix.
//
// A range crosses segment boundaries; each maximal run of one segment inside a range is a
// "piece". Starting a piece costs time of its own (its query rows, the end-of-piece reduction
// and output write), so the ranges are cut on a weighted line, not on the step count: every
// step weighs kStepWeight and every segment start weighs piece_weight more (a weightless mark
// placed before its first step). A worker owns the steps whose weighted start falls in its
// equal share [N_w * w / n, N_w * (w + 1) / n) of the weighted total N_w; those are still a
// contiguous run of steps, so nothing downstream changes. A range full of short sequences thus
// holds fewer steps than one inside a long sequence, and both take about the same time.
//
// A piece that is a whole segment writes the normalised output directly. Only the first and
// the last piece of a range can be part of a longer segment; those write a partial softmax
// state (m, l, acc) -- the per-block partials of "Paged Attention and vLLM", section "Paged
// Attention CUDA Kernel" -- to slot 2w (first piece) or 2w+1 (last piece, when it is not also
// the first) of worker w, and the merge kernel combines the partials of each split segment with
// the log-sum-exp rule of the same section.
//
// A worker walks its range with a wave-uniform cursor held in scalar registers. The physical
// block ids of a step come from scalar loads of the block table, issued two steps before the
// step's K/V loads, so no dependent table load sits between two steps and no vector-memory
// wait is ever spent on the schedule.
#pragma once

#include "device_common.h"

namespace pkv {

constexpr int kStepTokens = 32;
constexpr int kStepWeight = 4;          // weight of one step on the cut line
constexpr int kMaxSeqsPerCall = 4096;   // LDS holds the per-sequence prefixes
constexpr int kNonEmptyBits = 13;       // packs (steps, non-empty count <= 4096) into one int64

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Wave-uniform copies (scalar registers) of values every lane holds alike, e.g. LDS reads at a
// uniform address: branches on them are scalar branches, not exec-mask regions.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The block table seen through the constant address space: loads at uniform addresses become
// scalar loads (the table is read-only during a call).
typedef const __attribute__((address_space(4))) int32_t* ctable_t;

// Workgroup-wide exclusive prefixes over s of the steps ns(s) (into steps[0..S]) and of the
// weights kStepWeight * ns(s) + piece_weight * [ns(s) > 0] (into wts[0..S]). All threads of the
// workgroup must call it; sm_wave holds 16 int64.
__device__ inline void build_prefixes(const int32_t* lens, int S, int cap, int piece_weight,
                                      int64_t* steps, int64_t* wts, int64_t* sm_wave) {
  const int nthr = blockDim.x;
  const int t = threadIdx.x;
  const int per = (S + nthr - 1) / nthr;
  const int lo = t * per;
  const int hi = min(lo + per, S);
  auto packed = [&](int i) -> int64_t {
    const int ns = ceil_div(clamp_len(lens[i], cap), kStepTokens);
    return ((int64_t)ns << kNonEmptyBits) + (ns > 0 ? 1 : 0);
  };
  auto store = [&](int i, int64_t v) {
    const int64_t st = v >> kNonEmptyBits;
    const int64_t ne = v & ((1 << kNonEmptyBits) - 1);
    steps[i] = st;
    wts[i] = kStepWeight * st + (int64_t)piece_weight * ne;
  };
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += packed(i);
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
    store(i, run);
    run += packed(i);
  }
  if (t == nthr - 1) store(S, base + inc);
  __syncthreads();
}

// Largest s in [0, S) with Hkv * prefix[s] <= r (r < Hkv * prefix[S]); for a prefix that is
// constant over empty sequences this is a sequence with work. Wave-parallel: the predicate is
// monotone in s, so a ballot over 64 candidates brackets the answer -- one round for S <= 64,
// two (every stride-th entry, then the stride entries that follow the last passing one) for
// S <= 4096. All 64 lanes of the wavefront must be active.
__device__ inline int find_seq(const int64_t* prefix, int S, int Hkv, int64_t r) {
  const int lane = threadIdx.x & 63;
  const int stride = (S + 63) >> 6;
  int base = 0, cnt = S;
  if (stride > 1) {
    const int c = stride * lane;
    const bool ok = c < S && (int64_t)Hkv * prefix[c < S ? c : 0] <= r;
    base = stride * ((int)__popcll(__ballot(ok)) - 1);   // prefix[0] = 0 always passes
    cnt = S - base < stride ? S - base : stride;
  }
  const int c = base + lane;
  const bool ok = lane < cnt && (int64_t)Hkv * prefix[lane < cnt ? c : base] <= r;
  return base + (int)__popcll(__ballot(ok)) - 1;
}

// Start of share w of a line of N units cut into n shares. The host guarantees N * n < 2^62.
__device__ __forceinline__ int64_t range_begin(int64_t N, int n, int w) {
  return (int64_t)(((uint64_t)N * (uint64_t)w) / (uint64_t)n);
}

// Share that holds unit r < N: the largest w with range_begin(w) <= r.
__device__ __forceinline__ int worker_of(int64_t N, int n, int64_t r) {
  return (int)((((uint64_t)r + 1) * (uint64_t)n - 1) / (uint64_t)N);
}

// The weighted cut of the step line (prefix arrays in LDS or global memory).
struct Line {
  const int64_t* steps;   // [S + 1] step prefix
  const int64_t* wts;     // [S + 1] weight prefix
  int S, Hkv, pw, n;
  int64_t N, Nw;          // steps, total weight

  __device__ static Line make(const int64_t* steps, const int64_t* wts, int S, int Hkv, int pw,
                              int n) {
    Line l;
    l.steps = steps;
    l.wts = wts;
    l.S = S;
    l.Hkv = Hkv;
    l.pw = pw;
    l.n = n;
    l.N = (int64_t)Hkv * uni(steps[S]);
    l.Nw = (int64_t)Hkv * uni(wts[S]);
    return l;
  }
  // The same cut from the totals alone (steps[S], wts[S]); for code that needs no search.
  __device__ static Line from_totals(int64_t steps_total, int64_t wts_total, int S, int Hkv,
                                     int pw, int n) {
    Line l;
    l.steps = nullptr;
    l.wts = nullptr;
    l.S = S;
    l.Hkv = Hkv;
    l.pw = pw;
    l.n = n;
    l.N = (int64_t)Hkv * steps_total;
    l.Nw = (int64_t)Hkv * wts_total;
    return l;
  }
  __device__ int64_t wbegin(int w) const { return range_begin(Nw, n, w); }
  __device__ int owner(int64_t x) const { return worker_of(Nw, n, x); }

  // Steps of one segment (ns steps, weighted start ws0) whose weighted start is below x.
  __device__ int64_t in_segment_before(int64_t x, int64_t ws0, int64_t ns) const {
    const int64_t off = x - ws0 - pw;   // steps start at ws0 + pw + kStepWeight * k
    if (off <= 0) return 0;
    const int64_t c = (off + kStepWeight - 1) / kStepWeight;
    return c < ns ? c : ns;
  }

  // Steps of the whole line whose weighted start is below x (0 <= x <= Nw).
  __device__ int64_t steps_before(int64_t x) const {
    if (x >= Nw) return N;
    const int s = find_seq(wts, S, Hkv, x);
    const int64_t st0 = uni(steps[s]);
    const int64_t ns = uni(steps[s + 1]) - st0;
    const int64_t seg_w = kStepWeight * ns + pw;
    const int64_t w0 = (int64_t)Hkv * uni(wts[s]);
    const int64_t g = (x - w0) / seg_w;
    return (int64_t)Hkv * st0 + g * ns + in_segment_before(x, w0 + g * seg_w, ns);
  }
};

// Dynamic LDS of a decode workgroup: the step and weight prefixes (2 x (S+1) int64), the
// per-wavefront partial sums (16 int64) and the clamped lengths (S int32).
__host__ __device__ inline size_t decode_lds_bytes(int num_seqs) {
  return (2 * ((size_t)num_seqs + 1) + 16) * sizeof(int64_t) + (size_t)num_seqs * sizeof(int32_t);
}

// Start of whatever a kernel keeps in dynamic LDS after the schedule arrays (16-byte aligned).
__host__ __device__ inline size_t ring_offset(int num_seqs) {
  return (decode_lds_bytes(num_seqs) + 15) & ~(size_t)15;
}

// Store the clamped lengths (all threads of the workgroup call it; build_prefixes' barriers
// order it before any use).
__device__ inline void stage_lengths(const int32_t* lens, int S, int cap, int32_t* sm_len) {
  for (int i = threadIdx.x; i < S; i += blockDim.x) sm_len[i] = clamp_len(lens[i], cap);
}

// Uniform description of one step of a worker's stream.
struct StepInfo {
  int s, g, k, ns, L, b0, b1;
  int gp;           // the pool KV head of schedule head g (g / kv_split)
  int range;        // the worker (its partial slots are 2*range, 2*range+1)
  bool rfirst;      // first step of the worker's range
  bool rlast;       // last step of the worker's range
  bool past;        // described past the end of the range (its loads are never used)
};

// Wave-uniform position in the step line: segment (s, g), step k of ns, sequence length L;
// g = gp * kv_split + gc, gp the pool KV head.
struct Cursor {
  int s, g, k, ns, L, gp, gc;
};

__device__ inline Cursor cursor_at(const int64_t* sm_prefix, const int32_t* sm_len, int S,
                                   int Hkv, int ks, int64_t r) {
  Cursor c;
  c.s = find_seq(sm_prefix, S, Hkv, r);
  const int64_t p0 = uni(sm_prefix[c.s]);
  const int64_t rem = r - (int64_t)Hkv * p0;
  c.ns = (int)(uni(sm_prefix[c.s + 1]) - p0);
  c.g = (int)(rem / c.ns);
  c.k = (int)(rem - (int64_t)c.g * c.ns);
  c.L = uni(sm_len[c.s]);
  c.gp = c.g / ks;
  c.gc = c.g - c.gp * ks;
  return c;
}

// Next step of the line (the caller knows one exists; the walk stops at the last sequence
// regardless, so that a broken caller cannot loop or leave the prefix array).
__device__ inline void cursor_next(Cursor& c, const int64_t* sm_prefix, const int32_t* sm_len,
                                   int S, int Hkv, int ks) {
  if (++c.k < c.ns) return;
  c.k = 0;
  if (++c.g < Hkv) {
    if (++c.gc == ks) {
      c.gc = 0;
      ++c.gp;
    }
    return;
  }
  c.g = 0;
  c.gp = 0;
  c.gc = 0;
  do {
    ++c.s;
    c.ns = (int)(uni(sm_prefix[c.s + 1]) - uni(sm_prefix[c.s]));
  } while (c.ns == 0 && c.s < S - 1);
  c.L = uni(sm_len[c.s]);
}

// Physical block ids come from the caller's table; anything outside [0, num_blocks) is read as
// block 0 and poisons the row.
__device__ __forceinline__ bool valid_block(int b, int num_blocks) {
  return (unsigned)b < (unsigned)num_blocks;
}

// Describes the steps of one worker's range [b0, end) in order. next() returns the current
// step's description -- with its physical block ids fetched by scalar loads from the table row
// (raw: they are checked where they are used, so the loads' latency is hidden) -- and moves the
// cursor on; past the end of the range it keeps describing the last step, flagged `past` (the
// kernels point such a step's key/value loads at cached lines). A step whose tokens all sit in
// its first block (block size 16) gets that block for its second half too.
template <int B>
struct StepStream {
  const int64_t* sm_prefix;
  const int32_t* sm_len;
  ctable_t tables;
  int S, Hkv, ks, max_blocks, num_blocks, w;   // ks: schedule KV heads per pool KV head
  int64_t b0, end, j;   // the range and the line index of the next step to describe
  Cursor c;             // position of step j

  __device__ void init(int64_t range_b0, int64_t range_end) {
    b0 = range_b0;
    end = range_end;
    j = b0;
    if (j < end) c = cursor_at(sm_prefix, sm_len, S, Hkv, ks, j);
  }

  __device__ StepInfo next() {
    StepInfo si;
    si.s = c.s;
    si.g = c.g;
    si.gp = c.gp;
    si.k = c.k;
    si.ns = c.ns;
    si.L = c.L;
    const ctable_t row = tables + (size_t)c.s * max_blocks;
    const int jb0 = B == 16 ? 2 * c.k : c.k;
    si.b0 = row[jb0];
    if (B == 16) {
      const int jb1 = jb0 + 1 < ceil_div(c.L, B) ? jb0 + 1 : jb0;
      si.b1 = row[jb1];
    } else {
      si.b1 = si.b0;
    }
    si.range = w;
    si.rfirst = j == b0;
    si.rlast = j == end - 1;
    si.past = j >= end;
    ++j;
    if (j < end) cursor_next(c, sm_prefix, sm_len, S, Hkv, ks);
    return si;
  }
};

// Partial slot of the piece that starts at this step: the first piece of a worker's range uses
// slot 2*w, the last one (when it is not also the first) 2*w + 1.
__device__ __forceinline__ size_t piece_slot(int w, bool starts_range) {
  return 2 * (size_t)w + (starts_range ? 0 : 1);
}

}  // namespace pkv
