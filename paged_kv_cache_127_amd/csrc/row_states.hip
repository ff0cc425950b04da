// Softmax states of many query rows over the tokens of one block list, on the matrix cores.
// Two users:
//
// Shared-prefix decode. Sequences that begin with the same whole blocks ("PagedAttention:
// Virtual Memory for the KV Cache", section "Sharing a prefix and copying a partial block":
// sharers' tables point at the same physical blocks) need those blocks' keys and values only
// once per step. The softmax state over a token range merges with the state over the rest by
// the log-sum-exp rule ("Paged Attention and vLLM", section "Paged Attention CUDA Kernel"), so
// the work splits exactly: the states of the S * G query rows of every KV head over the prefix
// (here); the decode kernel over each sequence's own suffix, writing normalised rows with their
// log-sum-exp or partial states; the merge kernel, which folds every row's suffix state with
// its prefix states.
//
// Extend (multi-query) attention. The new tokens of a sequence -- a prefill chunk past a
// cached prefix, or speculated tokens to verify ("KV Cache Optimization and Management",
// section "RadixAttention: caching, not just packing, the prefix": only the tokens past the
// shared part need a fresh prefill pass) -- are already stored; new token t of n attends to
// positions 0 .. L - n + t of its sequence (causal). Its n * G rows of a KV head attend to the
// sequence's own blocks with a per-row token limit. With one chunk group a workgroup's merged
// state is its rows' whole softmax and is normalised into the output right here; with several,
// extend_finish folds each row's states and normalises. Runs long enough to give 128 or more rows
// per KV head (prefill chunks) take extend_rows_shared below, whose workgroups share each step's
// keys and values among four row tiles; row_states serves the short runs (speculative
// verification), whose four wavefronts split one row tile's tokens. Prefixes past 4096 tokens
// take extend_rows_shared's prefix mode.
//
// row_states. A workgroup of four wavefronts takes (row group of RB * 16 rows of one KV head,
// chunk group); wavefront w runs chunk 4 * cg + w, a run of 32-token steps. Per step the MFMA
// operands are laid out as in the decode kernel: key rows tau(a, i) = 8 * (i / 4) + 4a + i % 4
// as the A operand, so that the scores S^T[token][row] come out with lane l holding row l % 16
// and tokens 8 * (l / 16) + 4a + e -- the B-operand layout of the P.V product; value rows pass
// through the wavefront's swizzled LDS tile and come back transposed as the A operand of
// O^T[d][row] += V^T . P^T, with P split into a 16-bit high part and a remainder. Each
// key/value fragment a wavefront loads serves its RB row blocks; two wavefronts per SIMD, so
// that one computes while the other waits for memory. Block ids are scalar loads three steps
// ahead, keys one step ahead, values two (one step in registers, one in LDS). At the end the
// four wavefronts merge their states through LDS (over the value tiles, no longer needed), each
// folding and storing a quarter of the columns: one state (m, l, acc) per row and chunk group,
// m in the log2 domain, acc not normalised (or, extend mode with one chunk group, the
// normalised rows). In prefix mode the first workgroup also writes the suffix lengths
// max(L_s - P, 0).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "mfma_common.h"
#include "schedule.h"

namespace pkv {

constexpr int kRowsRB = 2;            // 16-row blocks per wavefront
constexpr int kRowWaves = 4;          // chunks per workgroup
constexpr int kMaxStepsPerWave = 32;  // planned 32-token steps of one wavefront
constexpr int kMaxChunkGroups = 16;   // states per row
constexpr int kMinExtendSteps = 8;    // extend mode: fewest 32-token steps a wavefront is given
constexpr int kWideRows = 32 * kRowWaves;   // rows of an extend_rows_shared workgroup

// Lazy softmax reference: the exponents of a row use its running reference m unless a step's
// maximum exceeds m by more than this (log2 domain), so probabilities stay below 2^8 -- harmless
// in fp32 and in the 16-bit split -- and the accumulators are rescaled only on those rare steps.
constexpr float kLazyRescale = 8.f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 probabilities as packed 16-bit high parts and remainders. bf16: the high part is the
// fp32 value truncated to its upper half (one AND each, packed by one byte permute), so the
// remainder p - hi is exact and is rounded once (both remainders by one packed conversion);
// |hi + lo - p| <= 2^-17 p. fp16 keeps the rounding split.
template <typename T>
__device__ __forceinline__ void split_hi_lo(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  if constexpr (__is_same(T, bf16_t)) {
    const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u;
    const uint32_t u1 = __float_as_uint(p1) & 0xffff0000u;
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // u0's upper half low, u1's high
    const f32x2_t r = f32x2_t{p0 - __uint_as_float(u0), p1 - __uint_as_float(u1)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
  } else {
    split_pair<T>(p0, p1, hi, lo);
  }
}

// Max over the lanes that differ in lane bits 4 and 5 (the four 16-lane rows of the wavefront),
// with the gfx950 lane-swap instructions: v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second, v_permlane32_swap the upper half of the first with
// the lower half of the second; given the same value twice, each returns every lane's value and
// that of its partner row (half). No LDS round trip, unlike a shuffle through ds_bpermute.
__device__ __forceinline__ float rows_max(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Four normalised output values (x * s) at element `off` of the output rows, fp32 or the
// cache's 16-bit type (rounded once from the fp32 product).
template <typename T>
__device__ __forceinline__ void store_row4(const RowStateParams& p, size_t off, f32x4 x, float s) {
  if (p.out_f32) {
    store_nt(reinterpret_cast<float*>(p.out) + off, x * s);
  } else {
    const uint32_t w0 =
        (uint32_t)scaled_to_16<T>(x[0], s) | ((uint32_t)scaled_to_16<T>(x[1], s) << 16);
    const uint32_t w1 =
        (uint32_t)scaled_to_16<T>(x[2], s) | ((uint32_t)scaled_to_16<T>(x[3], s) << 16);
    store_nt(reinterpret_cast<uint16_t*>(p.out) + off, u32x2{w0, w1});
  }
}

template <typename T, int D, int B, int RBK, bool NT>
__global__ __launch_bounds__(64 * kRowWaves) __attribute__((amdgpu_waves_per_eu(2)))
void row_states(RowStateParams p) {
  static_assert(B == 16 || B == 32, "block size");
  constexpr int NC = D / 32;
  constexpr int NF = D / 16;
  constexpr int ES = 2;
  constexpr int ROWB = D * ES;           // bytes per key / value row
  constexpr int VLPR = D / 8;            // lanes per value row (16 bytes each)
  constexpr int VTPI = 64 / VLPR;        // value rows per load instruction
  constexpr int TILE = 32 * ROWB;        // value tile per wavefront
  // value tiles during the steps; afterwards the four wavefronts' states for the merge
  constexpr int STATE = RBK * NF * 64 * 16;
  constexpr int LDS = TILE > STATE ? kRowWaves * TILE : kRowWaves * STATE;
  static_assert(NF % kRowWaves == 0, "column tiles per merging wavefront");
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  __shared__ float lds_ml[kRowWaves][2][RBK][64];

  const int lane = threadIdx.x & 63;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int jg = lane >> 4;
  const int S = p.num_seqs, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const bool extend = p.query_start != nullptr;   // uniform
  const int cgroups = p.chunk_groups;
  const int cg = blockIdx.x % cgroups;
  int g, rg, R, tok_end, qs = 0, n = 0, L = 0;
  ctable_t blocks;
  if (!extend) {
    // prefix mode: rows r = s * G + i of all S sequences, the shared blocks, P tokens for all
    const int P = p.prefix_len;
    if (blockIdx.x == 0)
      for (int s = threadIdx.x; s < S; s += blockDim.x)
        p.suffix_lens[s] = max(p.lens[s] - P, 0);
    R = S * G;
    const int groups = ceil_div(R, 16 * RBK);
    rg = (blockIdx.x / cgroups) % groups;
    g = blockIdx.x / (cgroups * groups);           // grid = Hkv * groups * cgroups
    tok_end = P;
    blocks = (ctable_t)p.prefix_blocks;
  } else {
    // extend mode: rows r = t * G + i of sequence s's n new tokens, its own blocks, tokens up
    // to the group's last row's limit (grid = S * Hkv * max_row_groups * cgroups). Dispatch
    // order: chunk groups fastest, then KV heads, then the row groups from the last one down,
    // then the sequences longest first (rank by context length, ties by index, when at most
    // one per thread), so that the longest workgroups start first.
    const int mg = p.max_row_groups;
    g = (blockIdx.x / cgroups) % Hkv;
    rg = mg - 1 - (int)((blockIdx.x / (cgroups * Hkv)) % mg);
    const int rank = blockIdx.x / (cgroups * Hkv * mg);
    int s = rank;
    if (S > 1 && S <= 64 * kRowWaves) {
      __shared__ int ranked;
      int* sl = reinterpret_cast<int*>(lds);          // value tiles, not in use yet
      for (int j = threadIdx.x; j < S; j += blockDim.x) sl[j] = clamp_len(p.lens[j], p.max_blocks * B);
      __syncthreads();
      if ((int)threadIdx.x < S) {
        const int j = threadIdx.x, lj = sl[j];
        int r = 0;
        for (int i = 0; i < S; ++i) r += (sl[i] > lj || (sl[i] == lj && i < j)) ? 1 : 0;
        if (r == rank) ranked = j;
      }
      __syncthreads();
      s = uni(ranked);
    }
    // out-of-contract starts are clamped into [0, T]: rows are never read or written outside
    qs = min(max(p.query_start[s], 0), p.num_query_tokens);
    n = min(max(p.query_start[s + 1] - qs, 0), p.num_query_tokens - qs);
    L = clamp_len(p.lens[s], p.max_blocks * B);
    R = n * G;
    if (rg * 16 * RBK >= R) return;                // the whole workgroup: no barrier yet
    const int t_last = (min((rg + 1) * 16 * RBK, R) - 1) / G;
    tok_end = min(max(L - n + t_last + 1, 0), L);
    blocks = (ctable_t)p.tables + (size_t)s * p.max_blocks;
  }
  // this row group's steps, split evenly over the chunk groups' wavefronts. In extend mode a
  // wavefront gets at least kMinExtendSteps of them: every wavefront pays a fixed start (the
  // dependent loads of its sequence's limits, block ids, queries and first keys and values)
  // and end (the merge and the state stores), so a short sequence is better served by a few
  // wavefronts than by short chunks on all of them; the others are left empty.
  const int nsteps = ceil_div(tok_end, 32);
  const int chunk = cg * kRowWaves + wave;
  int spc = ceil_div(nsteps, cgroups * kRowWaves);
  if (extend) spc = max(spc, kMinExtendSteps);
  const int k0 = min(chunk * spc, nsteps);
  const int k1 = min(k0 + spc, nsteps);
  const int nb = ceil_div(tok_end, B);             // blocks holding the tokens

  const char* kbase = reinterpret_cast<const char*>(p.k_pool);
  const char* vbase = reinterpret_cast<const char*>(p.v_pool);
  const size_t tile_stride = (size_t)B * D * ES;   // bytes per (block, head)
  const int tokA0 = 8 * (r16 >> 2) + (r16 & 3);
  const int kofs0 = ((tokA0 & (B - 1)) * D + 8 * jg) * ES;
  const int kofs1 = (((tokA0 + 4) & (B - 1)) * D + 8 * jg) * ES;
  const int vrow = lane / VLPR;
  const int vch = lane % VLPR;
  const int vtok = 8 * jg;

  // query rows of the RB row blocks (padding rows repeat the last row and are never stored),
  // each row's output / state index and its token limit
  size_t qrow[RBK];
  int lim[RBK];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const int r = min((rg * RBK + rb) * 16 + r16, R - 1);
    const int a = r / G;                           // sequence (prefix) or new token (extend)
    const int i = r - a * G;
    qrow[rb] = ((size_t)(extend ? qs + a : a)) * Hq + (size_t)g * G + i;
    lim[rb] = extend ? min(max(L - n + a + 1, 0), L) : tok_end;
  }

  // a workgroup none of whose chunks holds a step writes the empty state (-inf, 0, 0) of its
  // rows for this chunk group -- what the merge below would produce -- and leaves (uniform
  // over the workgroup, before any barrier)
  if (cg * kRowWaves * spc >= nsteps) {
    if (wave != 0) return;
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      const int r = (rg * RBK + rb) * 16 + r16;
      if (r >= R) continue;
      if (p.out) {                                 // nothing to attend: a zero row
#pragma unroll
        for (int f = 0; f < NF; ++f) store_row4<T>(p, qrow[rb] * D + 16 * f + 4 * jg,
                                                    f32x4{0.f, 0.f, 0.f, 0.f}, 0.f);
        continue;
      }
      const size_t row = (size_t)cg * p.state_rows + qrow[rb];
#pragma unroll
      for (int f = 0; f < NF; ++f)
        store_nt(p.st_acc + row * D + 16 * f + 4 * jg, f32x4{0.f, 0.f, 0.f, 0.f});
      if (jg == 0) {
        store_nt(p.st_m + row, kNegInf);
        store_nt(p.st_l + row, 0.f);
      }
    }
    return;
  }

  u32x4 q[RBK][NC];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const char* qp = reinterpret_cast<const char*>(p.q) + (qrow[rb] * D + 8 * jg) * ES;
#pragma unroll
    for (int c = 0; c < NC; ++c) q[rb][c] = load16(qp + 32 * c * ES);
  }

  char* vstage = lds + wave * TILE;
  int vw_ofs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int t = VTPI * f + vrow;
    vw_ofs[f] = t * ROWB + (((vch >> 1) ^ piece_swizzle<D>(t)) << 5) + 16 * (vch & 1);
  }
  int vr_ofs[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int t = 8 * jg + 4 * hh + (r16 >> 2);
    vr_ofs[hh] = t * ROWB + (piece_swizzle<D>(t) << 5) + 8 * (r16 & 3);
  }

  // the smallest token limit of the wavefront's rows: steps below it need no masking
  int lim_min = lim[0];
#pragma unroll
  for (int rb = 1; rb < RBK; ++rb) lim_min = min(lim_min, lim[rb]);
  lim_min = uni((int)-cross_max<1>(-(float)lim_min));

  float m_run[RBK], l_run[RBK];
  f32x4 oacc[RBK][NF];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[rb][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool poison = false;

  // physical blocks of step k (B = 16: two blocks; a second block past the prefix repeats the
  // first and its slots are masked); out-of-range ids read block 0 and poison the state
  // (scalar loads through the constant address space: their wait is not the vector-load
  // counter that the key/value loads in flight use; no branch, so that a step is one
  // scheduling region)
  auto step_blocks = [&](int k, int& b0, int& b1) {
    const int j0 = B == 16 ? 2 * k : k;
    b0 = blocks[j0];
    b1 = B == 16 ? blocks[min(j0 + 1, nb - 1)] : b0;
  };
  u32x4 kr[2][NC], vr[NF], va[NF];
  // NT: streaming loads, for key/value rows this launch reads once (extend mode with one row
  // group per sequence: the chunks split the tokens); shared prefix blocks, which every row
  // group reads, stay on plain loads so that they remain in the caches
  auto ld = [](const char* a) { return NT ? load16_stream(a) : load16(a); };
  auto load_k = [&](int b0, int b1) {
    b0 = valid_block(b0, p.num_blocks) ? b0 : 0;
    b1 = valid_block(b1, p.num_blocks) ? b1 : 0;
    const char* t0 = kbase + ((size_t)b0 * Hkv + g) * tile_stride;
    const char* t1 = kbase + ((size_t)b1 * Hkv + g) * tile_stride;
    const char* ka = ((B == 16 && tokA0 >= 16) ? t1 : t0) + kofs0;
    const char* kb = ((B == 16 && tokA0 + 4 >= 16) ? t1 : t0) + kofs1;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kr[0][c] = ld(ka + 32 * c * ES);
      kr[1][c] = ld(kb + 32 * c * ES);
    }
  };
  auto load_v = [&](int b0, int b1) {
    b0 = valid_block(b0, p.num_blocks) ? b0 : 0;
    b1 = valid_block(b1, p.num_blocks) ? b1 : 0;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int t = VTPI * f + vrow;
      const int blk = (B == 16 && t >= 16) ? b1 : b0;
      vr[f] = ld(vbase + ((size_t)blk * Hkv + g) * tile_stride + (size_t)(t & (B - 1)) * ROWB +
                 16 * vch);
    }
  };
  auto stage_v = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f) *reinterpret_cast<u32x4*>(vstage + vw_ofs[f]) = vr[f];
  };

  // Softmax of row block rb's scores z at step k against its reference m_ref: probabilities
  // as 16-bit high parts and remainders, their sum folded into l_run (l * alpha + sum).
  auto softmax = [&](const float (&z)[8], float m_ref, float alpha, float& l, u32x4& phi,
                     u32x4& plo) {
    float pr[8];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pr[t] = fast_exp2(fmaf(z[t], p.scale_log2, -m_ref));
      ps += pr[t];
    }
    l = l * alpha + ps;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t h, lo;
      split_hi_lo<T>(pr[2 * u], pr[2 * u + 1], h, lo);
      phi[u] = h;
      plo[u] = lo;
    }
  };
  auto pv = [&](int rb, const u32x4& phi, const u32x4& plo) {
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[rb][f] = mfma16x16x32<T>(va[f], phi, oacc[rb][f]);
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[rb][f] = mfma16x16x32<T>(va[f], plo, oacc[rb][f]);
  };

  // Step k: the transposed reads of the step's value tile (written to LDS during the previous
  // step) and the score MFMAs, the next step's key loads; the row maxima (a rare branch
  // rescales the accumulators when a reference moves); the softmax and P.V products of each
  // row block; the next step's value rows to LDS and the loads of the values of the step after
  // it. Keys are loaded one step ahead, values two (one step in registers, one in LDS), block
  // ids three (the scalar loads). (Scheduling hints that interleave the MFMAs with the softmax
  // and the LDS writes gave no measurable gain and made the block-size-32 loop spill.)
  if (k0 < k1) {
    const int kl = k1 - 1;
    int b0, b1, n0, n1, nn0, nn1;
    step_blocks(k0, b0, b1);
    load_k(b0, b1);
    load_v(b0, b1);
    step_blocks(min(k0 + 1, kl), n0, n1);
    step_blocks(min(k0 + 2, kl), nn0, nn1);
    stage_v();
    load_v(n0, n1);
#pragma unroll 1
    for (int k = k0; k < k1; ++k) {
      const int nvalid = min(32, tok_end - 32 * k);
      poison = poison || !valid_block(b0, p.num_blocks) || !valid_block(b1, p.num_blocks);
      int n30, n31;
      step_blocks(min(k + 3, kl), n30, n31);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const uint2 lo = lds_read_tr16(vstage + (vr_ofs[0] ^ (f << 5)));
        const uint2 hi = lds_read_tr16(vstage + (vr_ofs[1] ^ (f << 5)));
        va[f] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      f32x4 sacc[RBK][2];
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          sacc[rb][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NC; ++c) sacc[rb][a] = mfma16x16x32<T>(kr[a][c], q[rb][c], sacc[rb][a]);
        }
      load_k(n0, n1);

      // raw scores; masked tokens -inf (the scale is positive, so the row maximum of the
      // raw scores, scaled, is the maximum of the scaled ones)
      float z[RBK][8];
      if (32 * k + 32 <= lim_min) {   // every token of the step counts for every row
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) z[rb][4 * a + e] = sacc[rb][a][e];
      } else {
        if (nvalid < 32) {   // value rows past the end: zero, so that 0 * garbage cannot appear
          const int nv = nvalid - vtok;
          u32x4 msk;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            msk[u] = (2 * u < nv ? 0xffffu : 0u) | (2 * u + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
          for (int f = 0; f < NF; ++f) va[f] &= msk;
        }
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int tok = vtok + 4 * a + e;
              z[rb][4 * a + e] =
                  (tok < nvalid && 32 * k + tok < lim[rb]) ? sacc[rb][a][e] : kNegInf;
            }
      }
      float m_ref[RBK], alpha[RBK];
      bool upd_any = false;
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb) {
        float mx = z[rb][0];
#pragma unroll
        for (int t = 1; t < 8; ++t) mx = fmaxf(mx, z[rb][t]);
        const float m_step = rows_max(mx) * p.scale_log2;
        // the reference moves only when this step's maximum exceeds it by more than
        // kLazyRescale (a first finite maximum always moves it); otherwise alpha is exactly 1
        const bool upd = m_step > m_run[rb] + kLazyRescale;
        const float m_new = upd ? m_step : m_run[rb];
        // a row with nothing to attend yet (causal limit) keeps (-inf, 0, 0): exponents
        // against 0 instead of -inf, so that no -inf - -inf appears
        m_ref[rb] = m_new == kNegInf ? 0.f : m_new;
        alpha[rb] = fast_exp2(m_run[rb] - m_ref[rb]);
        m_run[rb] = m_new;
        upd_any = upd_any || upd;
      }
      if (__builtin_amdgcn_ballot_w64(upd_any) != 0) {
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
          for (int f = 0; f < NF; ++f) oacc[rb][f] *= alpha[rb];
      }

      // (LDS operations of one wavefront complete in order, and the compiler keeps a store
      // after the loads of the same tile that precede it: no fence is needed between this
      // step's transposed reads, the next step's value rows written below and their reads at
      // the top of the next step)
      u32x4 phi[RBK], plo[RBK];
      softmax(z[0], m_ref[0], alpha[0], l_run[0], phi[0], plo[0]);
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb) {
        if (rb + 1 < RBK)
          softmax(z[rb + 1], m_ref[rb + 1], alpha[rb + 1], l_run[rb + 1], phi[rb + 1], plo[rb + 1]);
        if (rb + 1 == RBK) {
          stage_v();            // the next step's values to LDS
          load_v(nn0, nn1);     // the values of the step after it
        }
        pv(rb, phi[rb], plo[rb]);
      }
      b0 = n0;
      b1 = n1;
      n0 = nn0;
      n1 = nn1;
      nn0 = n30;
      nn1 = n31;
    }
  }
  float l_tot[RBK];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    l_tot[rb] = cross_sum<16>(l_run[rb]);
    if (poison) l_tot[rb] = __builtin_nanf("");
  }

  // Merge the four wavefronts' states: each leaves its (m, l, acc) in LDS (the same lane ->
  // (row, column) mapping in every wavefront), one barrier, then wavefront w folds the four
  // states of column tiles w, w + 4, ... and stores them; wavefront 0 also stores m and l.
  f32x4* mrg = reinterpret_cast<f32x4*>(lds);
  __syncthreads();   // every wavefront is done with its value tile
  {
    f32x4* dst = mrg + (size_t)wave * RBK * NF * 64;
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
#pragma unroll
      for (int f = 0; f < NF; ++f) dst[(rb * NF + f) * 64 + lane] = oacc[rb][f];
      lds_ml[wave][0][rb][lane] = m_run[rb];
      lds_ml[wave][1][rb][lane] = l_tot[rb];
    }
  }
  __syncthreads();

  // state of chunk group cg: st_m / st_l [cgroups][state_rows], st_acc [..][state_rows][D]
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    float mw[kRowWaves];
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      mw[w] = lds_ml[w][0][rb][lane];
      mx = fmaxf(mx, mw[w]);
    }
    float wgt[kRowWaves];
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      wgt[w] = mx == kNegInf ? 0.f : fast_exp2(mw[w] - mx);
      lsum += lds_ml[w][1][rb][lane] * wgt[w];
    }
    const int r = (rg * RBK + rb) * 16 + r16;
    if (r >= R) continue;
    const size_t row = (size_t)cg * p.state_rows + qrow[rb];
    // one chunk group: this state is the row's whole softmax, normalised here exactly as the
    // finish kernel would (weight 1, den = l; 0 for a row with nothing to attend)
    const float sc = (mx == kNegInf || lsum == 0.f) ? 0.f : 1.0f / lsum;
#pragma unroll
    for (int j = 0; j < NF / kRowWaves; ++j) {
      const int f = wave + kRowWaves * j;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w)
        acc += mrg[((size_t)w * RBK * NF + rb * NF + f) * 64 + lane] * wgt[w];
      if (p.out) store_row4<T>(p, qrow[rb] * D + 16 * f + 4 * jg, acc, sc);
      else store_nt(p.st_acc + row * D + 16 * f + 4 * jg, acc);
    }
    if (!p.out && wave == 0 && jg == 0) {
      store_nt(p.st_m + row, mx);
      store_nt(p.st_l + row, lsum);
    }
  }
}

// extend_rows_shared: extend attention for long runs of new tokens (a prefill chunk), where one
// sequence's (new token, head) rows of a KV head number at least kWideRows. The four wavefronts
// of a workgroup take four different 32-row tiles (rows rg * 128 + 32 * wave + 16 * rb + r16)
// over the same 32-token steps, and each step's key and value rows are loaded once for the
// workgroup -- every thread loads its share -- and shared through LDS: per step and wavefront
// 4 KB (d = 128) go through the CU's vector memory path instead of the 16 KB that row_states
// loads for its own chunk. Two LDS stages of (keys, values): while the wavefronts read step k's
// tile they write step k + 1's, loaded during step k - 1, into the other stage and load step
// k + 2; one workgroup barrier per step separates a stage's writes from its reads. Keys are read
// from LDS as the score MFMA's A operand (rows tau(a, i) as in row_states), values as in
// row_states. The workgroup's token range ends at its last row's limit and is split evenly over
// the chunk groups; with one chunk group each wavefront normalises its rows into the output,
// otherwise it stores their states for extend_finish. The same kernel computes the prefix
// states of long shared prefixes (prefix mode, as in row_states: the S * G rows of a KV head
// against all P prefix tokens, one state per row and chunk group for the decode's merge).
template <typename T, int D, int B>
__global__ __launch_bounds__(64 * kRowWaves) __attribute__((amdgpu_waves_per_eu(2)))
void extend_rows_shared(RowStateParams p) {
  static_assert(B == 16 || B == 32, "block size");
  constexpr int RBK = kRowsRB;
  constexpr int NC = D / 32;
  constexpr int NF = D / 16;
  constexpr int ES = 2;
  constexpr int ROWB = D * ES;                          // bytes per key / value row
  constexpr int CPR = ROWB / 16;                        // 16-byte pieces per row
  constexpr int TILE = 32 * ROWB;                       // one step's keys (or values)
  constexpr int NT = 64 * kRowWaves;                    // threads
  constexpr int NLD = 2 * 32 * CPR / NT;                // pieces per thread per step
  constexpr int NLK = 32 * CPR / NT;                    // ... of them keys
  static_assert(NLD * NT == 2 * 32 * CPR && NLK * NT == 32 * CPR, "load split");
  __shared__ __attribute__((aligned(16))) char lds[2][2][TILE];   // [stage][keys, values]

  const int lane = threadIdx.x & 63;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int r16 = lane & 15;
  const int jg = lane >> 4;
  const int S = p.num_seqs, Hq = p.num_q_heads, Hkv = p.num_kv_heads;
  const int G = Hq / Hkv;
  const int cgroups = p.chunk_groups;
  const bool extend = p.query_start != nullptr;         // uniform
  int cg, g, rg, qs = 0, n = 0, L = 0, R, tok_end;
  ctable_t blocks;
  if (!extend) {
    // prefix mode: rows r = s * G + i of all S sequences, the shared blocks, P tokens for all
    // rows (grid = Hkv * wide row groups * cgroups). Dispatch order: KV heads fastest (with 8
    // heads each XCD streams one head's prefix through its L2), then chunk groups, then row
    // groups. The suffix lengths max(L_s - P, 0) are written one per thread over the grid.
    const int P = p.prefix_len;
    for (int j = blockIdx.x + (int)(gridDim.x * threadIdx.x); j < S;
         j += (int)(gridDim.x * blockDim.x))
      p.suffix_lens[j] = max(p.lens[j] - P, 0);
    g = blockIdx.x % Hkv;
    cg = (blockIdx.x / Hkv) % cgroups;
    rg = blockIdx.x / (Hkv * cgroups);
    R = S * G;
    tok_end = P;
    blocks = (ctable_t)p.prefix_blocks;
  } else {
    // extend mode (grid = S * Hkv * mg * cgroups). Dispatch order: chunk groups fastest, then
    // KV heads (with 8 heads each XCD keeps one head's keys and values), then the row groups
    // from the last one (the longest token range) down, then the sequences longest first --
    // their rank by context length, ties by index, when at most one per thread -- so that the
    // longest workgroups start first and the short ones fill in at the end.
    const int mg = p.max_row_groups;
    cg = blockIdx.x % cgroups;
    g = (blockIdx.x / cgroups) % Hkv;
    rg = mg - 1 - (int)((blockIdx.x / (cgroups * Hkv)) % mg);
    const int rank = blockIdx.x / (cgroups * Hkv * mg);
    int s = rank;
    if (S > 1 && S <= NT) {
      __shared__ int ranked;
      int* sl = reinterpret_cast<int*>(&lds[0][0][0]);   // stage memory, not in use yet
      for (int j = threadIdx.x; j < S; j += NT) sl[j] = clamp_len(p.lens[j], p.max_blocks * B);
      __syncthreads();
      if ((int)threadIdx.x < S) {
        const int j = threadIdx.x, lj = sl[j];
        int r = 0;
        for (int i = 0; i < S; ++i) r += (sl[i] > lj || (sl[i] == lj && i < j)) ? 1 : 0;
        if (r == rank) ranked = j;
      }
      __syncthreads();
      s = uni(ranked);
    }
    // out-of-contract starts are clamped into [0, T]: rows are never read or written outside
    qs = uni(min(max(p.query_start[s], 0), p.num_query_tokens));
    n = uni(min(max(p.query_start[s + 1] - qs, 0), p.num_query_tokens - qs));
    L = uni(clamp_len(p.lens[s], p.max_blocks * B));
    R = n * G;
    if (rg * kWideRows >= R) return;                    // the whole workgroup: no barrier yet
    const int t_last = (min((rg + 1) * kWideRows, R) - 1) / G;
    tok_end = min(max(L - n + t_last + 1, 0), L);
    blocks = (ctable_t)p.tables + (size_t)s * p.max_blocks;
  }
  const int nsteps = ceil_div(tok_end, 32);
  const int spc = ceil_div(nsteps, cgroups);
  const int k0 = min(cg * spc, nsteps);
  const int k1 = min(k0 + spc, nsteps);
  const int nb = ceil_div(tok_end, B);                  // blocks holding the tokens

  // this wavefront's rows (padding rows repeat the last row and are never stored)
  size_t qrow[RBK];
  int lim[RBK];
  bool live[RBK];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const int r0 = rg * kWideRows + 32 * wave + 16 * rb + r16;
    live[rb] = r0 < R;
    const int r = min(r0, R - 1);
    const int a = r / G;                                 // sequence (prefix) or new token
    const int i = r - a * G;
    qrow[rb] = ((size_t)(qs + a)) * Hq + (size_t)g * G + i;
    lim[rb] = extend ? min(max(L - n + a + 1, 0), L) : tok_end;
  }

  // a chunk group with no step (or nothing to attend) writes the empty state (-inf, 0, 0) of
  // its rows -- for the output, a zero row -- and leaves (uniform over the workgroup)
  if (k0 >= k1) {
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      if (!live[rb]) continue;
      if (p.out) {
#pragma unroll
        for (int f = 0; f < NF; ++f) store_row4<T>(p, qrow[rb] * D + 16 * f + 4 * jg,
                                                    f32x4{0.f, 0.f, 0.f, 0.f}, 0.f);
        continue;
      }
      const size_t row = (size_t)cg * p.state_rows + qrow[rb];
#pragma unroll
      for (int f = 0; f < NF; ++f)
        store_nt(p.st_acc + row * D + 16 * f + 4 * jg, f32x4{0.f, 0.f, 0.f, 0.f});
      if (jg == 0) {
        store_nt(p.st_m + row, kNegInf);
        store_nt(p.st_l + row, 0.f);
      }
    }
    return;
  }

  u32x4 q[RBK][NC];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    const char* qp = reinterpret_cast<const char*>(p.q) + (qrow[rb] * D + 8 * jg) * ES;
#pragma unroll
    for (int c = 0; c < NC; ++c) q[rb][c] = load16(qp + 32 * c * ES);
  }

  // this thread's share of a step's rows: piece u = j * NT + tid of the keys (j < NLK) or the
  // values -- row t, piece c, from the first or second block of the step (B = 16) -- and its
  // place in the stage
  const char* kbase = reinterpret_cast<const char*>(p.k_pool);
  const char* vbase = reinterpret_cast<const char*>(p.v_pool);
  const size_t tile_stride = (size_t)B * D * ES;       // bytes per (block, head)
  int gofs[NLD], wofs[NLD];
  bool second[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int u = (j % NLK) * NT + (int)threadIdx.x;
    const int t = u / CPR, c = u % CPR;
    second[j] = B == 16 && t >= 16;
    gofs[j] = (t & (B - 1)) * ROWB + 16 * c;
    wofs[j] = j < NLK ? t * ROWB + (key_piece<D>(t, c) << 4)
                      : TILE + t * ROWB + (((c >> 1) ^ piece_swizzle<D>(t)) << 5) + 16 * (c & 1);
  }
  // score-operand reads: key row tau(a, r16) = 8 * (r16 / 4) + 4a + r16 % 4, pieces jg + 4c
  int kro[2][NC];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int t = 8 * (r16 >> 2) + 4 * a + (r16 & 3);
#pragma unroll
    for (int c = 0; c < NC; ++c) kro[a][c] = t * ROWB + (key_piece<D>(t, jg + 4 * c) << 4);
  }
  int vr_ofs[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int t = 8 * jg + 4 * hh + (r16 >> 2);
    vr_ofs[hh] = TILE + t * ROWB + (piece_swizzle<D>(t) << 5) + 8 * (r16 & 3);
  }
  const int vtok = 8 * jg;

  int lim_min = lim[0];
#pragma unroll
  for (int rb = 1; rb < RBK; ++rb) lim_min = min(lim_min, lim[rb]);
  lim_min = uni((int)-cross_max<1>(-(float)lim_min));

  float m_run[RBK], l_run[RBK];
  f32x4 oacc[RBK][NF];
#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[rb][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool poison = false;

  // physical blocks of step k, as in row_states (scalar loads, no branch)
  auto step_blocks = [&](int k, int& b0, int& b1) {
    const int j0 = B == 16 ? 2 * k : k;
    b0 = blocks[j0];
    b1 = B == 16 ? blocks[min(j0 + 1, nb - 1)] : b0;
  };
  u32x4 ld[NLD];
  auto load_step = [&](int b0, int b1) {
    b0 = valid_block(b0, p.num_blocks) ? b0 : 0;
    b1 = valid_block(b1, p.num_blocks) ? b1 : 0;
    const size_t o0 = ((size_t)b0 * Hkv + g) * tile_stride;
    const size_t o1 = ((size_t)b1 * Hkv + g) * tile_stride;
#pragma unroll
    for (int j = 0; j < NLD; ++j)
      ld[j] = load16((j < NLK ? kbase : vbase) + (second[j] ? o1 : o0) + gofs[j]);
  };
  auto write_step = [&](char* stage) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) *reinterpret_cast<u32x4*>(stage + wofs[j]) = ld[j];
  };

  const int kl = k1 - 1;
  int b0, b1, n0, n1, nn0, nn1;
  step_blocks(k0, b0, b1);
  load_step(b0, b1);
  write_step(&lds[0][0][0]);
  step_blocks(min(k0 + 1, kl), n0, n1);
  load_step(n0, n1);
  step_blocks(min(k0 + 2, kl), nn0, nn1);
  __syncthreads();
#pragma unroll 1
  for (int k = k0; k < k1; ++k) {
    const int sti = (k - k0) & 1;
    const char* stage = &lds[sti][0][0];
    const int nvalid = min(32, tok_end - 32 * k);
    poison = poison || !valid_block(b0, p.num_blocks) || !valid_block(b1, p.num_blocks);
    int n30, n31;
    step_blocks(min(k + 3, kl), n30, n31);
    u32x4 kr[2][NC], va[NF];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[a][c] = *reinterpret_cast<const u32x4*>(stage + kro[a][c]);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint2 lo = lds_read_tr16(stage + (vr_ofs[0] ^ (f << 5)));
      const uint2 hi = lds_read_tr16(stage + (vr_ofs[1] ^ (f << 5)));
      va[f] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    f32x4 sacc[RBK][2];
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        sacc[rb][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc[rb][a] = mfma16x16x32<T>(kr[a][c], q[rb][c], sacc[rb][a]);
      }

    // raw scores; masked tokens -inf
    float z[RBK][8];
    if (32 * k + 32 <= lim_min) {
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) z[rb][4 * a + e] = sacc[rb][a][e];
    } else {
      if (nvalid < 32) {   // value rows past the end: zero, so that 0 * garbage cannot appear
        const int nv = nvalid - vtok;
        u32x4 msk;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          msk[u] = (2 * u < nv ? 0xffffu : 0u) | (2 * u + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
        for (int f = 0; f < NF; ++f) va[f] &= msk;
      }
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = vtok + 4 * a + e;
            z[rb][4 * a + e] =
                (tok < nvalid && 32 * k + tok < lim[rb]) ? sacc[rb][a][e] : kNegInf;
          }
    }
    float m_ref[RBK], alpha[RBK];
    bool upd_any = false;
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      float mx = z[rb][0];
#pragma unroll
      for (int t = 1; t < 8; ++t) mx = fmaxf(mx, z[rb][t]);
      const float m_step = rows_max(mx) * p.scale_log2;
      const bool upd = m_step > m_run[rb] + kLazyRescale;
      const float m_new = upd ? m_step : m_run[rb];
      m_ref[rb] = m_new == kNegInf ? 0.f : m_new;
      alpha[rb] = fast_exp2(m_run[rb] - m_ref[rb]);
      m_run[rb] = m_new;
      upd_any = upd_any || upd;
    }
    if (__builtin_amdgcn_ballot_w64(upd_any) != 0) {
#pragma unroll
      for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
        for (int f = 0; f < NF; ++f) oacc[rb][f] *= alpha[rb];
    }
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) {
      float pr[8];
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        pr[t] = fast_exp2(fmaf(z[rb][t], p.scale_log2, -m_ref[rb]));
        ps += pr[t];
      }
      l_run[rb] = l_run[rb] * alpha[rb] + ps;
      u32x4 phi, plo;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t h, lo;
        split_hi_lo<T>(pr[2 * u], pr[2 * u + 1], h, lo);
        phi[u] = h;
        plo[u] = lo;
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) oacc[rb][f] = mfma16x16x32<T>(va[f], phi, oacc[rb][f]);
#pragma unroll
      for (int f = 0; f < NF; ++f) oacc[rb][f] = mfma16x16x32<T>(va[f], plo, oacc[rb][f]);
    }
    // the next step's rows into the other stage (its reads ended before the last barrier),
    // then the loads of the step after it (past the end: the last step again)
    write_step(&lds[sti ^ 1][0][0]);
    load_step(nn0, nn1);
    __syncthreads();
    b0 = n0;
    b1 = n1;
    n0 = nn0;
    n1 = nn1;
    nn0 = n30;
    nn1 = n31;
  }

#pragma unroll
  for (int rb = 0; rb < RBK; ++rb) {
    float l_tot = cross_sum<16>(l_run[rb]);
    if (poison) l_tot = __builtin_nanf("");
    if (!live[rb]) continue;
    if (p.out) {
      // one chunk group: the row's whole softmax, normalised (0 for a row with nothing to attend)
      const float sc = (m_run[rb] == kNegInf || l_tot == 0.f) ? 0.f : 1.0f / l_tot;
#pragma unroll
      for (int f = 0; f < NF; ++f) store_row4<T>(p, qrow[rb] * D + 16 * f + 4 * jg, oacc[rb][f], sc);
    } else {
      const size_t row = (size_t)cg * p.state_rows + qrow[rb];
#pragma unroll
      for (int f = 0; f < NF; ++f) store_nt(p.st_acc + row * D + 16 * f + 4 * jg, oacc[rb][f]);
      if (jg == 0) {
        store_nt(p.st_m + row, m_run[rb]);
        store_nt(p.st_l + row, l_tot);
      }
    }
  }
}

// extend_finish: one thread per f32x4 chunk of the output rows; the row's states of every chunk
// group fold by the log-sum-exp rule and the sum is normalised. CM >= chunk_groups.
template <int D, typename T, int CM>
__global__ __launch_bounds__(256) void extend_finish(ExtendFinishParams p) {
  constexpr int Q = D / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= p.rows * Q) return;
  const size_t row = idx / Q;
  const size_t off = 4 * idx;                    // = row * D + 4 * (idx % Q)
  float m[CM], l[CM];
  f32x4 a[CM];
#pragma unroll
  for (int c = 0; c < CM; ++c) {
    if (c < p.chunk_groups) {
      m[c] = p.st_m[c * p.rows + row];
      l[c] = p.st_l[c * p.rows + row];
      a[c] = *reinterpret_cast<const f32x4*>(p.st_acc + c * p.rows * D + off);
    } else {
      m[c] = kNegInf;
      l[c] = 0.f;
      a[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int c = 0; c < CM; ++c) M = fmaxf(M, m[c]);
  f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int c = 0; c < CM; ++c) {
      const float w = fast_exp2(m[c] - M);
      num += a[c] * w;
      den += l[c] * w;
    }
  }
  const float sc = den == 0.f ? 0.f : 1.0f / den;
  if (p.out_f32) {
    store_nt(reinterpret_cast<float*>(p.out) + off, num * sc);
  } else {
    const uint32_t w0 = (uint32_t)scaled_to_16<T>(num[0], sc) |
                        ((uint32_t)scaled_to_16<T>(num[1], sc) << 16);
    const uint32_t w1 = (uint32_t)scaled_to_16<T>(num[2], sc) |
                        ((uint32_t)scaled_to_16<T>(num[3], sc) << 16);
    store_nt(reinterpret_cast<uint16_t*>(p.out) + off, u32x2{w0, w1});
  }
}

void row_state_plan(int64_t base_workgroups, int max_tokens, int num_cus, int* chunk_groups,
                    int* steps_per_chunk) {
  const int nsteps = (max_tokens + 31) / 32;
  // at least one workgroup per CU, at most kMaxStepsPerWave steps per wavefront, at most
  // kMaxChunkGroups states per row (each one more state for the merge to read)
  const int64_t base = std::max<int64_t>(base_workgroups, 1);
  const int64_t fill = (std::max(num_cus, 1) + base - 1) / base;
  const int64_t depth = (nsteps + kRowWaves * kMaxStepsPerWave - 1) /
                        (kRowWaves * kMaxStepsPerWave);
  const int64_t cg_max = std::max<int64_t>(
      1, std::min<int64_t>((nsteps + kRowWaves - 1) / kRowWaves, kMaxChunkGroups));
  const int64_t cg = std::max<int64_t>(1, std::min(std::max(fill, depth), cg_max));
  const int chunks = (int)cg * kRowWaves;
  *steps_per_chunk = std::max(1, (nsteps + chunks - 1) / chunks);
  *chunk_groups = (int)cg;
}

int64_t row_groups(int64_t rows) { return (rows + 16 * kRowsRB - 1) / (16 * kRowsRB); }

template <typename T, int D, int B>
static void launch_rows_tdb(const RowStateParams& p, int64_t grid, hipStream_t st) {
  if (p.query_start && p.max_row_groups == 1)
    launch_kernel((row_states<T, D, B, kRowsRB, true>), dim3((unsigned)grid),
                  dim3(64 * kRowWaves), 0, st, p);
  else
    launch_kernel((row_states<T, D, B, kRowsRB, false>), dim3((unsigned)grid),
                  dim3(64 * kRowWaves), 0, st, p);
}

template <typename T, int D>
static void launch_rows_td(const RowStateParams& p, int64_t grid, int block_size,
                           hipStream_t st) {
  if (block_size == 16) launch_rows_tdb<T, D, 16>(p, grid, st);
  else launch_rows_tdb<T, D, 32>(p, grid, st);
}

hipError_t launch_row_states(const RowStateParams& p, int kv_dtype, int head_dim,
                             int block_size, hipStream_t st) {
  if (p.num_seqs <= 0) return hipSuccess;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int64_t grid =
      p.query_start ? (int64_t)p.num_seqs * p.num_kv_heads * p.max_row_groups * p.chunk_groups
                    : (int64_t)p.num_kv_heads * row_groups((int64_t)p.num_seqs * G) *
                          p.chunk_groups;
  if (grid <= 0) return hipSuccess;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (kv_dtype == 2) {
    if (head_dim == 128) launch_rows_td<bf16_t, 128>(p, grid, block_size, st);
    else launch_rows_td<bf16_t, 64>(p, grid, block_size, st);
  } else if (kv_dtype == 1) {
    if (head_dim == 128) launch_rows_td<f16_t, 128>(p, grid, block_size, st);
    else launch_rows_td<f16_t, 64>(p, grid, block_size, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, typename T>
static void launch_finish_t(const ExtendFinishParams& p, hipStream_t st) {
  const int64_t chunks = (int64_t)p.rows * (D / 4);
  const dim3 grid((unsigned)((chunks + 255) / 256)), blk(256);
  const int C = p.chunk_groups;
  if (C <= 1) launch_kernel((extend_finish<D, T, 1>), grid, blk, 0, st, p);
  else if (C <= 2) launch_kernel((extend_finish<D, T, 2>), grid, blk, 0, st, p);
  else if (C <= 4) launch_kernel((extend_finish<D, T, 4>), grid, blk, 0, st, p);
  else if (C <= 8) launch_kernel((extend_finish<D, T, 8>), grid, blk, 0, st, p);
  else launch_kernel((extend_finish<D, T, 16>), grid, blk, 0, st, p);
}

template <typename T, int D>
static void launch_wide_td(const RowStateParams& p, int64_t grid, int block_size,
                           hipStream_t st) {
  if (block_size == 16)
    launch_kernel((extend_rows_shared<T, D, 16>), dim3((unsigned)grid), dim3(64 * kRowWaves), 0,
                  st, p);
  else
    launch_kernel((extend_rows_shared<T, D, 32>), dim3((unsigned)grid), dim3(64 * kRowWaves), 0,
                  st, p);
}

int64_t wide_row_groups(int64_t rows) { return (rows + kWideRows - 1) / kWideRows; }

void wide_row_plan(int64_t base_workgroups, int max_tokens, int num_cus, int* chunk_groups) {
  // one chunk group (the rows normalised in the kernel, no state round trip) whenever the
  // workgroups fill the CUs; otherwise enough groups to fill them, at most one per step and
  // at most kMaxChunkGroups
  const int64_t base = std::max<int64_t>(base_workgroups, 1);
  const int64_t nsteps = std::max((max_tokens + 31) / 32, 1);
  const int64_t fill = (std::max(num_cus, 1) + base - 1) / base;
  *chunk_groups = (int)std::max<int64_t>(
      1, std::min<int64_t>(fill, std::min<int64_t>(nsteps, kMaxChunkGroups)));
}

static hipError_t launch_wide(const RowStateParams& p, int64_t grid, int kv_dtype,
                              int head_dim, int block_size, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (kv_dtype == 2) {
    if (head_dim == 128) launch_wide_td<bf16_t, 128>(p, grid, block_size, st);
    else launch_wide_td<bf16_t, 64>(p, grid, block_size, st);
  } else if (kv_dtype == 1) {
    if (head_dim == 128) launch_wide_td<f16_t, 128>(p, grid, block_size, st);
    else launch_wide_td<f16_t, 64>(p, grid, block_size, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_extend_rows_shared(const RowStateParams& p, int kv_dtype, int head_dim,
                                     int block_size, hipStream_t st) {
  if (p.num_seqs <= 0) return hipSuccess;
  return launch_wide(p, (int64_t)p.num_seqs * p.num_kv_heads * p.max_row_groups * p.chunk_groups,
                     kv_dtype, head_dim, block_size, st);
}

hipError_t launch_wide_prefix_states(const RowStateParams& p, int kv_dtype, int head_dim,
                                     int block_size, hipStream_t st) {
  if (p.num_seqs <= 0 || p.query_start) return hipErrorInvalidValue;
  const int G = p.num_q_heads / p.num_kv_heads;
  return launch_wide(p, (int64_t)p.num_kv_heads * wide_row_groups((int64_t)p.num_seqs * G) *
                            p.chunk_groups,
                     kv_dtype, head_dim, block_size, st);
}

hipError_t launch_extend_finish(const ExtendFinishParams& p, int kv_dtype, int head_dim,
                                hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  if (kv_dtype == 2) {
    if (head_dim == 128) launch_finish_t<128, bf16_t>(p, st);
    else launch_finish_t<64, bf16_t>(p, st);
  } else if (kv_dtype == 1) {
    if (head_dim == 128) launch_finish_t<128, f16_t>(p, st);
    else launch_finish_t<64, f16_t>(p, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
