// Grouped-query paged decode attention on CDNA4 matrix cores (16-bit caches, G = 2..16).
//
// What it computes ("Paged Attention and vLLM", sections "Block Table and Logical-to-
// Physical Mapping" and "Paged Attention CUDA Kernel"): for one sequence s, one KV head g and
// one partition of the context, the partial softmax state (m, l, acc) of the G query heads
// g*G .. g*G+G-1 over the partition's tokens, with keys and values read straight from the
// physical blocks named by the block table (no contiguous copy). A single-partition sequence
// writes its normalised output directly; otherwise the split-K reduce kernel merges the
// partials with the log-sum-exp rule.
//
// Work decomposition. One workgroup = one (sequence, KV head, partition); W wavefronts share
// the partition's 32-token steps round-robin. The workgroup id is decoded KV-head-fastest, so
// with 8 KV heads every head stays on one XCD (consecutive ids go to consecutive XCDs): the L2
// of that XCD sees all reads of that head's blocks, which helps shared-prefix blocks.
//
// Per 32-token step a wavefront issues (per lane) 8 + 8 16-byte loads:
//   K operand, sub-tile a (0/1), d-chunk c: key row tau(a, i) = 8*(i/4) + 4a + i%4 of the
//     step, i = lane%16, head-dim slice [32c + 8*(lane/16), +8).
//   V operand, d-chunk f: value row d = 16f + lane%16 (values are stored [d][B] inside a
//     block), tokens 8*(lane/16) .. +8 of the step -- one contiguous 16-byte run.
// Scores S^T[token][head] = K . Q^T come out of v_mfma_f32_16x16x32 with lane l holding head
// l%16 and tokens 8*(l/16) + 4a + e (e = 0..3) -- exactly the 8 consecutive tokens whose
// values the same lane loaded, so the probabilities feed the P.V MFMA
// (O^T[d][head] += V^T . P^T) as its B operand without any data exchange.
// Probabilities are split into a 16-bit high part and a 16-bit remainder (two MFMAs), which
// keeps P.V at close to fp32 accuracy. Scores and the online softmax stay in fp32; the scale
// (times log2 e) is applied to the fp32 scores and exp2 is used throughout.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

template <typename T>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (__is_same(T, bf16_t)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

template <int D>
struct StepRegs {
  u32x4 k[2][D / 32];   // K operand per sub-tile and d-chunk
  u32x4 v[D / 16];      // V operand per d-chunk
};

// Split two fp32 probabilities into packed 16-bit high parts and remainders.
template <typename T>
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  uint16_t h0 = Elem<T>::from_f32(p0), h1 = Elem<T>::from_f32(p1);
  float r0 = p0 - Elem<T>::to_f32(h0), r1 = p1 - Elem<T>::to_f32(h1);
  hi = (uint32_t)h0 | ((uint32_t)h1 << 16);
  lo = (uint32_t)Elem<T>::from_f32(r0) | ((uint32_t)Elem<T>::from_f32(r1) << 16);
}

template <typename T, int D, int B, int W>
__global__ __launch_bounds__(64 * W) void decode_partial_mfma(DecodeParams p) {
  static_assert(B == 16 || B == 32, "block size");
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NC = D / 32;   // QK MFMAs per sub-tile
  constexpr int NF = D / 16;   // PV MFMA output chunks
  constexpr int ES = 2;        // element bytes

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int jg = lane >> 4;

  int wg = blockIdx.x;
  const int Hkv = p.num_kv_heads;
  const int g = wg % Hkv;
  wg /= Hkv;
  const int s = wg % p.num_seqs;
  const int part = wg / p.num_seqs;
  const int G = p.num_q_heads / Hkv;

  // lengths beyond the table or the launch are clamped: never read past either
  const int cap = min(p.max_blocks * B, p.n_part_max * p.partition);
  int L = p.lens[s];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int n_part = L > 0 ? ceil_div(L, p.partition) : 1;
  if (part >= n_part) return;   // uniform for the whole workgroup
  const int t0 = part * p.partition;
  const int t1 = min(t0 + p.partition, L);
  const int n_steps = t1 > t0 ? ceil_div(t1 - t0, 32) : 0;

  // Query operand: Q^T[d][head], lane holds head r16, d-slice [32c + 8jg, +8) of chunk c.
  u32x4 qv[NC];
  {
    const char* qp = reinterpret_cast<const char*>(p.q) +
                     (((size_t)s * p.num_q_heads + (size_t)g * G + r16) * D + 8 * jg) * ES;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qv[c] = r16 < G ? load16(qp + 32 * c * ES) : u32x4{0, 0, 0, 0};
  }

  // This partition's block-table entries (<= 64), one per lane.
  const int jb0 = t0 / B;
  const int nbp = t1 > t0 ? ceil_div(t1 - t0, B) : 0;
  int tbl = 0;
  bool bad = false;
  if (lane < nbp) {
    tbl = p.tables[(size_t)s * p.max_blocks + jb0 + lane];
    bad = (unsigned)tbl >= (unsigned)p.num_blocks;
    if (bad) tbl = 0;
  }
  const bool poisoned = __builtin_amdgcn_ballot_w64(bad) != 0;

  const char* kbase = reinterpret_cast<const char*>(p.k_pool);
  const char* vbase = reinterpret_cast<const char*>(p.v_pool);
  const size_t kv_block_stride = (size_t)B * D * ES;   // bytes per (block, head)

  // Fixed per-lane parts of the addresses.
  const int tokA0 = 8 * (r16 >> 2) + (r16 & 3);      // sub-tile 0 token (sub-tile 1: +4)
  const size_t k_lane_off = (size_t)(8 * jg) * ES;
  const int vtok = 8 * jg;                           // first of this lane's 8 value tokens

  auto load_step = [&](StepRegs<D>& r, int step) {
    const int rel = (step * 32) / B;                 // partition-relative block of the step
    int b0 = __builtin_amdgcn_readlane(tbl, rel);
    int b1 = b0;
    if constexpr (B == 16) {
      if (t0 + step * 32 + 16 < t1) b1 = __builtin_amdgcn_readlane(tbl, rel + 1);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int tok = tokA0 + 4 * a;
      const int blk = (B == 16 && tok >= 16) ? b1 : b0;
      const int off = tok & (B - 1);
      const char* kp = kbase + ((size_t)blk * Hkv + g) * kv_block_stride +
                       (size_t)off * D * ES + k_lane_off;
#pragma unroll
      for (int c = 0; c < NC; ++c) r.k[a][c] = load16(kp + 32 * c * ES);
    }
    {
      const int blk = (B == 16 && vtok >= 16) ? b1 : b0;
      const int off = vtok & (B - 1);
      const char* vp = vbase + ((size_t)blk * Hkv + g) * kv_block_stride +
                       ((size_t)r16 * B + off) * ES;
#pragma unroll
      for (int f = 0; f < NF; ++f) r.v[f] = load16(vp + (size_t)16 * f * B * ES);
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) oacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_step = [&](StepRegs<D>& r, int step) {
    const int tb = t0 + step * 32;
    const int nvalid = t1 - tb;                      // valid tokens in this step (>= 1)
    f32x4 sacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[a] = mfma16x16x32<T>(r.k[a][c], qv[c], sacc[a]);
    }
    float z[8];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = vtok + 4 * a + e;
        z[4 * a + e] = tok < nvalid ? sacc[a][e] * p.scale_log2 : kNegInf;
      }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = cross_max<16>(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float pr[8];
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = fast_exp2(z[i] - m_new);
      ps += pr[i];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[f] *= alpha;

    u32x4 phi, plo;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t h, l;
      split_pair<T>(pr[2 * w], pr[2 * w + 1], h, l);
      phi[w] = h;
      plo[w] = l;
    }
    if (nvalid < 32) {
      // zero the value entries of slots past the context (they may hold anything)
      const int nv = nvalid - vtok;
      u32x4 msk;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        msk[w] = (2 * w < nv ? 0xffffu : 0u) | (2 * w + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
      for (int f = 0; f < NF; ++f) r.v[f] &= msk;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      oacc[f] = mfma16x16x32<T>(r.v[f], phi, oacc[f]);
      oacc[f] = mfma16x16x32<T>(r.v[f], plo, oacc[f]);
    }
  };

  // Software pipeline: the next step's loads are in flight while the current one computes.
  // Past the last step the "next" load repeats the current step's addresses (cache hits),
  // which keeps every load unconditional.
  {
    StepRegs<D> R0, R1;
    int st = wave;
    if (st < n_steps) {
      load_step(R0, st);
      while (true) {
        int nx = st + W < n_steps ? st + W : st;
        load_step(R1, nx);
        compute_step(R0, st);
        st += W;
        if (st >= n_steps) break;
        nx = st + W < n_steps ? st + W : st;
        load_step(R0, nx);
        compute_step(R1, st);
        st += W;
        if (st >= n_steps) break;
      }
    }
  }

  // l over the four lane groups that hold the same head
  l_run = cross_sum<16>(l_run);
  if (poisoned) {
    l_run = __builtin_nanf("");
  }

  // ---- merge the W wavefronts of this workgroup (wave 0 keeps the result) --------------
  constexpr int DP = D + 4;   // padded row: spreads heads over LDS banks
  __shared__ float sm_m[W][16];
  __shared__ float sm_l[W][16];
  __shared__ float sm_acc[W > 1 ? W - 1 : 1][16][DP];
  if constexpr (W > 1) {
    if (wave > 0) {
      if (jg == 0) {
        sm_m[wave][r16] = m_run;
        sm_l[wave][r16] = l_run;
      }
#pragma unroll
      for (int f = 0; f < NF; ++f)
        *reinterpret_cast<f32x4*>(&sm_acc[wave - 1][r16][16 * f + 4 * jg]) = oacc[f];
    }
    __syncthreads();
    if (wave > 0) return;
    float mw[W];
    mw[0] = m_run;
    float m_star = m_run;
#pragma unroll
    for (int w = 1; w < W; ++w) {
      mw[w] = sm_m[w][r16];
      m_star = fmaxf(m_star, mw[w]);
    }
    const bool empty = m_star == kNegInf;
    float c0 = empty ? 0.f : fast_exp2(m_run - m_star);
    l_run *= c0;
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[f] *= c0;
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const float cw = empty ? 0.f : fast_exp2(mw[w] - m_star);
      l_run += cw * sm_l[w][r16];
#pragma unroll
      for (int f = 0; f < NF; ++f)
        oacc[f] += cw * *reinterpret_cast<const f32x4*>(&sm_acc[w - 1][r16][16 * f + 4 * jg]);
    }
    m_run = m_star;
  }

  if (r16 >= G) return;
  const int h = g * G + r16;
  const size_t row = (size_t)s * p.num_q_heads + h;
  if (n_part == 1) {
    const float inv_ok = l_run;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = inv_ok == 0.f ? 0.f : oacc[f][e] / inv_ok;
      const int d0 = 16 * f + 4 * jg;
      if (p.out_f32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + d0) = o;
      } else {
        uint16_t* op = reinterpret_cast<uint16_t*>(p.out) + row * D + d0;
        uint32_t w0 = (uint32_t)Elem<T>::from_f32(o[0]) | ((uint32_t)Elem<T>::from_f32(o[1]) << 16);
        uint32_t w1 = (uint32_t)Elem<T>::from_f32(o[2]) | ((uint32_t)Elem<T>::from_f32(o[3]) << 16);
        *reinterpret_cast<uint2*>(op) = make_uint2(w0, w1);
      }
    }
  } else {
    const size_t pr = row * p.n_part_max + part;
    if (jg == 0) {
      p.ws_m[pr] = m_run;
      p.ws_l[pr] = l_run;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
      *reinterpret_cast<f32x4*>(p.ws_acc + pr * D + 16 * f + 4 * jg) = oacc[f];
  }
}

template <typename T, int D, int B>
static hipError_t launch_t(const DecodeParams& p, int waves, hipStream_t st) {
  const int64_t grid = (int64_t)p.num_kv_heads * p.num_seqs * p.n_part_max;
  if (grid <= 0) return hipSuccess;
  switch (waves) {
    case 1: hipLaunchKernelGGL((decode_partial_mfma<T, D, B, 1>), dim3((unsigned)grid), dim3(64), 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_partial_mfma<T, D, B, 2>), dim3((unsigned)grid), dim3(128), 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_partial_mfma<T, D, B, 4>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int head_dim, int block_size,
                              int waves, hipStream_t st) {
  const bool bf = kv_dtype == 2;
#define PKV_CASE(D, B)                                                              \
  if (head_dim == D && block_size == B)                                             \
    return bf ? launch_t<bf16_t, D, B>(p, waves, st) : launch_t<f16_t, D, B>(p, waves, st);
  PKV_CASE(64, 16)
  PKV_CASE(64, 32)
  PKV_CASE(128, 16)
  PKV_CASE(128, 32)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
