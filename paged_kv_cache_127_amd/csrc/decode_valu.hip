// Paged decode attention on the vector ALUs: any cache type (fp32 / fp16 / bf16) with one to
// eight query heads per KV head. Used for multi-head caches (G = 1), where a matrix-core tile
// would be 1/16 full, and for fp32 caches.
//
// Same contract and work decomposition as the matrix-core kernel (one workgroup per
// (sequence, KV head, partition); W wavefronts share the partition's 32-token steps), same
// partial-state output ("Paged Attention and vLLM", section "Paged Attention CUDA Kernel").
//
// Scores. A key row of d elements is LPR = d*esize/16 sixteen-byte chunks; lane l covers
// chunk l%LPR of row l/LPR, so one load instruction reads TPI = 64/LPR whole rows and a step
// reads its 32 key rows with NI = 32/TPI fully coalesced instructions. Each lane forms partial
// dot products with its slice of the G query rows; DPP butterflies inside each group of LPR
// lanes finish them.
// Values. Stored [d][B] inside a block, so lane l owns head-dim rows l and l+64 and reads their
// token runs contiguously; the step's probabilities go through LDS (one broadcast read per
// four tokens) and each lane accumulates its own output rows -- no cross-lane reduction.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

template <typename T, int D, int B, int G, int W>
__global__ __launch_bounds__(64 * W) void decode_partial_valu(DecodeParams p) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int EPC = 16 / ES;        // elements per 16-byte chunk
  constexpr int LPR = D / EPC;        // lanes per key row
  constexpr int TPI = 64 / LPR;       // key rows per load instruction
  constexpr int NI = 32 / TPI;        // key load instructions per step
  constexpr int DU = D / 64;          // head-dim rows of V owned per lane
  constexpr int BPS = 32 / B;         // blocks per step
  constexpr int VCH = B * ES / 16;    // 16-byte chunks in one value row of a block
  constexpr int VE = 16 / ES;         // elements per value chunk

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / LPR;
  const int ch = lane % LPR;

  int wg = blockIdx.x;
  const int Hkv = p.num_kv_heads;
  const int g = wg % Hkv;
  wg /= Hkv;
  const int s = wg % p.num_seqs;
  const int part = wg / p.num_seqs;

  // lengths beyond the table or the launch are clamped: never read past either
  const int cap = min(p.max_blocks * B, p.n_part_max * p.partition);
  int L = p.lens[s];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int n_part = L > 0 ? ceil_div(L, p.partition) : 1;
  if (part >= n_part) return;
  const int t0 = part * p.partition;
  const int t1 = min(t0 + p.partition, L);
  const int n_steps = t1 > t0 ? ceil_div(t1 - t0, 32) : 0;

  // this lane's slice of the G query rows, widened to fp32
  float qf[G][EPC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const char* qp = reinterpret_cast<const char*>(p.q) +
                     (((size_t)s * p.num_q_heads + (size_t)g * G + h) * D + (size_t)ch * EPC) * ES;
    u32x4 w = load16(qp);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if constexpr (ES == 4) qf[h][e] = __uint_as_float(w[e]);
      else qf[h][e] = (e & 1) ? hi16<T>(w[e >> 1]) : lo16<T>(w[e >> 1]);
    }
  }

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
  const size_t blk_stride = (size_t)B * D * ES;

  struct Regs {
    u32x4 k[NI];
    u32x4 v[DU][BPS][VCH];
  };

  auto load_step = [&](Regs& r, int step) {
    const int rel = (step * 32) / B;
    int b0 = __builtin_amdgcn_readlane(tbl, rel);
    int b1 = b0;
    if constexpr (B == 16) {
      if (t0 + step * 32 + 16 < t1) b1 = __builtin_amdgcn_readlane(tbl, rel + 1);
    }
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int tt = TPI * c + row;
      const int blk = (B == 16 && tt >= 16) ? b1 : b0;
      const int off = tt & (B - 1);
      r.k[c] = load16(kbase + ((size_t)blk * Hkv + g) * blk_stride + (size_t)off * D * ES +
                      (size_t)ch * 16);
    }
#pragma unroll
    for (int u = 0; u < DU; ++u)
#pragma unroll
      for (int bb = 0; bb < BPS; ++bb) {
        const int blk = bb ? b1 : b0;
        const char* vp = vbase + ((size_t)blk * Hkv + g) * blk_stride +
                         (size_t)(lane + 64 * u) * B * ES;
#pragma unroll
        for (int x = 0; x < VCH; ++x) r.v[u][bb][x] = load16(vp + 16 * x);
      }
  };

  float m_run[G], l_run[G], acc[G][DU];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[h][u] = 0.f;
  }

  __shared__ float sp[W][G][32];

  auto value_at = [&](const Regs& r, int u, int t) -> float {
    const int bb = t / B;
    const int tt = t % B;
    const uint32_t w = r.v[u][bb][tt / VE][(tt % VE) / (4 / ES)];
    if constexpr (ES == 4) return __uint_as_float(w);
    else return (tt & 1) ? hi16<T>(w) : lo16<T>(w);
  };

  auto compute_step = [&](Regs& r, int step) {
    const int tb = t0 + step * 32;
    const int nvalid = t1 - tb;
    float z[NI][G];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      float kx[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (ES == 4) kx[e] = __uint_as_float(r.k[c][e]);
        else kx[e] = (e & 1) ? hi16<T>(r.k[c][e >> 1]) : lo16<T>(r.k[c][e >> 1]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) a = fmaf(qf[h][e], kx[e], a);
        a = group_sum<LPR>(a);
        z[c][h] = (TPI * c + row < nvalid) ? a * p.scale_log2 : kNegInf;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = z[0][h];
#pragma unroll
      for (int c = 1; c < NI; ++c) mx = fmaxf(mx, z[c][h]);
      mx = cross_max<LPR>(mx);
      const float m_new = fmaxf(m_run[h], mx);
      const float alpha = fast_exp2(m_run[h] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int c = 0; c < NI; ++c) {
        z[c][h] = fast_exp2(z[c][h] - m_new);
        ps += z[c][h];
      }
      l_run[h] = l_run[h] * alpha + ps;
      m_run[h] = m_new;
#pragma unroll
      for (int u = 0; u < DU; ++u) acc[h][u] *= alpha;
    }
    if (ch == 0) {
#pragma unroll
      for (int c = 0; c < NI; ++c)
#pragma unroll
        for (int h = 0; h < G; ++h) sp[wave][h][TPI * c + row] = z[c][h];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool tail = nvalid < 32;
#pragma unroll
    for (int t4 = 0; t4 < 8; ++t4) {
      f32x4 pw[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pw[h] = *reinterpret_cast<const f32x4*>(&sp[wave][h][4 * t4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * t4 + e;
#pragma unroll
        for (int u = 0; u < DU; ++u) {
          float v = value_at(r, u, t);
          if (tail && t >= nvalid) v = 0.f;   // slots past the context may hold anything
#pragma unroll
          for (int h = 0; h < G; ++h) acc[h][u] = fmaf(pw[h][e], v, acc[h][u]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  {
    Regs R0, R1;
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

#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = cross_sum<LPR>(l_run[h]);
    if (poisoned) l_run[h] = __builtin_nanf("");
  }

  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  __shared__ float sm_acc[W > 1 ? W - 1 : 1][G][D];
  if constexpr (W > 1) {
    if (wave > 0) {
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          sm_m[wave][h] = m_run[h];
          sm_l[wave][h] = l_run[h];
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int u = 0; u < DU; ++u) sm_acc[wave - 1][h][lane + 64 * u] = acc[h][u];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m_star = m_run[h];
#pragma unroll
      for (int w = 1; w < W; ++w) m_star = fmaxf(m_star, sm_m[w][h]);
      const bool empty = m_star == kNegInf;
      const float c0 = empty ? 0.f : fast_exp2(m_run[h] - m_star);
      l_run[h] *= c0;
#pragma unroll
      for (int u = 0; u < DU; ++u) acc[h][u] *= c0;
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float cw = empty ? 0.f : fast_exp2(sm_m[w][h] - m_star);
        l_run[h] += cw * sm_l[w][h];
#pragma unroll
        for (int u = 0; u < DU; ++u) acc[h][u] += cw * sm_acc[w - 1][h][lane + 64 * u];
      }
      m_run[h] = m_star;
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t orow = (size_t)s * p.num_q_heads + (size_t)g * G + h;
    if (n_part == 1) {
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const float o = l_run[h] == 0.f ? 0.f : acc[h][u] / l_run[h];
        const int d = lane + 64 * u;
        if (p.out_f32) {
          reinterpret_cast<float*>(p.out)[orow * D + d] = o;
        } else {
          if constexpr (ES == 2)
            reinterpret_cast<uint16_t*>(p.out)[orow * D + d] = Elem<T>::from_f32(o);
        }
      }
    } else {
      const size_t pr = orow * p.n_part_max + part;
      if (lane == 0) {
        p.ws_m[pr] = m_run[h];
        p.ws_l[pr] = l_run[h];
      }
#pragma unroll
      for (int u = 0; u < DU; ++u) p.ws_acc[pr * D + lane + 64 * u] = acc[h][u];
    }
  }
}

template <typename T, int D, int B, int G>
static hipError_t launch_g(const DecodeParams& p, int waves, hipStream_t st) {
  const int64_t grid = (int64_t)p.num_kv_heads * p.num_seqs * p.n_part_max;
  if (grid <= 0) return hipSuccess;
  switch (waves) {
    case 1: hipLaunchKernelGGL((decode_partial_valu<T, D, B, G, 1>), dim3((unsigned)grid), dim3(64), 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_partial_valu<T, D, B, G, 2>), dim3((unsigned)grid), dim3(128), 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_partial_valu<T, D, B, G, 4>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D, int B>
static hipError_t launch_t(const DecodeParams& p, int group, int waves, hipStream_t st) {
  switch (group) {
    case 1: return launch_g<T, D, B, 1>(p, waves, st);
    case 2: if constexpr (sizeof(T) == 4) return launch_g<T, D, B, 2>(p, waves, st); break;
    case 4: if constexpr (sizeof(T) == 4) return launch_g<T, D, B, 4>(p, waves, st); break;
    case 8: if constexpr (sizeof(T) == 4) return launch_g<T, D, B, 8>(p, waves, st); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, int head_dim, int block_size,
                              int group, int waves, hipStream_t st) {
#define PKV_CASE(D, B)                                                                    \
  if (head_dim == D && block_size == B) {                                                 \
    if (kv_dtype == 0) return launch_t<float, D, B>(p, group, waves, st);                 \
    if (kv_dtype == 1) return launch_t<f16_t, D, B>(p, group, waves, st);                 \
    if (kv_dtype == 2) return launch_t<bf16_t, D, B>(p, group, waves, st);                \
  }
  PKV_CASE(64, 16)
  PKV_CASE(64, 32)
  PKV_CASE(128, 16)
  PKV_CASE(128, 32)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
