// Paged decode attention on the vector ALUs: any cache type (fp32 / fp16 / bf16) with one to
// eight query heads per KV head. Used for multi-head caches (G = 1), where a matrix-core tile
// would be 1/16 full, and for fp32 caches.
//
// Same contract and balanced step schedule as the matrix-core kernel (schedule.h), same
// output: normalised rows for whole segments, partial states (m, l, acc) for split pieces
// ("Paged Attention and vLLM", section "Paged Attention CUDA Kernel").
//
// Scores. A key row of d elements is LPR = d*esize/16 sixteen-byte chunks; lane l covers
// chunk l%LPR of row l/LPR, so one load instruction reads TPI = 64/LPR whole rows and a step
// reads its 32 key rows with NI = 32/TPI fully coalesced instructions. Each lane forms partial
// dot products with its slice of the G query rows; DPP butterflies inside each group of LPR
// lanes finish them.
// Values. Stored like the keys, so the value rows are read with the same instructions and each
// lane already holds the probabilities of its own token rows: it accumulates p * v over them
// into G x EPC partial sums of its head-dim slice; a piece's end sums them across the TPI
// row groups (cross-lane swaps) before the output or partial state is written.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace pkv {

template <typename T, int D, int B, int G, int W>
__global__ __launch_bounds__(64 * W) void decode_valu(DecodeParams p) {
  constexpr int ES = Elem<T>::kBytes;
  constexpr int EPC = 16 / ES;        // elements per 16-byte chunk
  constexpr int LPR = D / EPC;        // lanes per key row
  constexpr int TPI = 64 / LPR;       // key rows per load instruction
  constexpr int NI = 32 / TPI;        // key load instructions per step

  extern __shared__ int64_t smem[];
  const int S = p.num_seqs;
  int64_t* sm_prefix = smem;
  int64_t* sm_wts = smem + S + 1;
  int64_t* sm_wave = smem + 2 * (S + 1);
  int32_t* sm_len = reinterpret_cast<int32_t*>(smem + 2 * (S + 1) + 16);
  const int cap = min(p.max_context_len, p.max_blocks * B);   // the workspace is sized for it
  stage_lengths(p.lens, S, cap, sm_len);
  build_prefixes(p.lens, S, cap, p.piece_weight, sm_prefix, sm_wts, sm_wave);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= S; i += blockDim.x) {
      p.prefix[i] = sm_prefix[i];
      p.wprefix[i] = sm_wts[i];
    }

  const int lane = threadIdx.x & 63;
  const int wave = uni((int)(threadIdx.x >> 6));
  const int row = lane / LPR;
  const int ch = lane % LPR;
  const int Hkv = p.num_kv_heads;
  const int Hp = p.pool_kv_heads;
  const int w = blockIdx.x * W + wave;
  if (w >= p.num_workers) return;

  StepStream<B> ss;
  ss.sm_prefix = sm_prefix;
  ss.sm_len = sm_len;
  ss.tables = (ctable_t)p.tables;
  ss.S = S;
  ss.Hkv = Hkv;
  ss.ks = p.kv_split;
  ss.max_blocks = p.max_blocks;
  ss.num_blocks = p.num_blocks;
  ss.w = w;
  {
    const Line line = Line::make(sm_prefix, sm_wts, S, Hkv, p.piece_weight, p.num_workers);
    ss.init(line.steps_before(line.wbegin(w)), line.steps_before(line.wbegin(w + 1)));
  }
  const int64_t nsteps = ss.end - ss.b0;
  if (nsteps <= 0) return;

  const char* kbase = reinterpret_cast<const char*>(p.k_pool);
  const char* vbase = reinterpret_cast<const char*>(p.v_pool);
  const char* qbase = reinterpret_cast<const char*>(p.q);
  const size_t blk_stride = (size_t)B * D * ES;

  struct Regs {
    u32x4 k[NI];
    u32x4 v[NI];
    u32x4 q[G];   // this lane's slice of the G query rows of the step's KV head
  };

  float m_run[G], l_run[G], acc[G][EPC];
  bool poison = false, piece_rfirst = true;
  int piece_k0 = 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
  }

  auto starts_piece = [](const StepInfo& si) { return si.rfirst || si.k == 0; };

  auto load_step = [&](Regs& r, const StepInfo& si) {
    // the query rows every step, so that no load is conditional (cache hits after the first)
#pragma unroll
    for (int h = 0; h < G; ++h)
      r.q[h] = load16(qbase + (((size_t)si.s * p.num_q_heads + (size_t)si.g * G + h) * D +
                               (size_t)ch * EPC) * ES);
    const int b0 = valid_block(si.b0, p.num_blocks) ? si.b0 : 0;   // out-of-range: block 0,
    const int b1 = valid_block(si.b1, p.num_blocks) ? si.b1 : 0;   // then poison
    // fused append: the newest token's rows come from k_new / v_new
    const bool sub = p.k_new && si.k == si.ns - 1;
    const int tn = si.L - 1 - 32 * si.k;
    const size_t nofs = ((size_t)si.s * Hp + si.gp) * D * ES + (size_t)ch * 16;
    // rows at or past the step's valid tokens (every row of a step described past the end of
    // the range) are masked out, so their lanes load the first query row's line, which this
    // step loads anyway: no HBM bytes are spent on them
    const int nvalid = si.past ? 0 : si.L - 32 * si.k;
    const char* q0 = qbase + (((size_t)si.s * p.num_q_heads + (size_t)si.g * G) * D +
                              (size_t)ch * EPC) * ES;
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int tt = TPI * c + row;
      const int blk = (B == 16 && tt >= 16) ? b1 : b0;
      const size_t ofs = ((size_t)blk * Hp + si.gp) * blk_stride +
                         (size_t)(tt & (B - 1)) * D * ES + (size_t)ch * 16;
      const bool nw = sub && tt == tn;
      const bool dead = tt >= nvalid;
      const char* ka = nw ? reinterpret_cast<const char*>(p.k_new) + nofs : kbase + ofs;
      const char* va = nw ? reinterpret_cast<const char*>(p.v_new) + nofs : vbase + ofs;
      r.k[c] = load16_stream(dead ? q0 : ka);
      r.v[c] = load16_stream(dead ? q0 : va);
    }
  };

  auto begin_step = [&](const StepInfo& si) {
    if (starts_piece(si)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m_run[h] = kNegInf;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
      }
      poison = false;
      piece_rfirst = si.rfirst;
      piece_k0 = si.k;
    }
  };

  auto compute_step = [&](Regs& r, const StepInfo& si) {
    float qf[G][EPC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (ES == 4) qf[h][e] = __uint_as_float(r.q[h][e]);
        else qf[h][e] = (e & 1) ? hi16<T>(r.q[h][e >> 1]) : lo16<T>(r.q[h][e >> 1]);
      }
    const int nvalid = si.L - 32 * si.k;
    poison = poison || !valid_block(si.b0, p.num_blocks) ||
             (B == 16 && nvalid > 16 && !valid_block(si.b1, p.num_blocks));
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
      for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      // slots past the context may hold anything (NaN included): their values count as zero
      const bool live = TPI * c + row < nvalid;
      float vx[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float v;
        if constexpr (ES == 4) v = __uint_as_float(r.v[c][e]);
        else v = (e & 1) ? hi16<T>(r.v[c][e >> 1]) : lo16<T>(r.v[c][e >> 1]);
        vx[e] = live ? v : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(z[c][h], vx[e], acc[h][e]);
    }

    if (si.rlast || si.k == si.ns - 1) {
      const bool whole = piece_k0 == 0 && si.k == si.ns - 1;
      const size_t slot = piece_slot(si.range, piece_rfirst);
      const int d0 = ch * EPC;   // this lane's head-dim slice; row group 0 stores it
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float l_tot = cross_sum<LPR>(l_run[h]);
        if (poison) l_tot = __builtin_nanf("");
        float o[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[e] = cross_sum<LPR>(acc[h][e]);
        if (whole) {
          const size_t orow = (size_t)si.s * p.num_q_heads + (size_t)si.g * G + h;
          const float inv = l_tot == 0.f ? 0.f : 1.0f / l_tot;
          if (row == 0) {
            if (p.out_f32) {
              float* op = reinterpret_cast<float*>(p.out) + orow * D + d0;
#pragma unroll
              for (int e4 = 0; e4 < EPC; e4 += 4)
                store_nt(op + e4,
                         f32x4{o[e4] * inv, o[e4 + 1] * inv, o[e4 + 2] * inv, o[e4 + 3] * inv});
            } else {
              if constexpr (ES == 2) {
                u32x4 w;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  w[u] = (uint32_t)scaled_to_16<T>(o[2 * u], inv) |
                         ((uint32_t)scaled_to_16<T>(o[2 * u + 1], inv) << 16);
                store_nt(reinterpret_cast<uint16_t*>(p.out) + orow * D + d0, w);
              }
            }
          }
        } else {
          const size_t pr = slot * G + h;
          if (lane == 0) {
            store_nt(p.ws_m + pr, m_run[h]);
            store_nt(p.ws_l + pr, l_tot);
          }
          if (row == 0) {
#pragma unroll
            for (int e4 = 0; e4 < EPC; e4 += 4)
              store_nt(p.ws_acc + pr * D + d0 + e4, f32x4{o[e4], o[e4 + 1], o[e4 + 2], o[e4 + 3]});
          }
        }
      }
    }
  };

  // Software pipeline over two register buffers: while step i computes, the loads of step
  // i + 1 are in flight; the loads of step i + 2 are issued into the buffer step i has just
  // consumed, and the block ids of the step after that are being fetched (scalar loads). Past
  // the last step the stream repeats it, flagged past (its loads hit cached query lines), which
  // keeps every vector load unconditional. The loop runs over pairs of steps with its only exit
  // at the bottom, so the compiler's wait counts stay exact; an odd last step is finished after
  // it.
  Regs RA, RB;
  StepInfo sa = ss.next();
  StepInfo sb = ss.next();
  load_step(RA, sa);
  load_step(RB, sb);
  StepInfo sc = ss.next();
  for (int64_t i = 0; i + 2 <= nsteps; i += 2) {
    // RA: step i (sa); RB: step i + 1 (sb); sc describes step i + 2
    begin_step(sa);
    compute_step(RA, sa);
    load_step(RA, sc);
    const StepInfo sd = ss.next();
    begin_step(sb);
    compute_step(RB, sb);
    load_step(RB, sd);
    sa = sc;
    sb = sd;
    sc = ss.next();
  }
  if (nsteps & 1) {
    begin_step(sa);
    compute_step(RA, sa);
  }
}

template <typename T, int D, int B, int G>
static int resident_g(int waves, size_t lds) {
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (waves) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_valu<T, D, B, G, 1>, 64, lds); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_valu<T, D, B, G, 2>, 128, lds); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_valu<T, D, B, G, 4>, 256, lds); break;
    default: break;
  }
  return e == hipSuccess ? blocks * waves : 0;
}

template <typename T, int D, int B>
static int resident_t(int group, int waves, size_t lds) {
  switch (group) {
    case 1: return resident_g<T, D, B, 1>(waves, lds);
    case 2: if constexpr (sizeof(T) == 4) return resident_g<T, D, B, 2>(waves, lds); break;
    case 4: if constexpr (sizeof(T) == 4) return resident_g<T, D, B, 4>(waves, lds); break;
    case 8: if constexpr (sizeof(T) == 4) return resident_g<T, D, B, 8>(waves, lds); break;
    default: break;
  }
  return 0;
}

int decode_valu_resident_waves(int kv_dtype, int head_dim, int block_size, int group,
                               int waves, int num_seqs) {
  const size_t lds = decode_lds_bytes(num_seqs);
#define PKV_CASE(D, B)                                                                    \
  if (head_dim == D && block_size == B) {                                                 \
    if (kv_dtype == 0) return resident_t<float, D, B>(group, waves, lds);                 \
    if (kv_dtype == 1) return resident_t<f16_t, D, B>(group, waves, lds);                 \
    if (kv_dtype == 2) return resident_t<bf16_t, D, B>(group, waves, lds);                \
  }
  PKV_CASE(64, 16)
  PKV_CASE(64, 32)
  PKV_CASE(128, 16)
  PKV_CASE(128, 32)
#undef PKV_CASE
  return 0;
}

template <typename T, int D, int B, int G>
static hipError_t launch_g(const DecodeParams& p, int waves, hipStream_t st) {
  const int grid = (p.num_workers + waves - 1) / waves;
  if (grid <= 0) return hipSuccess;
  const size_t lds = decode_lds_bytes(p.num_seqs);
  switch (waves) {
    case 1: launch_kernel((decode_valu<T, D, B, G, 1>), dim3(grid), dim3(64), lds, st, p); break;
    case 2: launch_kernel((decode_valu<T, D, B, G, 2>), dim3(grid), dim3(128), lds, st, p); break;
    case 4: launch_kernel((decode_valu<T, D, B, G, 4>), dim3(grid), dim3(256), lds, st, p); break;
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
