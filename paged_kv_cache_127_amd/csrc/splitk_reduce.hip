// Merge of split segments. A (sequence, KV head) segment whose steps span several worker ranges
// of the decode schedule (schedule.h) left one partial state (m, l, acc) per range; they combine
// with the log-sum-exp rule of "Paged Attention and vLLM", section "Paged Attention CUDA Kernel":
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) acc_k / sum_k 2^(m_k - m*) l_k
// (m is kept in the log2 domain). Segments of empty sequences get a zero row here; segments
// that one range finished were written by the decode kernel and are skipped. With p.lse set,
// each merged row's log-sum-exp m* + log2(sum) is written too (-inf for an empty sequence).
// Shared-prefix mode (p.pst_m set): every segment ends here. The suffix state -- the merged
// partials, or the decode's normalised rows with their log-sum-exp for a segment one range
// finished, or nothing for an empty suffix -- is folded with the rows' prefix states by the
// same rule, and the result goes to p.final_out.
//
// WPS wavefronts per segment, four wavefronts per workgroup. The slots of a segment follow from
// the schedule arithmetic alone, range by range, so the WPS wavefronts split the segment's
// ranges among themselves (range rf + j goes to wavefront j mod WPS) and each loads the
// (m, l, acc) of up to four slots at once; lane l holds f32x4 chunks l, l + 64, ... of the
// segment's G rows (contiguous in a slot and in the output) and folds its slots into a running
// (max, numerator, denominator). With WPS = 4 the four running states meet in LDS and
// wavefront 0 writes the result. WPS = 1 (one segment per wavefront) suits segments split into
// a few ranges (fewer segments than workers is rare then); WPS = 4 suits long contexts, where
// every segment spans many ranges: up to 16 of them cost one round trip for the prefixes and
// one for the partials.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace pkv {

constexpr int kMergeBatch = 4;

// KMAX = ceil(G * D / 256): f32x4 chunks per lane (G rows of D floats over 64 lanes).
template <int D, typename T, int KMAX, int WPS>
__global__ __launch_bounds__(256) void splitk_merge(DecodeParams p) {
  static_assert(WPS == 1 || WPS == 4, "wavefronts per segment");
  constexpr int SH = WPS > 1 ? WPS : 1;
  __shared__ float sh_m[SH][WPS > 1 ? KMAX : 1][64];
  __shared__ float sh_den[SH][WPS > 1 ? KMAX : 1][64];
  __shared__ f32x4 sh_num[SH][WPS > 1 ? KMAX : 1][64];
  const int lane = threadIdx.x & 63;
  const int wv = uni((int)(threadIdx.x >> 6));
  const int wave = wv % WPS;                         // index inside the segment's wavefronts
  const int Hkv = p.num_kv_heads;
  const int seg = blockIdx.x * (4 / WPS) + wv / WPS;
  if (seg >= p.num_seqs * Hkv) return;
  const int s = seg / Hkv;
  const int g = seg - s * Hkv;
  const int G = p.num_q_heads / Hkv;
  const int n4 = G * D / 4;                          // f32x4 chunks of the segment's rows
  // the schedule values are wave-uniform: scalar loads through the constant address space
  typedef const __attribute__((address_space(4))) int64_t* cptr64;
  const cptr64 pre = (cptr64)p.prefix;
  const cptr64 wpre = (cptr64)p.wprefix;
  const int S = p.num_seqs;
  const int64_t ns = pre[s + 1] - pre[s];
  const int64_t wpre_s = wpre[s], steps_total = pre[S], wts_total = wpre[S];
  const size_t base = ((size_t)s * p.num_q_heads + (size_t)g * G) * D;

  // Fused append (k_new set): the segment's newest row -- token L - 1, keys on lanes [0, LPR),
  // values on [LPR, 2 LPR), 16 bytes per lane -- goes into its slot here, after the decode
  // kernel (which took that row from k_new / v_new) has finished: nothing in this call reads
  // the slot any more. The length, the new data and then the table entry are loaded alongside
  // the merge's own loads; a slot whose table entry is out of range is not written.
  constexpr int RB = D * (int)sizeof(T);   // bytes per row
  constexpr int LPR = RB / 16;
  // the pool KV head of schedule head g; of the kv_split segments that share it, the first
  // stores the new row (the others would store the same bytes)
  const int ks = p.kv_split;
  const int gp = g / ks;
  const int Hp = p.pool_kv_heads;
  const bool app_wave = p.k_new != nullptr && wave == 0 && g - gp * ks == 0;   // uniform
  const bool app = app_wave && lane < 2 * LPR;
  const int kvsel = lane < LPR ? 0 : 1;
  const int ch = lane % LPR;
  int Lnew = 0, blk = -1;
  u32x4 xnew = u32x4{0u, 0u, 0u, 0u};
  if (app_wave) {
    const int cap = min(p.max_context_len, p.max_blocks * p.block_size);
    Lnew = clamp_len(((ctable_t)p.lens)[s], cap);
    if (Lnew > 0) {
      blk = ((ctable_t)p.tables)[(size_t)s * p.max_blocks + (Lnew - 1) / p.block_size];
      if (app)
        xnew = load16(reinterpret_cast<const char*>(kvsel ? p.v_new : p.k_new) +
                      ((size_t)s * Hp + gp) * RB + 16 * ch);
    }
  }
  auto append_store = [&]() {
    if (app && Lnew > 0 && valid_block(blk, p.num_blocks)) {
      const int off = (Lnew - 1) % p.block_size;
      char* dst = reinterpret_cast<char*>(kvsel ? p.v_pool_w : p.k_pool_w) +
                  (((size_t)blk * Hp + gp) * p.block_size + off) * RB + 16 * ch;
      *reinterpret_cast<u32x4*>(dst) = xnew;
    }
  };

  // o * sc to the result (16-bit: the fp32 value rounded, see scaled_to_16)
  auto store = [&](int e4, f32x4 o, float sc) {
    if (p.final_f32) {
      store_nt(reinterpret_cast<float*>(p.final_out) + base + 4 * e4, o * sc);
    } else {
      if constexpr (sizeof(T) == 2) {
        const uint32_t w0 = (uint32_t)scaled_to_16<T>(o[0], sc) |
                            ((uint32_t)scaled_to_16<T>(o[1], sc) << 16);
        const uint32_t w1 = (uint32_t)scaled_to_16<T>(o[2], sc) |
                            ((uint32_t)scaled_to_16<T>(o[3], sc) << 16);
        store_nt(reinterpret_cast<uint16_t*>(p.final_out) + base + 4 * e4, u32x2{w0, w1});
      }
    }
  };

  // log-sum-exp of row (4 e4) / D, written by the lane holding the row's first chunk
  const bool prefix_mode = p.pst_m != nullptr;     // uniform
  auto store_lse = [&](int e4, float m, float den) {
    if (p.lse && !prefix_mode && e4 < n4 && (4 * e4) % D == 0)
      p.lse[base / D + (4 * e4) / D] = den > 0.f ? m + __log2f(den) : kNegInf;
  };

  // running (max, denominator, numerator) of this lane's chunks; fold(k, m, l, acc) merges one
  // more state into chunk k's
  float M[KMAX], den[KMAX];
  f32x4 num[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    M[k] = kNegInf;
    den[k] = 0.f;
    num[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto fold = [&](int k, float m, float l, f32x4 a) {
    const float m_new = fmaxf(M[k], m);
    if (m_new == kNegInf) return;
    const float a_old = fast_exp2(M[k] - m_new);
    const float a_new = fast_exp2(m - m_new);
    num[k] = num[k] * a_old + a * a_new;
    den[k] = den[k] * a_old + l * a_new;
    M[k] = m_new;
  };
  // Shared-prefix mode: the states of the rows over the shared prefix, one per chunk group
  // ([groups][S * Hq] maxima and sums, [groups][S * Hq][D] accumulators). Wavefront 0 loads
  // group c's into registers; group 0's are requested right here, before the schedule work,
  // so that their latency overlaps it.
  const size_t SHn = (size_t)S * p.num_q_heads;
  float pm[KMAX], pl[KMAX];
  f32x4 pa[KMAX];
  auto load_prefix = [&](int c) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int e4 = lane + 64 * k;
      pm[k] = kNegInf;
      pl[k] = 0.f;
      pa[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (e4 < n4) {
        const size_t row = base / D + (size_t)(4 * e4) / D;
        pm[k] = p.pst_m[c * SHn + row];
        pl[k] = p.pst_l[c * SHn + row];
        pa[k] = *reinterpret_cast<const f32x4*>(p.pst_acc + c * SHn * D + base + 4 * e4);
      }
    }
  };
  if (prefix_mode && wave == 0) load_prefix(0);
  auto fold_prefix = [&]() {
#pragma unroll 1
    for (int c = 0; c < p.pst_groups; ++c) {
      if (c > 0) load_prefix(c);
#pragma unroll
      for (int k = 0; k < KMAX; ++k) fold(k, pm[k], pl[k], pa[k]);
    }
  };

  if (ns == 0 && !prefix_mode) {   // empty sequence: zero rows (and no new row: length 0)
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (lane + 64 * k < n4) store(lane + 64 * k, f32x4{0.f, 0.f, 0.f, 0.f}, 1.f);
        store_lse(lane + 64 * k, kNegInf, 0.f);
      }
    }
    return;
  }
  const Line line = Line::from_totals(steps_total, wts_total, S, Hkv, p.piece_weight,
                                      p.num_workers);
  const int64_t seg_w = kStepWeight * ns + line.pw;
  const int64_t ws0 = (int64_t)Hkv * wpre_s + g * seg_w;              // weighted segment start
  const int64_t first = ws0 + line.pw;                                 // weighted start of step 0
  const int rf = ns > 0 ? line.owner(first) : 0;
  int rl = ns > 0 ? line.owner(first + kStepWeight * (ns - 1)) : -1;   // no slots if empty
  if (rf == rl) {   // one range holds the whole segment: written by the decode kernel
    if (!prefix_mode) {
      append_store();
      return;
    }
    // shared-prefix mode: the decode wrote the normalised rows (fp32, to out) and their
    // log-sum-exp; they are the suffix state (lse, 1, o)
    if (wave == 0) {
      float lk[KMAX];
      f32x4 ok[KMAX];
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int e4 = lane + 64 * k;
        lk[k] = kNegInf;
        ok[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (e4 < n4) {
          lk[k] = p.lse[base / D + (4 * e4) / D];
          ok[k] = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.out) + base +
                                                  4 * e4);
        }
      }
#pragma unroll
      for (int k = 0; k < KMAX; ++k) fold(k, lk[k], 1.f, ok[k]);
    }
    rl = rf - 1;
  }

  // Slot of range r's piece of this segment, or -1 if r holds none of its steps. rf's piece is
  // its first one (slot 2 rf) unless rf also holds the previous segment's last step, which
  // starts at ws0 - kStepWeight; a later range r starts inside the segment, so its piece is its
  // first one (slot 2r) if it holds any of the segment's steps.
  auto slot_of = [&](int r) -> int64_t {
    if (r == rf) return 2 * (int64_t)rf + (line.wbegin(rf) > ws0 - kStepWeight ? 0 : 1);
    const int64_t before = line.in_segment_before(line.wbegin(r), ws0, ns);
    const int64_t after = r == rl ? ns : line.in_segment_before(line.wbegin(r + 1), ws0, ns);
    return after > before ? 2 * (int64_t)r : -1;
  };

  const f32x4* acc4 = reinterpret_cast<const f32x4*>(p.ws_acc);
#pragma unroll 1
  for (int r0 = rf + wave; r0 <= rl; r0 += WPS * kMergeBatch) {
    int64_t slot[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int r = r0 + WPS * j;
      slot[j] = r <= rl ? slot_of(r) : -1;
    }
    float mj[kMergeBatch][KMAX], lj[kMergeBatch][KMAX];
    f32x4 aj[kMergeBatch][KMAX];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int e4 = lane + 64 * k;
        mj[j][k] = kNegInf;
        lj[j][k] = 0.f;
        aj[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (slot[j] >= 0 && e4 < n4) {
          const int64_t pr = slot[j] * G + (4 * e4) / D;
          mj[j][k] = p.ws_m[pr];
          lj[j][k] = p.ws_l[pr];
          aj[j][k] = acc4[slot[j] * n4 + e4];
        }
      }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (slot[j] >= 0) fold(k, mj[j][k], lj[j][k], aj[j][k]);
  }
  if (prefix_mode && wave == 0) fold_prefix();
  append_store();
  if constexpr (WPS == 1) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int e4 = lane + 64 * k;
      if (e4 < n4) store(e4, num[k], den[k] == 0.f ? 0.f : 1.0f / den[k]);
      store_lse(e4, M[k], den[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      sh_m[wave][k][lane] = M[k];
      sh_den[wave][k][lane] = den[k];
      sh_num[wave][k][lane] = num[k];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int e4 = lane + 64 * k;
      float Mx = sh_m[0][k][lane];
#pragma unroll
      for (int v = 1; v < WPS; ++v) Mx = fmaxf(Mx, sh_m[v][k][lane]);
      f32x4 nm = f32x4{0.f, 0.f, 0.f, 0.f};
      float dn = 0.f;
      if (Mx != kNegInf) {
#pragma unroll
        for (int v = 0; v < WPS; ++v) {
          const float a = fast_exp2(sh_m[v][k][lane] - Mx);
          nm += sh_num[v][k][lane] * a;
          dn += sh_den[v][k][lane] * a;
        }
      }
      if (e4 < n4) store(e4, nm, dn == 0.f ? 0.f : 1.0f / dn);
      store_lse(e4, Mx, dn);
    }
  }
}

template <int D, typename T, int WPS>
static void launch_merge_w(const DecodeParams& p, hipStream_t st) {
  const int64_t segs = (int64_t)p.num_seqs * p.num_kv_heads;
  const dim3 grid((unsigned)((segs * WPS + 3) / 4)), blk(256);
  const int chunks = (p.num_q_heads / p.num_kv_heads * D / 4 + 63) / 64;
  if (chunks <= 1)
    launch_kernel((splitk_merge<D, T, 1, WPS>), grid, blk, 0, st, p);
  else if (chunks <= 2)
    launch_kernel((splitk_merge<D, T, 2, WPS>), grid, blk, 0, st, p);
  else if (chunks <= 4)
    launch_kernel((splitk_merge<D, T, 4, WPS>), grid, blk, 0, st, p);
  else
    launch_kernel((splitk_merge<D, T, 8, WPS>), grid, blk, 0, st, p);
}

// Fewer segments than workers means every segment spans several ranges on average: four
// wavefronts per segment; else one.
template <int D, typename T>
static void launch_merge_t(const DecodeParams& p, hipStream_t st) {
  if ((int64_t)p.num_seqs * p.num_kv_heads < (int64_t)p.num_workers)
    launch_merge_w<D, T, 4>(p, st);
  else
    launch_merge_w<D, T, 1>(p, st);
}

hipError_t launch_splitk_reduce(const DecodeParams& p, int kv_dtype, int head_dim,
                                hipStream_t st) {
  const int64_t segs = (int64_t)p.num_seqs * p.num_kv_heads;
  if (segs <= 0) return hipSuccess;
  if (head_dim == 64) {
    if (kv_dtype == 1) launch_merge_t<64, f16_t>(p, st);
    else if (kv_dtype == 2) launch_merge_t<64, bf16_t>(p, st);
    else launch_merge_t<64, float>(p, st);
  } else if (head_dim == 128) {
    if (kv_dtype == 1) launch_merge_t<128, f16_t>(p, st);
    else if (kv_dtype == 2) launch_merge_t<128, bf16_t>(p, st);
    else launch_merge_t<128, float>(p, st);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
