// Grouped-query paged decode attention on CDNA4 matrix cores (16-bit caches, G = 2..16).
//
// What it computes ("Paged Attention and vLLM", sections "Block Table and Logical-to-
// Physical Mapping" and "Paged Attention CUDA Kernel"): for every piece of a (sequence, KV
// head) segment in this wavefront's range of the balanced step line (schedule.h), the
// softmax state (m, l, acc) of the G query heads g*G .. g*G+G-1 over the piece's tokens, with
// keys and values read straight from the physical blocks named by the block table (no
// contiguous copy). Whole segments are normalised and written to the output; split pieces
// write partial states that the merge kernel combines.
//
// Per 32-token step (D = 128) a wavefront issues (per lane) 8 + 8 16-byte loads, key rows and
// value rows alike: instruction f reads row 4f + lane/16 of the step, head-dim slice
// [8*(lane%16), +8) -- four whole 256-byte rows per instruction. (Loading the keys straight in
// the score operand's layout -- 16 rows x 64 bytes per instruction -- streamed about 10 % slower
// in a gather probe of the same tiles: 6.1-6.3 against 6.8 TB/s.) The key rows go through the
// wavefront's LDS tile and come back as the score MFMA's A operand: sub-tile a (0/1), d-chunk c
// is key row tau(a, i) = 8*(i/4) + 4a + i%4 of the step, i = lane%16, head-dim slice
// [32c + 8*(lane/16), +8) (16-byte pieces XOR-swizzled per row, key_piece).
// Scores S^T[token][head] = K . Q^T come out of v_mfma_f32_16x16x32 with lane l holding head
// l%16 and tokens 8*(l/16) + 4a + e (e = 0..3), i.e. 8 consecutive tokens, which is the B
// operand layout of the P.V MFMA (O^T[d][head] += V^T . P^T): the probabilities need no data
// exchange. Its A operand wants, per lane, those 8 tokens of one head-dim column: the value
// rows go through the same per-wavefront LDS tile after the keys (32-byte pieces XOR-swizzled by
// row so that both the row writes and the column reads spread over the banks) and come back
// transposed with
// ds_read_b64_tr_b16 (in each 16-lane group, lane i receives element i%4 of the 4 x 16-bit
// words that lanes 4k + i/4 address, k = 0..3: lanes 4k + c address token row k, head-dim
// columns 4c .. 4c + 3 of the 16-column chunk).
// Probabilities are split into a 16-bit high part and a 16-bit remainder (two MFMAs), which
// keeps P.V at close to fp32 accuracy. Scores and the online softmax stay in fp32; the scale
// (times log2 e) is applied to the fp32 scores and exp2 is used throughout.
// Two steps' loads (with their query rows) are in flight while a step computes.
// Fused append (k_new set): in a segment's last step, the lanes of the row of token L - 1 read
// it from k_new / v_new instead of the pool (the merge kernel stores it into its slot later).
// With p.lse set, a whole segment also writes each row's log-sum-exp m + log2(l) (the
// shared-prefix path merges the output with the prefix's states through it).
#include "device_common.h"
#include "kernels.h"
#include "mfma_common.h"
#include "schedule.h"

namespace pkv {

template <int D>
struct StepRegs {
  u32x4 k[D / 16];      // key rows, 16 bytes per lane per instruction
  u32x4 v[D / 16];      // value rows, the same
  u32x4 q[D / 32];      // Q operand (the step's query rows)
};

#ifndef PKV_MFMA_WAVES_PER_EU
#define PKV_MFMA_WAVES_PER_EU 1
#endif

// At least PKV_MFMA_WAVES_PER_EU resident wavefronts per SIMD: the compiler keeps the whole
// state (two steps of K/V/Q operands, accumulators) within that register budget.
// STREAM: key/value rows through streaming (non-temporal) loads -- the choice for a decode that
// reads its blocks once (GQA batch: 168 vs 177 us); plain loads when blocks are re-read from
// the caches within the call (128 sequences over a shared 800-token prefix: 66 us plain vs
// 94 us streaming; the suffix decode of the shared-prefix call: 40 vs 43 us).
template <typename T, int D, int B, int W, bool STREAM = true>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_WAVES_PER_EU)))
void decode_mfma(DecodeParams p) {
  static_assert(B == 16 || B == 32, "block size");
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NC = D / 32;   // QK MFMAs per sub-tile
  constexpr int NF = D / 16;   // PV MFMA output chunks
  constexpr int ES = 2;        // element bytes

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
  const int r16 = lane & 15;
  const int jg = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const int Hp = p.pool_kv_heads;
  const int G = p.num_q_heads / Hkv;
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
  const size_t kv_block_stride = (size_t)B * D * ES;   // bytes per (block, head)
  const int tokA0 = 8 * (r16 >> 2) + (r16 & 3);        // sub-tile 0 key row (sub-tile 1: +4)
  const int vtok = 8 * jg;                             // first of this lane's 8 value tokens
  constexpr int VLPR = D / 8;           // lanes per key / value row (16 bytes each)
  constexpr int VTPI = 64 / VLPR;       // value rows per load instruction
  constexpr int RB = D * ES;            // bytes per value row
  const int vrow = lane / VLPR;
  const int vch = lane % VLPR;

  // Output ring (dynamic LDS after the schedule arrays and the workgroup's value tiles): piece
  // results are staged here and written to memory only when the ring is full or the range is
  // done. A vector store that is still in flight makes every later wait for a vector load a
  // full drain (loads and stores share one counter and stores complete out of order), so
  // stores stay out of the streaming loop. Entry: G rows of D floats, then the G running maxima
  // and sums (partials); header: destination element offset and (slot << 2 | kind).
  const int R = p.ring_cap;
  const int EF = G * D + 2 * G;
  char* ring = reinterpret_cast<char*>(smem) + ring_offset(S) + (size_t)W * 32 * RB +
               (size_t)wave * R * (16 + (size_t)EF * 4);
  int64_t* rhdr = reinterpret_cast<int64_t*>(ring);
  // staging tile of this wavefront (before the rings): a step's key rows, then its value rows.
  // Per-lane byte offsets of the key row writes (instruction f) and score-operand reads
  // (sub-tile a, d-chunk c), of the value row writes and of the transposed reads (token half
  // hh, piece f: XOR f << 5)
  char* vstage = reinterpret_cast<char*>(smem) + ring_offset(S) + (size_t)wave * 32 * RB;
  int kw_ofs[NF], vw_ofs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int t = VTPI * f + vrow;
    kw_ofs[f] = t * RB + (key_piece<D>(t, vch) << 4);
    vw_ofs[f] = t * RB + (((vch >> 1) ^ piece_swizzle<D>(t)) << 5) + 16 * (vch & 1);
  }
  int kr_ofs[2][NC];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int t = tokA0 + 4 * a;
      kr_ofs[a][c] = t * RB + (key_piece<D>(t, jg + 4 * c) << 4);
    }
  int vr_ofs[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int t = 8 * jg + 4 * hh + (r16 >> 2);
    vr_ofs[hh] = t * RB + (piece_swizzle<D>(t) << 5) + 8 * (r16 & 3);
  }
  float* rdat = reinterpret_cast<float*>(ring + (size_t)R * 16);
  int ring_n = 0;
  float m_run = kNegInf, l_run = 0.f;
  bool poison = false, piece_rfirst = true;
  int piece_k0 = 0;
  f32x4 oacc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) oacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto starts_piece = [](const StepInfo& si) { return si.rfirst || si.k == 0; };

  // All loads of a step are unconditional and branch-free, so the compiler's wait counts stay
  // exact across the pipelined loop. The query rows are loaded every step (cache hits after a
  // piece's first step); the padding columns of the 16-wide tile repeat head G-1 and are never
  // stored.
  const int qrow = r16 < G ? r16 : G - 1;
  // A step described past the end of the range is never computed: its lanes load the lane's
  // own query row instead, a line the same step loads anyway, so no HBM bytes are spent on it.
  // (Pointing the masked rows past a real step's valid tokens there as well made the 16-token
  // block kernel slower on the GQA batch, 169 -> 174 us, so those rows are read as they are.)
  auto qrow_addr = [&](const StepInfo& si) {
    return qbase + (((size_t)si.s * p.num_q_heads + (size_t)si.g * G + qrow) * D + 8 * jg) * ES;
  };
  auto load_q = [&](StepRegs<D>& r, const StepInfo& si) {
    const char* qp = qrow_addr(si);
#pragma unroll
    for (int c = 0; c < NC; ++c) r.q[c] = load16(qp + 32 * c * ES);
  };
  // rows of a step from K (kv = 0) or V (kv = 1): instruction f reads row VTPI * f + lane / VLPR
  auto load_rows = [&](u32x4 (&dst)[NF], const StepInfo& si, int kv) {
    const int b0 = valid_block(si.b0, p.num_blocks) ? si.b0 : 0;   // out-of-range: block 0,
    const int b1 = valid_block(si.b1, p.num_blocks) ? si.b1 : 0;   // then poison
    // fused append: in a segment's last step, the newest token's row from k_new / v_new
    const bool sub = p.k_new && si.k == si.ns - 1;
    const int tn = si.L - 1 - 32 * si.k;
    const char* qp = qrow_addr(si);
    const char* base = kv ? vbase : kbase;
    const char* nrow = reinterpret_cast<const char*>(kv ? p.v_new : p.k_new) +
                       ((size_t)si.s * Hp + si.gp) * RB + 16 * vch;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int t = VTPI * f + vrow;
      const int blk = (B == 16 && t >= 16) ? b1 : b0;
      const char* a = base + ((size_t)blk * Hp + si.gp) * kv_block_stride +
                      (size_t)(t & (B - 1)) * RB + 16 * vch;
      if (sub && t == tn) a = nrow;
      if (si.past) a = qp;
      dst[f] = STREAM ? load16_stream(a) : load16(a);
    }
  };
  // STREAM: key rows (through the LDS tile); otherwise straight in the score operand's layout,
  // r.k[NC * a + c] = sub-tile a, d-chunk c -- for blocks re-read from the caches, whose latency
  // bound the extra LDS round trip would lengthen
  const int kofs0 = ((tokA0 & (B - 1)) * D + 8 * jg) * ES;
  const int kofs1 = (((tokA0 + 4) & (B - 1)) * D + 8 * jg) * ES;
  auto load_k = [&](StepRegs<D>& r, const StepInfo& si) {
    if constexpr (STREAM) {
      load_rows(r.k, si, 0);
    } else {
      const int b0 = valid_block(si.b0, p.num_blocks) ? si.b0 : 0;
      const int b1 = valid_block(si.b1, p.num_blocks) ? si.b1 : 0;
      const char* t0 = kbase + ((size_t)b0 * Hp + si.gp) * kv_block_stride;
      const char* t1 = kbase + ((size_t)b1 * Hp + si.gp) * kv_block_stride;
      const char* ka = ((B == 16 && tokA0 >= 16) ? t1 : t0) + kofs0;
      const char* kb = ((B == 16 && tokA0 + 4 >= 16) ? t1 : t0) + kofs1;
      if (p.k_new && si.k == si.ns - 1) {   // fused append, as in load_rows
        const int tn = si.L - 1 - 32 * si.k;
        const char* kn = reinterpret_cast<const char*>(p.k_new) +
                         ((size_t)si.s * Hp + si.gp) * RB + 8 * jg * ES;
        if (tokA0 == tn) ka = kn;
        if (tokA0 + 4 == tn) kb = kn;
      }
      if (si.past) {
        const char* qp = qrow_addr(si);
        ka = qp;
        kb = qp;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        r.k[c] = load16(ka + 32 * c * ES);
        r.k[NC + c] = load16(kb + 32 * c * ES);
      }
    }
  };
  auto load_v = [&](StepRegs<D>& r, const StepInfo& si) { load_rows(r.v, si, 1); };

  // Write the staged piece results: every store instruction covers 1 KB of contiguous memory
  // (the G rows of one (sequence, KV head) are adjacent in the output and in a partial slot).
  auto flush = [&](bool drain) {
    wave_lds_sync();
    const int n4 = G * D / 4;
    for (int e = 0; e < ring_n; ++e) {
      const float* so = rdat + (size_t)e * EF;
      const int64_t dst = uni(rhdr[2 * e]);
      const int64_t tag = uni(rhdr[2 * e + 1]);
      const int kind = (int)(tag & 3);
      if (kind == 2 && lane < G) {
        const int64_t slot = tag >> 2;
        store_nt(p.ws_m + slot * G + lane, so[G * D + lane]);
        store_nt(p.ws_l + slot * G + lane, so[G * D + G + lane]);
      } else if (kind != 2 && p.lse && lane < G) {
        store_nt(p.lse + dst / D + lane, so[G * D + lane]);
      }
#pragma unroll
      for (int k = 0; k < (16 * D / 4) / 64; ++k) {
        const int e4 = lane + 64 * k;
        if (e4 < n4) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(so + 4 * e4);
          if (kind == 0) {
            store_nt(reinterpret_cast<float*>(p.out) + dst + 4 * e4, o);
          } else if (kind == 1) {
            const uint32_t w0 = (uint32_t)Elem<T>::from_f32(o[0]) |
                                ((uint32_t)Elem<T>::from_f32(o[1]) << 16);
            const uint32_t w1 = (uint32_t)Elem<T>::from_f32(o[2]) |
                                ((uint32_t)Elem<T>::from_f32(o[3]) << 16);
            store_nt(reinterpret_cast<uint16_t*>(p.out) + dst + 4 * e4, u32x2{w0, w1});
          } else {
            store_nt(p.ws_acc + dst + 4 * e4, o);
          }
        }
      }
    }
    ring_n = 0;
    // Inside the loop (ring full, rare) wait for the stores right here, so that no store is
    // pending when the next vector-load wait comes; the s_waitcnt immediate is vmcnt(0) with
    // the other counters left free.
    if (drain) __builtin_amdgcn_s_waitcnt(0x0F70);
    wave_lds_sync();
  };

  // Start of a step: open a new piece.
  auto begin_step = [&](const StepInfo& si) {
    if (starts_piece(si)) {
      m_run = kNegInf;
      l_run = 0.f;
      poison = false;
      piece_rfirst = si.rfirst;
      piece_k0 = si.k;
#pragma unroll
      for (int f = 0; f < NF; ++f) oacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Step si from buffer r; the loads of step nx (two steps ahead) go into r as soon as each
  // part of r has been consumed: K once its rows are in LDS, Q after the score MFMAs, V once its
  // rows are in LDS. The softmax and P.V of this step then run with two steps of loads in
  // flight.
  auto compute_step = [&](StepRegs<D>& r, const StepInfo& si, const StepInfo& nx) {
    const int nvalid = si.L - 32 * si.k;             // valid tokens in this step (>= 1)
    poison = poison || !valid_block(si.b0, p.num_blocks) ||
             (B == 16 && nvalid > 16 && !valid_block(si.b1, p.num_blocks));
    // key rows into the LDS tile, then back as the score MFMA's A operands
    u32x4 kop[2][NC];
    if constexpr (STREAM) {
      wave_lds_sync();   // the previous step's transposed reads come first
#pragma unroll
      for (int f = 0; f < NF; ++f) *reinterpret_cast<u32x4*>(vstage + kw_ofs[f]) = r.k[f];
      load_k(r, nx);
      wave_lds_sync();
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          kop[a][c] = *reinterpret_cast<const u32x4*>(vstage + kr_ofs[a][c]);
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NC; ++c) kop[a][c] = r.k[NC * a + c];
    }
    f32x4 sacc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[a] = mfma16x16x32<T>(kop[a][c], r.q[c], sacc[a]);
    }
    if constexpr (!STREAM) load_k(r, nx);
    load_q(r, nx);
    // value rows into the LDS tile (over the key rows, whose reads come first, and the previous
    // step's transposed reads), then back as A operands (head-dim column 16f + lane%16, tokens
    // 8*(lane/16) .. +8 of the step)
    wave_lds_sync();
#pragma unroll
    for (int f = 0; f < NF; ++f) *reinterpret_cast<u32x4*>(vstage + vw_ofs[f]) = r.v[f];
    load_v(r, nx);
    wave_lds_sync();
    u32x4 va[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint2 lo = lds_read_tr16(vstage + (vr_ofs[0] ^ (f << 5)));
      const uint2 hi = lds_read_tr16(vstage + (vr_ofs[1] ^ (f << 5)));
      va[f] = u32x4{lo.x, lo.y, hi.x, hi.y};
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
    for (int t = 1; t < 8; ++t) mx = fmaxf(mx, z[t]);
    mx = cross_max<16>(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float pr[8];
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      pr[t] = fast_exp2(z[t] - m_new);
      ps += pr[t];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int f = 0; f < NF; ++f) oacc[f] *= alpha;

    u32x4 phi, plo;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t h, l;
      split_pair<T>(pr[2 * u], pr[2 * u + 1], h, l);
      phi[u] = h;
      plo[u] = l;
    }
    if (nvalid < 32) {
      // zero the value entries of slots past the context (they may hold anything)
      const int nv = nvalid - vtok;
      u32x4 msk;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        msk[u] = (2 * u < nv ? 0xffffu : 0u) | (2 * u + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
      for (int f = 0; f < NF; ++f) va[f] &= msk;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      oacc[f] = mfma16x16x32<T>(va[f], phi, oacc[f]);
      oacc[f] = mfma16x16x32<T>(va[f], plo, oacc[f]);
    }

    // End of a piece: stage the output (whole segment, normalised) or the partial state.
    if (si.rlast || si.k == si.ns - 1) {
      float l_tot = cross_sum<16>(l_run);
      if (poison) l_tot = __builtin_nanf("");
      const bool whole = piece_k0 == 0 && si.k == si.ns - 1;
      const float so_scale = whole ? (l_tot == 0.f ? 0.f : 1.0f / l_tot) : 1.f;
      float* so = rdat + (size_t)ring_n * EF;
      if (r16 < G) {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          *reinterpret_cast<f32x4*>(so + r16 * D + 16 * f + 4 * jg) = oacc[f] * so_scale;
        if (!whole && jg == 0) {
          so[G * D + r16] = m_run;
          so[G * D + G + r16] = l_tot;
        } else if (whole && jg == 0 && p.lse) {
          so[G * D + r16] = l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
        }
      }
      if (lane == 0) {
        if (whole) {
          rhdr[2 * ring_n] = ((int64_t)si.s * p.num_q_heads + (int64_t)si.g * G) * D;
          rhdr[2 * ring_n + 1] = p.out_f32 ? 0 : 1;
        } else {
          const int64_t slot = (int64_t)piece_slot(si.range, piece_rfirst);
          rhdr[2 * ring_n] = slot * G * D;
          rhdr[2 * ring_n + 1] = (slot << 2) | 2;
        }
      }
      if (++ring_n == R) flush(true);
    }
  };

  // Software pipeline over two register buffers: while step i computes, the loads of step
  // i + 1 are in flight and those of step i + 2 are issued into the parts of step i's buffer
  // that are consumed (inside compute_step); the block ids of the step after that are being
  // fetched (scalar loads). Past the last step the stream repeats it, flagged past (its loads
  // hit cached query lines), which keeps every vector load unconditional. The loop runs over
  // pairs of steps with its only exit at the bottom, so the compiler's wait counts stay exact;
  // an odd last step is finished after it.
  StepRegs<D> BA, BB;
  StepInfo sa = ss.next();
  StepInfo sb = ss.next();
  load_q(BA, sa);
  load_k(BA, sa);
  load_v(BA, sa);
  load_q(BB, sb);
  load_k(BB, sb);
  load_v(BB, sb);
  StepInfo sc = ss.next();
  for (int64_t i = 0; i + 2 <= nsteps; i += 2) {
    // BA: step i (sa); BB: step i + 1 (sb); sc describes step i + 2
    begin_step(sa);
    compute_step(BA, sa, sc);
    const StepInfo sd = ss.next();
    begin_step(sb);
    compute_step(BB, sb, sd);
    sa = sc;
    sb = sd;
    sc = ss.next();
  }
  if (nsteps & 1) {
    begin_step(sa);
    StepInfo none = sa;         // loads issued for no step: cached lines, never used
    none.past = true;
    compute_step(BA, sa, none);
  }
  flush(false);
}

template <typename T, int D, int B>
static int resident_t(int waves, size_t lds) {   // lds: dynamic bytes for this many waves
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (waves) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_mfma<T, D, B, 1>, 64, lds); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_mfma<T, D, B, 2>, 128, lds); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_mfma<T, D, B, 4>, 256, lds); break;
    default: break;
  }
  return e == hipSuccess ? blocks * waves : 0;
}

int decode_mfma_resident_waves(int kv_dtype, int head_dim, int block_size, int group, int waves,
                               int num_seqs) {
  const size_t lds = mfma_lds_bytes(num_seqs, group, head_dim, waves);
  const bool bf = kv_dtype == 2;
#define PKV_CASE(D, B)                                                                   \
  if (head_dim == D && block_size == B)                                                  \
    return bf ? resident_t<bf16_t, D, B>(waves, lds) : resident_t<f16_t, D, B>(waves, lds);
  PKV_CASE(64, 16)
  PKV_CASE(64, 32)
  PKV_CASE(128, 16)
  PKV_CASE(128, 32)
#undef PKV_CASE
  return 0;
}

template <typename T, int D, int B>
static hipError_t launch_t(const DecodeParams& p, int waves, hipStream_t st) {
  const int grid = (p.num_workers + waves - 1) / waves;
  if (grid <= 0) return hipSuccess;
  const size_t lds = mfma_lds_bytes(p.num_seqs, p.num_q_heads / p.num_kv_heads, D, waves);
  switch (waves) {
    case 1: launch_kernel((decode_mfma<T, D, B, 1>), dim3(grid), dim3(64), lds, st, p); break;
    case 2: launch_kernel((decode_mfma<T, D, B, 2>), dim3(grid), dim3(128), lds, st, p); break;
    case 4:
      if (p.stream_loads)
        launch_kernel((decode_mfma<T, D, B, 4>), dim3(grid), dim3(256), lds, st, p);
      else
        launch_kernel((decode_mfma<T, D, B, 4, false>), dim3(grid), dim3(256), lds, st, p);
      break;
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
