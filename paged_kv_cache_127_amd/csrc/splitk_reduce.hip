// Merge of split segments. A (sequence, KV head) segment whose steps span several worker ranges
// of the decode schedule (schedule.h) left one partial state (m, l, acc) per range; they combine
// with the log-sum-exp rule of "Paged Attention and vLLM", section "Paged Attention CUDA Kernel":
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) acc_k / sum_k 2^(m_k - m*) l_k
// (m is kept in the log2 domain). Segments of empty sequences get a zero row here; segments
// that one range finished were written by the decode kernel and are skipped.
//
// One workgroup per segment, one thread per few output elements. The slots of the segment
// follow from the schedule arithmetic alone; each thread loads (m, l, acc) of four slots at a
// time with independent loads and folds them into a running (max, numerator, denominator), so
// a segment costs one round trip for the prefixes and one per four partials.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace pkv {

constexpr int kMergeBatch = 4;

template <int D, typename T>
__global__ __launch_bounds__(256) void splitk_merge(DecodeParams p) {
  const int Hkv = p.num_kv_heads;
  const int seg = blockIdx.x;
  const int s = seg / Hkv;
  const int g = seg - s * Hkv;
  const int G = p.num_q_heads / Hkv;
  const int64_t ns = p.prefix[s + 1] - p.prefix[s];
  const size_t row0 = (size_t)s * p.num_q_heads + (size_t)g * G;
  const int t = threadIdx.x;
  constexpr int kPer = (16 * D + 255) / 256;   // elements per thread at the largest group (16)

  auto store = [&](int e, float o) {
    const size_t idx = row0 * D + e;
    if (p.out_f32) {
      reinterpret_cast<float*>(p.out)[idx] = o;
    } else {
      if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t*>(p.out)[idx] = Elem<T>::from_f32(o);
    }
  };

  if (ns == 0) {
    for (int e = t; e < G * D; e += blockDim.x) store(e, 0.f);
    return;
  }
  const Line line = Line::make(p.prefix, p.wprefix, p.num_seqs, Hkv, p.piece_weight,
                               p.num_workers);
  const int64_t seg_w = kStepWeight * ns + line.pw;
  const int64_t ws0 = (int64_t)Hkv * p.wprefix[s] + g * seg_w;   // weighted segment start
  const int64_t first = ws0 + line.pw;                            // weighted start of step 0
  const int rf = line.owner(first);
  const int rl = line.owner(first + kStepWeight * (ns - 1));
  if (rf == rl) return;   // one worker wrote the whole segment
  // rf's piece is its first one (slot 2 rf) unless rf also holds the previous segment's last
  // step, which starts at ws0 - kStepWeight
  const int64_t first_slot = 2 * (int64_t)rf + (line.wbegin(rf) > ws0 - kStepWeight ? 0 : 1);

  float M[kPer], num[kPer], den[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    M[q] = kNegInf;
    num[q] = 0.f;
    den[q] = 0.f;
  }
  // Workers rf+1 .. rl start inside the segment: their first piece (slot 2r) belongs to it if
  // they hold any of its steps.
  int64_t before_r = line.in_segment_before(line.wbegin(rf + 1), ws0, ns);
  for (int r0 = rf; r0 <= rl; r0 += kMergeBatch) {
    int64_t slot[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int r = r0 + j;
      slot[j] = -1;
      if (r == rf) {
        slot[j] = first_slot;
      } else if (r <= rl) {
        const int64_t after_r = r == rl ? ns : line.in_segment_before(line.wbegin(r + 1), ws0, ns);
        if (after_r > before_r) slot[j] = 2 * (int64_t)r;
        before_r = after_r;
      }
    }
    float mj[kMergeBatch][kPer], lj[kMergeBatch][kPer], aj[kMergeBatch][kPer];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int e = t + 256 * q;
        mj[j][q] = kNegInf;
        lj[j][q] = 0.f;
        aj[j][q] = 0.f;
        if (slot[j] >= 0 && e < G * D) {
          const int64_t pr = slot[j] * G + e / D;
          mj[j][q] = p.ws_m[pr];
          lj[j][q] = p.ws_l[pr];
          aj[j][q] = p.ws_acc[pr * D + (e % D)];
        }
      }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        if (slot[j] < 0) continue;
        const float m_new = fmaxf(M[q], mj[j][q]);
        if (m_new == kNegInf) continue;
        const float a_old = fast_exp2(M[q] - m_new);
        const float a_new = fast_exp2(mj[j][q] - m_new);
        num[q] = num[q] * a_old + a_new * aj[j][q];
        den[q] = den[q] * a_old + a_new * lj[j][q];
        M[q] = m_new;
      }
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = t + 256 * q;
    if (e < G * D) store(e, den[q] == 0.f ? 0.f : num[q] / den[q]);
  }
}

hipError_t launch_splitk_reduce(const DecodeParams& p, int kv_dtype, int head_dim,
                                hipStream_t st) {
  const int64_t grid = (int64_t)p.num_seqs * p.num_kv_heads;
  if (grid <= 0) return hipSuccess;
#define PKV_RED(D, T) \
  hipLaunchKernelGGL((splitk_merge<D, T>), dim3((unsigned)grid), dim3(256), 0, st, p)
  if (head_dim == 64) {
    if (kv_dtype == 1) PKV_RED(64, f16_t); else if (kv_dtype == 2) PKV_RED(64, bf16_t); else PKV_RED(64, float);
  } else if (head_dim == 128) {
    if (kv_dtype == 1) PKV_RED(128, f16_t); else if (kv_dtype == 2) PKV_RED(128, bf16_t); else PKV_RED(128, float);
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_RED
  return hipGetLastError();
}

}  // namespace pkv
