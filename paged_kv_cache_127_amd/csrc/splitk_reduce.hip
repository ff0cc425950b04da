// Merge of split segments. A (sequence, KV head) segment whose steps span the ranges of
// several workers left one partial state (m, l, acc) per worker (schedule.h gives the slot of
// each); they combine with the log-sum-exp rule of "Paged Attention and vLLM", section
// "Paged Attention CUDA Kernel":
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) acc_k / sum_k 2^(m_k - m*) l_k
// (m is kept in the log2 domain). Segments of empty sequences get a zero row here; segments
// that one worker finished were written by the decode kernel and are skipped.
// One workgroup per segment; threads cover the G x D outputs of its query heads (G <= 16).
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace pkv {

template <int D, typename T>
__global__ __launch_bounds__(256) void splitk_merge(DecodeParams p) {
  const int Hkv = p.num_kv_heads;
  const int seg = blockIdx.x;
  const int s = seg / Hkv;
  const int g = seg - s * Hkv;
  const int G = p.num_q_heads / Hkv;
  const int64_t ps = p.prefix[s];
  const int64_t ns = p.prefix[s + 1] - ps;
  const size_t row0 = (size_t)s * p.num_q_heads + (size_t)g * G;

  auto store = [&](int h, int d, float o) {
    const size_t idx = (row0 + h) * D + d;
    if (p.out_f32) {
      reinterpret_cast<float*>(p.out)[idx] = o;
    } else {
      if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t*>(p.out)[idx] = Elem<T>::from_f32(o);
    }
  };

  if (ns == 0) {
    for (int e = threadIdx.x; e < G * D; e += blockDim.x) store(e / D, e % D, 0.f);
    return;
  }
  const int n = p.num_workers;
  const int64_t N = (int64_t)Hkv * p.prefix[p.num_seqs];
  const int64_t G0 = (int64_t)Hkv * ps + (int64_t)g * ns;
  const int wf = worker_of(N, n, G0);
  const int wl = worker_of(N, n, G0 + ns - 1);
  if (wf == wl) return;
  // the first worker's piece is its last piece (slot 2w+1) unless it also starts its range
  const int first_slot = 2 * wf + (G0 != range_begin(N, n, wf) ? 1 : 0);
  constexpr int kChunk = 256;
  __shared__ int sm_slot[kChunk];
  __shared__ int sm_cnt;
  // per-thread online merge state for its (head, dim) outputs
  constexpr int kPer = (16 * D + 255) / 256;
  float mrun[kPer], num[kPer], den[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    mrun[j] = kNegInf;
    num[j] = 0.f;
    den[j] = 0.f;
  }
  for (int c0 = wf; c0 <= wl; c0 += kChunk) {
    // wavefront 0 lists the slots of the non-empty workers in [c0, c0 + kChunk): workers whose
    // range is empty (more workers than steps) wrote nothing
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int cnt = 0;
      for (int b = c0; b < c0 + kChunk && b <= wl; b += 64) {
        const int w = b + lane;
        const bool ok = w <= wl && range_begin(N, n, w + 1) != range_begin(N, n, w);
        const uint64_t mask = __builtin_amdgcn_ballot_w64(ok);
        if (ok) {
          const int pos = cnt + __popcll(mask & ((1ull << lane) - 1));
          sm_slot[pos] = w == wf ? first_slot : 2 * w;
        }
        cnt += __popcll(mask);
      }
      if (lane == 0) sm_cnt = cnt;
    }
    __syncthreads();
    const int cnt = sm_cnt;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = threadIdx.x + 256 * j;
      if (e >= G * D) break;
      const int h = e / D, d = e - h * D;
      for (int t = 0; t < cnt; ++t) {
        const size_t r = (size_t)sm_slot[t] * G + h;
        const float m = p.ws_m[r];
        if (m == kNegInf) continue;
        const float m_new = fmaxf(mrun[j], m);
        const float a = fast_exp2(mrun[j] - m_new);   // 0 while mrun is still -inf
        const float c = fast_exp2(m - m_new);
        num[j] = num[j] * a + c * p.ws_acc[r * D + d];
        den[j] = den[j] * a + c * p.ws_l[r];
        mrun[j] = m_new;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = threadIdx.x + 256 * j;
    if (e >= G * D) break;
    store(e / D, e % D, den[j] == 0.f ? 0.f : num[j] / den[j]);
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
