// Split-K merge of per-partition partial states into the attention output, with the
// log-sum-exp rule of "Paged Attention and vLLM", section "Paged Attention CUDA Kernel":
//   m* = max_k m_k,  o = sum_k 2^(m_k - m*) acc_k / sum_k 2^(m_k - m*) l_k
// (the partial states keep m in the log2 domain). One workgroup per (sequence, query head),
// one thread per head-dim element. Sequences that fit one partition were finalised by the
// decode kernel and are skipped here.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

template <int D, typename T>
__global__ __launch_bounds__(D) void splitk_reduce(DecodeParams p) {
  const int orow = blockIdx.x;                 // s * Hq + h
  const int s = orow / p.num_q_heads;
  int L = p.lens[s];
  const int cap = min(p.max_blocks * p.block_size, p.n_part_max * p.partition);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int n_part = L > 0 ? ceil_div(L, p.partition) : 1;
  if (n_part <= 1) return;
  const int d = threadIdx.x;
  const size_t base = (size_t)orow * p.n_part_max;
  const float* wm = p.ws_m + base;
  const float* wl = p.ws_l + base;
  const float* wa = p.ws_acc + base * D + d;
  float m_star = kNegInf;
  for (int k = 0; k < n_part; ++k) m_star = fmaxf(m_star, wm[k]);
  float num = 0.f, den = 0.f;
  for (int k = 0; k < n_part; ++k) {
    const float c = fast_exp2(wm[k] - m_star);
    num = fmaf(c, wa[(size_t)k * D], num);
    den = fmaf(c, wl[k], den);
  }
  const float o = den == 0.f ? 0.f : num / den;
  if (p.out_f32) {
    reinterpret_cast<float*>(p.out)[(size_t)orow * D + d] = o;
  } else {
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<uint16_t*>(p.out)[(size_t)orow * D + d] = Elem<T>::from_f32(o);
  }
}

hipError_t launch_splitk_reduce(const DecodeParams& p, int kv_dtype, int head_dim,
                                hipStream_t st) {
  const int64_t grid = (int64_t)p.num_seqs * p.num_q_heads;
  if (grid <= 0 || p.n_part_max <= 1) return hipSuccess;
#define PKV_RED(D, T) \
  hipLaunchKernelGGL((splitk_reduce<D, T>), dim3((unsigned)grid), dim3(D), 0, st, p)
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
