// Cache mutations: bitwise stores of new tokens into their slots, and copy-on-write of the
// valid slots of a shared block.
//
// Append ("PagedAttention: Virtual Memory for the KV Cache", section "Growing a request";
// "Paged Attention and vLLM", section "KV Cache Fundamentals"): token i of sequence
// seq_ids[i] at position positions[i] goes to block table[seq][pos / B], offset pos % B.
// Copy-on-write (first page, section "Sharing a prefix and copying a partial block"; second
// page, the copy-on-write rule under "Continuous Batching and Scheduler"): slots [0, n) of
// every KV head, keys and values, from block src to block dst.
// Out-of-range sequence ids, positions or block ids are skipped (never dereferenced).
#include "device_common.h"
#include "kernels.h"

namespace pkv {

// One thread per E-sized unit of a new row (E = 16 bytes when every pointer allows it, else
// the element). Keys and values share the layout, so row (i, g) of k_new / v_new lands in one
// contiguous row of its block: the writes of a token are whole cache lines. The new rows are
// loaded before the slot lookup (they do not depend on it), so a thread waits for two rounds
// of memory latency: ids, position and row data, then the table entry. 32-bit index
// arithmetic (the host checks num_tokens * H * units < 2^31).
template <typename E>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p, int units_per_row) {
  const int U = units_per_row, B = p.block_size, H = p.num_kv_heads;
  const int total = p.num_tokens * H * U;
  E* kp = reinterpret_cast<E*>(p.k_pool);
  E* vp = reinterpret_cast<E*>(p.v_pool);
  const E* kn = reinterpret_cast<const E*>(p.k_new);
  const E* vn = reinterpret_cast<const E*>(p.v_new);
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += gridDim.x * blockDim.x) {
    const int t = idx / U;            // (token, head) row
    const int u = idx - t * U;
    const int i = t / H;
    const int g = t - i * H;
    const E kx = kn[idx];
    const E vx = vn[idx];
    const int s = p.seq_ids[i];
    const int pos = p.positions[i];
    if ((unsigned)s >= (unsigned)p.num_seqs || pos < 0) continue;
    const int j = pos / B;
    if (j >= p.max_blocks) continue;
    const int blk = p.tables[(size_t)s * p.max_blocks + j];
    if ((unsigned)blk >= (unsigned)p.num_blocks) continue;
    const int off = pos - j * B;
    const size_t row = ((size_t)blk * H + g) * B + off;
    kp[row * U + u] = kx;
    vp[row * U + u] = vx;
  }
}

template <typename E>
__global__ __launch_bounds__(256) void cow_kernel(CowParams p) {
  const int D = p.head_dim, B = p.block_size, H = p.num_kv_heads;
  const int pair = blockIdx.x / H;
  const int g = blockIdx.x % H;
  const int src = p.src[pair];
  const int dst = p.dst[pair];
  const int n = p.ntok ? p.ntok[pair] : B;
  if ((unsigned)src >= (unsigned)p.num_blocks || (unsigned)dst >= (unsigned)p.num_blocks ||
      src == dst || n < 0 || n > B)
    return;
  E* kp = reinterpret_cast<E*>(p.k_pool);
  E* vp = reinterpret_cast<E*>(p.v_pool);
  const size_t sb = ((size_t)src * H + g) * B * D;
  const size_t db = ((size_t)dst * H + g) * B * D;
  // slots [0, n) are the first n rows of the (block, head) tile, keys and values alike
  for (int e = threadIdx.x; e < n * D; e += blockDim.x) {
    kp[db + e] = kp[sb + e];
    vp[db + e] = vp[sb + e];
  }
}

hipError_t launch_append(const AppendParams& p, int elem_bytes, hipStream_t st) {
  const int row_bytes = p.head_dim * elem_bytes;
  const bool wide = row_bytes % 16 == 0 &&
                    ((reinterpret_cast<uintptr_t>(p.k_pool) | reinterpret_cast<uintptr_t>(p.v_pool) |
                      reinterpret_cast<uintptr_t>(p.k_new) | reinterpret_cast<uintptr_t>(p.v_new)) &
                     15) == 0;
  const int units = wide ? row_bytes / 16 : p.head_dim;
  const int64_t total = (int64_t)p.num_tokens * p.num_kv_heads * units;
  if (total <= 0) return hipSuccess;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (wide)
    launch_kernel(append_kernel<u32x4>, dim3((unsigned)blocks), dim3(256), 0, st, p, units);
  else if (elem_bytes == 4)
    launch_kernel(append_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st, p, units);
  else
    launch_kernel(append_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st, p, units);
  return hipGetLastError();
}

hipError_t launch_cow(const CowParams& p, int elem_bytes, hipStream_t st) {
  const int64_t grid = (int64_t)p.num_pairs * p.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (elem_bytes == 4)
    launch_kernel(cow_kernel<uint32_t>, dim3((unsigned)grid), dim3(256), 0, st, p);
  else
    launch_kernel(cow_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace pkv
