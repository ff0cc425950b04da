// Block swap between the device pools and a host pool of the same block shape ("Paged
// Attention and vLLM", section "Continuous Batching and Scheduler": the blocks of a preempted
// sequence move to CPU memory block by block and come back when it resumes).
//
// One launch moves a whole list of blocks. The host pool is pinned memory mapped into the
// GPU's address space, so the kernel reads or writes it directly across the host link: no
// staging copy in HBM and no DMA call per block. A block of one pool is one contiguous run of
// H_kv * B * d elements. A (pair, chunk) item is up to 16 KiB of keys and 16 KiB of values of
// one pair, moved in 16-byte accesses; each lane issues its eight loads before its stores, and
// each wave instruction covers one contiguous KiB. Pairs with an id outside its pool are
// skipped (never dereferenced). The same kernel gathers blocks into (or scatters them out of) a
// contiguous device staging buffer for the copy-engine variant, whose host side is one DMA
// copy per pool (no id list on the staging side: pair i is staging block i).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

constexpr int kSwapThreads = 256;
constexpr int kSwapUnits = 4;   // 16-byte units per lane per pool
constexpr int kSwapChunk = kSwapThreads * kSwapUnits;

// Moves units [c0, c0 + kSwapChunk) of one block of each pool. All eight loads of a lane are
// issued before its first store. kFull: the whole chunk lies inside the block, nothing is
// guarded. Otherwise an index past the block re-reads its last unit and only the stores are
// guarded.
template <bool kFull>
__device__ __forceinline__ void move_chunk(const u32x4* __restrict__ sk,
                                           const u32x4* __restrict__ sv, u32x4* __restrict__ dk,
                                           u32x4* __restrict__ dv, int c0, int U) {
  const int base = c0 + (int)threadIdx.x;
  u32x4 kx[kSwapUnits], vx[kSwapUnits];
#pragma unroll
  for (int k = 0; k < kSwapUnits; ++k) {
    const int u = kFull ? base + k * kSwapThreads : min(base + k * kSwapThreads, U - 1);
    kx[k] = sk[u];
    vx[k] = sv[u];
  }
#pragma unroll
  for (int k = 0; k < kSwapUnits; ++k) {
    const int u = base + k * kSwapThreads;
    if (kFull || u < U) {
      dk[u] = kx[k];
      dv[u] = vx[k];
    }
  }
}

__global__ __launch_bounds__(kSwapThreads) void block_copy_kernel(SwapParams p, int chunks) {
  const int items = p.num_pairs * chunks;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int pair = it / chunks;
    const int chunk = it - pair * chunks;
    const int s = p.src_ids ? p.src_ids[pair] : pair;   // no list: block i of a staging buffer
    const int d = p.dst_ids ? p.dst_ids[pair] : pair;
    if ((unsigned)s >= (unsigned)p.src_count || (unsigned)d >= (unsigned)p.dst_count) continue;
    const int U = p.units;
    const u32x4* sk = reinterpret_cast<const u32x4*>(p.src_k) + (size_t)s * U;
    const u32x4* sv = reinterpret_cast<const u32x4*>(p.src_v) + (size_t)s * U;
    u32x4* dk = reinterpret_cast<u32x4*>(p.dst_k) + (size_t)d * U;
    u32x4* dv = reinterpret_cast<u32x4*>(p.dst_v) + (size_t)d * U;
    const int c0 = chunk * kSwapChunk;
    if (c0 + kSwapChunk <= U)
      move_chunk<true>(sk, sv, dk, dv, c0, U);
    else
      move_chunk<false>(sk, sv, dk, dv, c0, U);
  }
}

// The host link, not the device, bounds a swap: 8 to 16 workgroups already keep enough 16-byte
// accesses in flight to reach it. The grid is one workgroup per compute unit, looping over
// (pair, chunk) items. With decode running on another stream meanwhile, an even spread of one
// workgroup per CU slows every decode worker alike; a smaller grid sits on some CUs only and
// stretches the static decode schedule more (measured: decode 277 us with one workgroup per CU,
// 313-334 us with 32-64 workgroups, 182 us alone).
hipError_t launch_block_copy(const SwapParams& p, int num_cus, hipStream_t st) {
  if (p.num_pairs <= 0 || p.units <= 0) return hipSuccess;
  const int chunks = (p.units + kSwapChunk - 1) / kSwapChunk;
  const int64_t items = (int64_t)p.num_pairs * chunks;
  if (items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int grid = (int)std::min<int64_t>(items, std::max(num_cus, 1));
  launch_kernel(block_copy_kernel, dim3(grid), dim3(kSwapThreads), 0, st, p, chunks);
  return hipGetLastError();
}

}  // namespace pkv
