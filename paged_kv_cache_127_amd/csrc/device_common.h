// Device helpers shared by the gfx950 kernels: element types, 16-byte loads, conversions,
// wavefront reductions (DPP within 16-lane rows, cross-row swaps), launch parameter blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct bf16_t { uint16_t bits; };   // storage tag for bfloat16 caches
struct f16_t { uint16_t bits; };    // storage tag for IEEE half caches

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static float to_f32(uint32_t u) { return __uint_as_float(u); }
};
template <> struct Elem<f16_t> {
  static constexpr int kBytes = 2;
  typedef f16x8 mfma_vec;
  __device__ static float to_f32(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
  }
  __device__ static uint16_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  typedef bf16x8 mfma_vec;
  __device__ static float to_f32(uint32_t u) { return __uint_as_float(u << 16); }
  __device__ static uint16_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

// x * s as an fp32 value, then rounded to the 16-bit type T. The empty asm makes the product
// opaque, so the compiler cannot fuse multiply and narrowing into one mixed-precision FMA
// (which rounds once, straight to 16 bits): a 16-bit output is exactly the fp32 output, rounded.
template <typename T>
__device__ __forceinline__ uint16_t scaled_to_16(float x, float s) {
  float y = x * s;
  asm("" : "+v"(y));
  return Elem<T>::from_f32(y);
}

// 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte streaming load (global_load_dwordx4 ... nt): for cache rows a call reads once. On
// gfx950 a gather of random 4 KiB key/value tiles through these reads 6.7 TB/s where plain
// loads of the same tiles reach 5.9 TB/s (contiguous reads: 7.1 vs 6.2 TB/s).
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Result stores (outputs, partial states) are non-temporal: written once, read by another
// kernel at most, so they need not sit dirty in L2 until the end-of-kernel write-back (the
// decode kernel measured 2-3 us shorter on the GQA batch).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_nt(uint16_t* p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

// low / high 16-bit halves of a packed word, widened to fp32
template <typename T> __device__ __forceinline__ float lo16(uint32_t w) {
  return Elem<T>::to_f32(w & 0xffffu);
}
template <typename T> __device__ __forceinline__ float hi16(uint32_t w) {
  return Elem<T>::to_f32(w >> 16);
}

// ---- wavefront data movement ----------------------------------------------------------
// DPP controls (GCN/CDNA encoding)
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i inside each half row
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i inside each row

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Sum over aligned groups of N lanes (N = 2..64); every lane of a group receives the sum.
template <int N> __device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kRowMirror>(v);
  if constexpr (N >= 32) v += xor_lane(v, 16);
  if constexpr (N >= 64) v += xor_lane(v, 32);
  return v;
}

// Max over lanes that differ only in the lane-index bits from FIRST_BIT up to bit 5.
template <int FIRST> __device__ __forceinline__ float cross_max(float v) {
  if constexpr (FIRST <= 1) v = fmaxf(v, dpp<kQuadXor1>(v));
  if constexpr (FIRST <= 2) v = fmaxf(v, dpp<kQuadXor2>(v));
  if constexpr (FIRST <= 4) v = fmaxf(v, xor_lane(v, 4));
  if constexpr (FIRST <= 8) v = fmaxf(v, xor_lane(v, 8));
  if constexpr (FIRST <= 16) v = fmaxf(v, xor_lane(v, 16));
  if constexpr (FIRST <= 32) v = fmaxf(v, xor_lane(v, 32));
  return v;
}
template <int FIRST> __device__ __forceinline__ float cross_sum(float v) {
  if constexpr (FIRST <= 1) v += dpp<kQuadXor1>(v);
  if constexpr (FIRST <= 2) v += dpp<kQuadXor2>(v);
  if constexpr (FIRST <= 4) v += xor_lane(v, 4);
  if constexpr (FIRST <= 8) v += xor_lane(v, 8);
  if constexpr (FIRST <= 16) v += xor_lane(v, 16);
  if constexpr (FIRST <= 32) v += xor_lane(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr float kNegInf = -__builtin_huge_valf();

// ---- launch parameter blocks ----------------------------------------------------------
struct DecodeParams {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  // fused append: token L_s - 1 of every sequence is k_new/v_new[s] ([S][H_kv][D]); the kernel
  // reads that row from there and stores it into its slot (null: plain decode)
  const void* k_new;
  const void* v_new;
  void* k_pool_w;      // the pools, writable (fused append only)
  void* v_pool_w;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;       // [slots][G][D] partial accumulators
  float* ws_m;         // [slots][G]    partial running max (log2 domain)
  float* ws_l;         // [slots][G]    partial running sum
  int64_t* prefix;     // [S + 1] exclusive prefix of steps per sequence
  int64_t* wprefix;    // [S + 1] exclusive prefix of schedule weights per sequence
  // [S][H_q] log2-domain log-sum-exp of each output row, m + log2(l) (-inf for an empty
  // context), written beside the output when set (matrix-core kernel and merge only)
  float* lse;
  // where the merge writes results: out / out_f32, except in shared-prefix mode (pst_m set),
  // where out receives the decode's normalised fp32 rows and the merge folds every segment
  // with the prefix states ([pst_groups][S * H_q] maxima and sums, [..][D] accumulators)
  void* final_out;
  int final_f32;
  const float* pst_m;
  const float* pst_l;
  const float* pst_acc;
  int pst_groups;
  int out_f32;         // 1: fp32 output, 0: output in the cache's 16-bit type
  int max_blocks;
  int max_context_len;   // lengths are clamped to [0, max_context_len]
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;    // KV heads of the schedule: pool KV heads x kv_split
  int kv_split;        // schedule KV heads per pool KV head (>= 1): more query heads per KV
                       // head than one segment takes run as kv_split segments of
                       // num_q_heads / num_kv_heads query heads each over the same KV head
  int pool_kv_heads;   // KV heads of the pools and of k_new / v_new
  int num_blocks;
  int block_size;
  int num_workers;     // wavefronts of the decode kernel
  int piece_weight;    // schedule weight of a segment start (a step weighs 4)
  int stream_loads;    // 1: key/value rows through streaming loads (read once); 0: plain
                       // loads (blocks re-read from the caches; matrix-core kernel with four
                       // wavefronts per workgroup only)
  int ring_cap;        // staged piece results per wavefront (matrix-core kernel)
  float scale_log2;    // softmax scale * log2(e)
};

}  // namespace pkv
