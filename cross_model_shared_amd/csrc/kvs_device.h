// Device-side building blocks shared by the gfx950 kernels: vector types, the
// pool tile addressing, matrix-core steps and the online-softmax update.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
// bits OR-ed into the caller's device status word (values of the C ABI enum)
constexpr int KVS_DEV_BAD_PAGE_BIT = 1;
constexpr int KVS_DEV_BAD_LEN_BIT = 2;
constexpr int KVS_DEV_ALIAS_BIT = 4;

// Element offset of the (layer, page, head) tile: K part (16*D) then V part (16*D).
__device__ __forceinline__ int64_t tile_offset(int layer, int page, int head, int num_pages,
                                               int num_kv_heads, int D) {
  return ((int64_t(layer) * num_pages + page) * num_kv_heads + head) * int64_t(32 * D);
}

// Tile geometry in 16-byte units: a K part of 2*D runs (run (i, kg, t) = 8 head
// dims 32i+8kg.. of slot t at index 64i + 16kg + t), then a V part of 2*D runs
// (run (s, o, m) = slots 8o..8o+7 of head dim 16s+m at index 2*D + 32s + 16o + m).
__device__ __forceinline__ constexpr int k_run(int i, int kg, int t) { return 64 * i + 16 * kg + t; }
__device__ __forceinline__ constexpr int v_run(int D, int s, int o, int m) { return 2 * D + 32 * s + 16 * o + m; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i16x4 as_i16x4(u32x2 v) { return __builtin_bit_cast(i16x4, v); }

// C += A(16x32) * B(32x16), bf16 in, fp32 accumulate.
__device__ __forceinline__ f32x4 mma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// C += A(16x16) * B(16x16), bf16 in, fp32 accumulate.
__device__ __forceinline__ f32x4 mma_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(a), as_i16x4(b), c, 0, 0, 0);
}

// Pack four fp32 into four bf16 (round to nearest even) as two dwords.
__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return __builtin_bit_cast(u32x2, v);
}

// Reductions over lanes l, l^16, l^32, l^48 (the four lane groups that hold one
// row of a 16x16 matrix-core result).  gfx950's row swaps exchange 16-lane rows
// (permlane16) and 32-lane halves (permlane32) between two registers; with both
// operands equal, the element-wise max/sum of the two results is the pairwise
// reduction, in plain VALU instructions.
__device__ __forceinline__ float wave_max_across_quads(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_across_quads(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x on the transcendental unit (no subnormal range handling: results below
// 2^-126 flush to zero, which a softmax weight can afford).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Zero the entries of slots >= nvalid in 4 consecutive slots first..first+3 of
// one head-dim value (8 bytes).  Slots past a session's end may hold anything,
// NaN included, and 0 * NaN would poison PV.
__device__ __forceinline__ u32x2 mask_v_quad(u32x2 v, int first, int nvalid) {
  v[0] &= (first + 0 < nvalid ? 0x0000FFFFu : 0u) | (first + 1 < nvalid ? 0xFFFF0000u : 0u);
  v[1] &= (first + 2 < nvalid ? 0x0000FFFFu : 0u) | (first + 3 < nvalid ? 0xFFFF0000u : 0u);
  return v;
}
// The same for 8 consecutive slots first..first+7 (16 bytes).
__device__ __forceinline__ u32x4 mask_v_run(u32x4 v, int first, int nvalid) {
  const u32x2 lo = mask_v_quad(u32x2{v[0], v[1]}, first, nvalid);
  const u32x2 hi = mask_v_quad(u32x2{v[2], v[3]}, first + 4, nvalid);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Load through the constant address space: with a wave-uniform address this is
// a scalar load (lgkmcnt), which keeps it out of the vector-memory counter that
// paces the LDS ring.  Only for data that no kernel of the call writes.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ void flag_error(int32_t* dev_status, int bits) {
  if (dev_status) atomicOr(dev_status, bits);
}

}  // namespace kvs
