// Device-side building blocks shared by the gfx950 attention kernels:
// vector types for the bf16 MFMA operands, 16-byte global/LDS accesses,
// the cross-half lane exchange and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// 16-byte and 8-byte LDS accesses (addresses are element offsets into a
// __shared__ uint16_t array; callers keep them 16- or 8-byte aligned).
__device__ __forceinline__ u32x4 ld_lds16(const uint16_t* base, int elem) {
  return *reinterpret_cast<const u32x4*>(base + elem);
}
__device__ __forceinline__ void st_lds16(uint16_t* base, int elem, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + elem) = v;
}
__device__ __forceinline__ void st_lds8(uint16_t* base, int elem, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + elem) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Combine a lane's value with the one held by lane (l ^ 32). v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; feeding x as both gives {x_lo, x_lo} and {x_hi, x_hi}, so any
// symmetric op of the two results pairs lane l with lane l ^ 32.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// exp2 on the VALU transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two floats to bf16 (nearest-even) and pack them, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace fa
