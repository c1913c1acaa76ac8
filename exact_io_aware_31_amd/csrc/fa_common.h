// fa_common.h -- device types and helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (CDNA4 wave64):
//   v_mfma_f32_32x32x16_{bf16,f16}:  D[32x32] += A[32x16] * B[16x32]
//     lane l (h = l / 32) supplies A[l % 32][8h .. 8h+7] and B[8h .. 8h+7][l % 32];
//     accumulator register r of lane l holds D[8 (r / 4) + 4 h + (r % 4)][l % 32].
//   Any consistent permutation of the 16 reduction indices between A and B
//   gives the same product; the kernels use that freedom so an accumulator
//   can be fed back as a B operand without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Vec;
template <> struct Vec<__bf16> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Vec<_Float16> { typedef f16x8 v8; typedef f16x4 v4; };

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Value held by lane l ^ 32 (the other half of the wave), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0-31 receive lane l+32's value in r[1]; lanes 32-63 receive lane l-32's in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load / store helpers (dwordx4).
template <typename V>
__device__ __forceinline__ V ld16(const void* p) {
  return __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(p));
}
template <typename V>
__device__ __forceinline__ void st16(void* p, V v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

// Round 8 floats to the storage type (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 to_v8(const float* x) {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)x[i];
  return r;
}

}  // namespace fa
