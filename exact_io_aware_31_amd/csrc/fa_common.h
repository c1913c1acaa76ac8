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

// Max / sum of x over lanes l and l ^ 32 (the two halves of the wave), via
// v_permlane32_swap on (x, x): afterwards lanes 0-31 hold (own, partner) and
// lanes 32-63 hold (partner, own), so no lane-dependent select is needed and
// both lanes of a pair get the same result (max and + are commutative).
__device__ __forceinline__ float half_pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
#define FA_VMCNT(n) ((((n) & 15) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14)))
// ... and additionally until every LDS operation of this wave has completed.
#define FA_VMCNT_LGKM0(n) (FA_VMCNT(n) & ~(15 << 8))

// Wait on this wave's outstanding counters.  The empty asm statements with a
// memory clobber keep the compiler from moving LDS accesses across the wait
// (the builtin alone is not a memory barrier to the compiler).
template <int IMM>
__device__ __forceinline__ void wait_counts() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(IMM);
  asm volatile("" ::: "memory");
}
// Makes the kernel arguments given load at the kernel's start.  The compiler
// loads an argument with a scalar load just before its first use; one still
// outstanding when a kernel's main loop starts makes it wait for every LDS
// read at the first LDS wait of each iteration (scalar and LDS loads share
// one counter, and scalar loads may return out of order).
template <typename X>
__device__ __forceinline__ void load_arg_now(X x) {
  asm volatile("" ::"s"(x));
}
template <typename... A>
__device__ __forceinline__ void load_args_now(A... a) {
  (load_arg_now(a), ...);
}

// Workgroup barrier without the memory fence of __syncthreads() (the fence
// waits for every outstanding memory operation of the wave, including loads
// issued for later tiles); the memory clobbers keep every LDS access on its
// side of the barrier.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Work item of workgroup p in a grid of nheads x nblk items, where block rank
// 0 of a head is its heaviest.  The hardware deals workgroups round-robin
// over the 8 XCDs (p mod 8), and items are mapped so that each XCD works on
// its own heads (their K and V are read through its L2):
//   * uneven blocks (causal, no window) and heads that split evenly over the
//     XCDs: an XCD runs its heads' blocks rank-major, every head's heaviest
//     block first, then every head's next one, so the lightest blocks of all
//     its heads fill the end (head-major leaves heavy blocks of the last
//     heads starting late);
//   * otherwise, when the grid splits evenly over the XCDs: head-major over
//     a contiguous range of items per XCD, which keeps fewer heads' K and V
//     in its L2 at a time;
//   * else items in plain order.
__device__ __forceinline__ void work_item(int p, int nheads, int nblk, bool uneven, int& head,
                                          int& rank) {
  if (uneven && nheads % 8 == 0) {
    const int hpx = nheads / 8, local = p / 8;
    head = (p % 8) * hpx + local % hpx;
    rank = local / hpx;
  } else {
    const int total = nheads * nblk;
    const int w = (total % 8 == 0) ? (p % 8) * (total / 8) + p / 8 : p;
    head = w / nblk;
    rank = w % nblk;
  }
}

// Round 8 floats to the storage type (round to nearest even).
template <typename T>
__device__ __forceinline__ typename Vec<T>::v8 to_v8(const float* x) {
  typename Vec<T>::v8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)x[i];
  return r;
}

// The 8 values of a packed vector as floats (exact).  For bfloat16 this is a
// shift or a mask per value, done on the packed words so the compiler does not
// round each value separately to recover it.
__device__ __forceinline__ void from_v8(bf16x8 v, float* x) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void from_v8(f16x8 v, float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}

}  // namespace fa
