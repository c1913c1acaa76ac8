// fa_probe.hip -- the two measurement kernels of libfa_probe (include/fa_probe.h):
// the dense bf16 matrix-core rate with the shader clock under that load, and
// the streaming HBM read rate.  They bound what any kernel of libfa can reach
// on the chip in hand (the compute roof and the bandwidth roof of a roofline).
#include "fa_common.h"
#include "fa_launch.h"
#include "fa_probe_launch.h"
#include "../../include/fa_probe.h"

namespace fa_probe {

using fa::bf16x8;
using fa::f32x16;
using fa::u32x4;

// A pseudo-random value in [-1, 1) with a full mantissa: the matrix cores'
// power draw, and so the clock they sustain, depends on how many operand bits
// switch, so the probe's operands look like attention data (N(0,1)-like bf16
// values), not like small round numbers.
__device__ __forceinline__ float probe_value(uint32_t x) {
  x = x * 2654435761u + 0x9e3779b9u;
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  return (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;
}

// Four independent accumulate chains per wave, operands in registers.  The
// empty asm statements order the clock reads around the loop: the first
// makes the loop's operand depend on an instruction issued after the first
// reads, the second consumes the loop's result before the last reads.
__global__ __launch_bounds__(FA_PROBE_THREADS) void mfma_probe_kernel(float* __restrict__ out,
                                                                      unsigned long long* __restrict__ stamps,
                                                                      int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)probe_value((uint32_t)(blockIdx.x * 4096 + tid * 16 + i));
    b[i] = (__bf16)probe_value((uint32_t)(blockIdx.x * 4096 + tid * 16 + 8 + i) ^ 0x5bd1e995u);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  asm volatile("" : "+v"(a));
  for (int i = 0; i < iters; ++i) {
    c0 = fa::mfma32x32x16(a, b, c0);
    c1 = fa::mfma32x32x16(a, b, c1);
    c2 = fa::mfma32x32x16(a, b, c2);
    c3 = fa::mfma32x32x16(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  asm volatile("" ::"v"(s));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * FA_PROBE_THREADS + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
    stamps[0] = t0;
    stamps[1] = r0;
    stamps[2] = t1;
    stamps[3] = r1;
  }
}

// Chunk c covers 16-byte elements c * 4096 .. c * 4096 + 4095; lane t of a
// workgroup loads elements t + 256 u, u = 0..15, so every load instruction of
// a wave reads 1 KiB of consecutive bytes.  Workgroup b reads the contiguous
// run of chunks b * cpb .. b * cpb + cpb - 1 (cpb = ceil(chunks / workgroups)),
// as a decode workgroup streams its own part of a history.
constexpr int kLoads = FA_PROBE_READ_CHUNK / (16 * FA_PROBE_THREADS);
static_assert(kLoads == 16, "sixteen 16-byte loads per lane per chunk");

__global__ __launch_bounds__(FA_PROBE_THREADS) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                                       size_t nchunks,
                                                                       unsigned* __restrict__ out) {
  const int tid = threadIdx.x;
  const size_t cpb = (nchunks + gridDim.x - 1) / gridDim.x;
  const size_t c0 = (size_t)blockIdx.x * cpb;
  const size_t c1 = c0 + cpb < nchunks ? c0 + cpb : nchunks;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = c0; c < c1; ++c) {
    const u32x4* __restrict__ p = buf + c * (size_t)(kLoads * FA_PROBE_THREADS) + tid;
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) v[u] = __builtin_nontemporal_load(p + u * FA_PROBE_THREADS);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u];
  }
  out[(size_t)blockIdx.x * FA_PROBE_THREADS + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

hipError_t launch_mfma(float* out, unsigned long long* stamps, int blocks, int iters,
                       hipStream_t s) {
  return fa::launch_kernel(mfma_probe_kernel, dim3(blocks), dim3(FA_PROBE_THREADS), s, out, stamps,
                           iters);
}

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* out, int blocks,
                              hipStream_t s) {
  return fa::launch_kernel(stream_read_kernel, dim3(blocks), dim3(FA_PROBE_THREADS), s,
                           static_cast<const u32x4*>(buf), bytes / FA_PROBE_READ_CHUNK, out);
}

}  // namespace fa_probe
