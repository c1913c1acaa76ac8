// fa_launch.h -- host-side launchers for the gfx950 attention kernels.
// Arguments are validated by the C ABI layer (fa_api.cpp) before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <tuple>
#include <utility>

namespace fa {

// Launch `kernel` on stream s and return the runtime's verdict on this launch
// alone.  hipLaunchKernel reports the launch's own error; reading it back
// with hipGetLastError() after a triple-chevron launch would also return
// (and clear) an error an earlier, unrelated call of the same thread left.
// The arguments are converted to the kernel's parameter types first.
template <typename... Params, size_t... I>
hipError_t launch_packed(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         std::tuple<Params...>& p, std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(p))..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, s);
}
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t s,
                         Args&&... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> p(std::forward<Args>(args)...);
  return launch_packed(kernel, grid, block, s, p, std::index_sequence_for<Params...>{});
}

enum class DType { F16 = 0, BF16 = 1 };

struct FwdArgs {
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  int B, H, N, d;
  int Hkv;         // key/value heads; H is a multiple of Hkv
  int window;      // 0 = none; else (causal) key j visible to query i iff i - window < j <= i
  float scale;
  bool causal;
  DType dt;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* o;
  const float* lse; const void* dout;
  void* dq; void* dk; void* dv;
  float* drow;     // [B,H,N] float32 workspace
  int B, H, N, d;
  int Hkv;         // key/value heads (k, v, dk, dv are [B,Hkv,N,d])
  int window;      // as in FwdArgs
  float scale;
  bool causal;
  DType dt;
};

struct DecodeArgs {
  const void* q; const void* k; const void* v;
  void* o; float* lse;      // lse may be null
  float* part_o;            // [B,H,S,d] float32 workspace
  float* part_lse;          // [B,H,S] float32 workspace
  int B, H, Nkv, d, splits;
  int Hkv;                  // key/value heads (k, v are [B,Hkv,Nkv,d])
  const int* kv_lens;       // device int32 [B] history lengths, or null (all Nkv)
  float scale;
  DType dt;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Device address of fa_decode_noalloc's static scratch on the current device
// (FA_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), looked up on the first
// call per device.
hipError_t noalloc_scratch(void** ptr);

// Workspace layouts (bytes), shared by the size queries and the launchers:
// the backward's float32 row terms D [B, H, N]; the decode's float32 partial
// outputs [B, H, splits, d], then partial log-sum-exps [B, H, splits]; each
// part rounded up to 256 bytes.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bwd_drow_bytes(int B, int H, int N) {
  return align256((size_t)B * H * N * sizeof(float));
}
inline size_t decode_part_o_bytes(int B, int H, int d, int splits) {
  return align256((size_t)B * H * splits * d * sizeof(float));
}
inline size_t decode_part_lse_bytes(int B, int H, int splits) {
  return align256((size_t)B * H * splits * sizeof(float));
}

}  // namespace fa
