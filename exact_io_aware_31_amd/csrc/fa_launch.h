// fa_launch.h -- host-side launchers for the gfx950 attention kernels.
// Arguments are validated by the C ABI layer (fa_api.cpp) before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

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

// Workspace layouts (bytes), shared by the size queries and the launchers.
size_t bwd_drow_bytes(int B, int H, int N);
size_t decode_part_o_bytes(int B, int H, int d, int splits);
size_t decode_part_lse_bytes(int B, int H, int splits);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace fa
