// fa_api.cpp -- the C ABI declared in include/fa.h.
//
// Every argument is checked here, before any HIP call, so error paths can be
// exercised on a machine without a GPU.  The launchers (fa_fwd.hip,
// fa_bwd.hip, fa_decode.hip) only enqueue kernels on the caller's stream
// (on small grids the backward also on a second stream of its own, forked
// from and joined back into the caller's).
#include "../../include/fa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace {

constexpr long long kMaxElems = 1LL << 40;  // per tensor
constexpr long long kMaxGrid = 0x7fffffffLL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fa_status check_common(int B, int H, int N, int d, float scale, fa_dtype dt) {
  if (dt != FA_F16 && dt != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long elems = (long long)B * H * N * d;
  if (elems > kMaxElems) return FA_ERR_SHAPE;
  // every kernel grid is at most one workgroup per 64 rows or per 32 row-chunks
  if ((long long)B * H * ((N + 63) / 64) > kMaxGrid) return FA_ERR_SHAPE;
  // per-head element offsets are 32-bit inside the kernels
  if ((long long)N * d >= (1LL << 31)) return FA_ERR_SHAPE;
  if (elems / 8 / 256 + 1 > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

fa::DType to_dt(fa_dtype dt) { return dt == FA_BF16 ? fa::DType::BF16 : fa::DType::F16; }

// Shared checks of the grouped-head and window arguments.
fa_status check_ext(int H, int H_kv, int window, int causal) {
  if (H_kv < 1 || H % H_kv != 0) return FA_ERR_SHAPE;
  if (window < 0) return FA_ERR_SHAPE;
  if (window > 0 && !causal) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Checks shared by every decode entry point, apart from the workspace.
fa_status check_decode(const void* q, const void* k, const void* v, void* o, int B, int H,
                       int H_kv, int Nkv, int d, float scale, int num_splits, fa_dtype dt) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  fa_status st = check_common(B, H, Nkv, d, scale, dt);
  if (st != FA_OK) return st;
  if ((st = check_ext(H, H_kv, 0, 0)) != FA_OK) return st;
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if ((long long)B * H * num_splits > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

// Shared body of fa_decode_ex and fa_decode_varlen (kv_lens may be null), and
// of fa_decode_noalloc once its scratch is known.
fa_status decode_impl(const void* q, const void* k, const void* v, const int* kv_lens, void* o,
                      float* lse, int B, int H, int H_kv, int Nkv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes, fa_dtype dt,
                      void* stream) {
  fa_status st = check_decode(q, k, v, o, B, H, H_kv, Nkv, d, scale, num_splits, dt);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < fa_decode_workspace_bytes(B, H, d, num_splits))
    return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             fa::decode_part_o_bytes(B, H, d, num_splits));
  fa::DecodeArgs a{q, k, v, o, lse, part_o, part_lse, B, H, Nkv, d, num_splits, H_kv, kv_lens,
                   scale, to_dt(dt)};
  return fa::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK
                                                                                : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int H_kv, int N, int d, float scale, int causal, int window,
                    fa_dtype dt, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_status st = check_common(B, H, N, d, scale, dt);
  if (st != FA_OK) return st;
  if ((st = check_ext(H, H_kv, window, causal)) != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, H_kv, window >= N ? 0 : window, scale, causal != 0,
                to_dt(dt)};
  return fa::launch_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, fa_dtype dt, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, N, d, scale, causal, 0, dt, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return fa::bwd_drow_bytes(B, H, N);
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N, int d,
                    float scale, int causal, int window, fa_dtype dt, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  fa_status st = check_common(B, H, N, d, scale, dt);
  if (st != FA_OK) return st;
  if ((st = check_ext(H, H_kv, window, causal)) != FA_OK) return st;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  float* drow = static_cast<float*>(workspace);
  fa::BwdArgs a{q,     k,    v, o, lse, dout, dq,   dk, dv, drow, B, H, N, d, H_kv,
                window >= N ? 0 : window, scale, causal != 0, to_dt(dt)};
  return fa::launch_bwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                 fa_dtype dt, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, H, N, d,
                   scale, causal, 0, dt, stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || d < 1 || num_splits < 1) return 0;
  return fa::decode_part_o_bytes(B, H, d, num_splits) + fa::decode_part_lse_bytes(B, H, num_splits);
}

fa_status fa_decode_varlen(const void* q, const void* k, const void* v, const int* kv_lens,
                           void* o, float* lse, int B, int H, int H_kv, int Nkv, int d,
                           float scale, int num_splits, void* workspace, size_t workspace_bytes,
                           fa_dtype dt, void* stream) {
  if (!kv_lens) return FA_ERR_NULL;
  if (!aligned(kv_lens, 4)) return FA_ERR_ALIGN;
  return decode_impl(q, k, v, kv_lens, o, lse, B, H, H_kv, Nkv, d, scale, num_splits, workspace,
                     workspace_bytes, dt, stream);
}

fa_status fa_decode_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int H_kv, int Nkv, int d, float scale, int num_splits,
                       void* workspace, size_t workspace_bytes, fa_dtype dt, void* stream) {
  return decode_impl(q, k, v, nullptr, o, lse, B, H, H_kv, Nkv, d, scale, num_splits, workspace,
                     workspace_bytes, dt, stream);
}

fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int Nkv, int d, float scale, int num_splits,
                            fa_dtype dt, void* stream) {
  fa_status st = check_decode(q, k, v, o, B, H, H_kv, Nkv, d, scale, num_splits, dt);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (lse && !aligned(lse, 4)))
    return FA_ERR_ALIGN;
  void* scratch = nullptr;
  if (fa::noalloc_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  return decode_impl(q, k, v, nullptr, o, lse, B, H, H_kv, Nkv, d, scale, num_splits, scratch,
                     FA_NOALLOC_SCRATCH_BYTES, dt, stream);
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int Nkv, int d, float scale, int num_splits, void* workspace,
                    size_t workspace_bytes, fa_dtype dt, void* stream) {
  return fa_decode_ex(q, k, v, o, lse, B, H, H, Nkv, d, scale, num_splits, workspace,
                      workspace_bytes, dt, stream);
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: bad sizes or scale";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: element type must be FA_F16 or FA_BF16";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointer not aligned as required";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128; a window needs causal";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a kernel launch";
    case FA_ERR_SPLITS: return "FA_ERR_SPLITS: num_splits out of range";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the call needs more than the library's static decode scratch "
             "(FA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown fa_status";
}

const char* fa_version(void) { return "0.1.0"; }

}  // extern "C"
