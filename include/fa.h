/*
 * fa.h -- C ABI of libfa: exact, IO-aware scaled-dot-product attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes O = softmax(scale * Q K^T [+ causal mask]) V without
 * ever writing the N x N score or probability matrix to device memory: for
 * each block of query rows, key/value tiles stream through on-chip memory
 * and a running maximum and running sum rescale the partial output ("FlashAttention
 * ontleed", § "Algoritmische kern in pseudocode"; Lensa ML explainer, Steps 3
 * and 4).  Three calls make up the library:
 *
 *   fa_fwd     fused forward; writes O and the per-row log-sum-exp L.
 *   fa_bwd     backward by recomputation from Q, K, V, O and L ("03.
 *              FlashAttention", § "Backward pass"); writes dQ, dK, dV.
 *   fa_decode  one query token per head against a long key/value history,
 *              split across workgroups and merged by log-sum-exp ("FlashAttention
 *              ontleed", § "Interactie met de KV-cache tijdens inferentie";
 *              "03. FlashAttention", § "Variantes et extensions").
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major [B, H, N, d] (d contiguous, then N, H, B),
 *     in device memory, of element type `dt` (IEEE fp16 or bfloat16).
 *   - d (head dimension) must be 64 or 128.
 *   - L ("lse") is float32 [B, H, N]: the natural-log log-sum-exp of row i's
 *     scaled, masked scores, L_i = m_i + ln(l_i) in the pages' notation
 *     (running max m and running sum l).
 *   - causal != 0: key j is visible to query i iff j <= i (query and key
 *     positions both count from 0; N_q = N_k in fa_fwd and fa_bwd).
 *   - scale must be finite and > 0 (the pages use 1/sqrt(d)).
 *   - Input values must be finite; results for inputs holding NaN or Inf
 *     are unspecified.
 *   - Arithmetic: exact fp16/bf16 products with fp32 accumulation (matrix
 *     cores in fa_fwd and fa_bwd, packed dot products in fa_decode);
 *     softmax statistics in fp32; P is rounded to `dt` before the P V
 *     product; outputs are rounded to nearest even.
 *   - Pointers to fp16/bf16 tensors and workspaces must be 16-byte aligned;
 *     float32 pointers 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return; errors during execution surface at the
 *     caller's next synchronisation.  fa_bwd on small grids (and fa_bwd_ex
 *     with grouped heads) runs one of its kernels on a second stream of the
 *     library's, forked from `stream` and joined back into it with events,
 *     so the call is still ordered on `stream` as a whole (also inside a
 *     stream capture); with a stream of a device other than the current
 *     one it uses `stream` alone.
 *   - Ownership: the caller allocates and owns every buffer, including the
 *     workspaces sized by the *_workspace_bytes queries.  The library never
 *     allocates or frees device memory.  The state it keeps, per device and
 *     until the process ends: the device address of fa_decode_noalloc's
 *     static scratch, looked up on its first call; fa_bwd's second stream
 *     and two events, created on the first call that uses them outside a
 *     stream capture (a capture before that runs the backward on `stream`
 *     alone).  Outputs must not alias inputs.
 *   - Errors: every argument is validated before any HIP call; on a
 *     validation error (every code but FA_ERR_HIP) nothing is enqueued and
 *     no output is touched.  FA_ERR_HIP means the runtime refused a kernel
 *     launch or a stream or event call (each call's own error code is
 *     checked, so an error an earlier, unrelated HIP call left behind is not
 *     reported here).  A call that launches several kernels may have
 *     enqueued the earlier ones when a later launch is refused, so after
 *     FA_ERR_HIP the outputs and the workspace are undefined.  No C++
 *     exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, H, N, Nkv < 1, sizes overflow, or bad scale */
  FA_ERR_DTYPE = 3,       /* dt is not FA_F16 or FA_BF16 */
  FA_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  FA_ERR_UNSUPPORTED = 5, /* head dimension other than 64 or 128; window without causal */
  FA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the query says */
  FA_ERR_HIP = 7,         /* the HIP runtime refused a launch */
  FA_ERR_SPLITS = 8,      /* num_splits < 1 or above FA_MAX_SPLITS */
  FA_ERR_SCRATCH = 9      /* fa_decode_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

typedef enum fa_dtype { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

#define FA_MAX_SPLITS 256

/*
 * Fused forward ("FlashAttention ontleed", § "Algoritmische kern in
 * pseudocode"; "03. FlashAttention", § "Mécanisme").
 *   q, k, v  in : [B, H, N, d], dt
 *   o        out: [B, H, N, d], dt      -- softmax(scale * q k^T [masked]) v
 *   lse      out: [B, H, N], float32    -- per-row natural-log log-sum-exp
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, fa_dtype dt,
                 void* stream);

/* Bytes of device workspace fa_bwd needs: the float32 row terms
 * D_i = sum_k dout_ik o_ik, [B, H, N], rounded up to 256 bytes (d is only
 * checked). */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward by recomputation ("FlashAttention ontleed", § "Geheugencomplexiteit:
 * van O(N²) naar O(N)"; "03. FlashAttention", § "Backward pass"): P is rebuilt
 * on chip from q, k and the saved lse instead of being stored.
 *   q, k, v, o, dout in : [B, H, N, d], dt (o and lse exactly as fa_fwd wrote
 *                         them for the same q, k, v, scale, causal)
 *   lse             in : [B, H, N], float32
 *   dq, dk, dv      out: [B, H, N, d], dt
 *   workspace           : device scratch of at least fa_bwd_workspace_bytes;
 *                         contents on entry are ignored, on exit undefined.
 * Every output element is written once, without atomics: results are
 * deterministic (bitwise equal across runs with the same inputs).  For
 * grids of at most 512 blocks of 128 keys (B * H * ceil(N / 128)) the dQ
 * kernel runs on the library's second stream, beside the dK/dV kernel (in
 * fa_bwd_ex also whenever H_kv < H).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                 float scale, int causal, fa_dtype dt, void* stream);

/* Bytes of device workspace fa_decode needs: per-split float32 partial
 * outputs [B, H, num_splits, d] and log-sum-exps [B, H, num_splits]. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * Split-history decode for one query token per head ("FlashAttention ontleed",
 * § "Interactie met de KV-cache tijdens inferentie"; Lensa ML explainer,
 * question on decoding).  The Nkv keys of each head are cut into num_splits
 * contiguous chunks of ceil(Nkv / num_splits) keys (the last may be shorter
 * or empty); each chunk yields its normalised partial output and its
 * log-sum-exp, and a second kernel merges the chunks by the online-softmax
 * rescaling rule (Lensa ML explainer, Step 4).  No mask.
 *   q        in : [B, H, 1, d], dt
 *   k, v     in : [B, H, Nkv, d], dt
 *   o        out: [B, H, 1, d], dt
 *   lse      out: [B, H] float32, or NULL if not wanted
 *   workspace   : device scratch of at least fa_decode_workspace_bytes.
 */
fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nkv, int d, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, fa_dtype dt, void* stream);

/*
 * Grouped key/value heads and a causal sliding window.
 *
 * Several query heads may share one key/value head ("FlashAttention ontleed",
 * § "Interactie met de KV-cache tijdens inferentie"), and the keys a query
 * sees may be restricted to a window of the most recent ones ("03.
 * FlashAttention", § "Variantes et extensions": the sliding-window variant
 * tiles only the keys inside the window).  fa_fwd, fa_bwd and fa_decode are
 * these calls with H_kv = H and window = 0.
 *   q, o, dq, dout : [B, H,    N, d]   (decode: [B, H, 1, d])
 *   k, v, dk, dv   : [B, H_kv, N, d]   (decode: [B, H_kv, Nkv, d])
 *   H_kv           : key/value heads, >= 1, dividing H.  Query head h reads
 *                    key/value head h / (H / H_kv) (contiguous groups); dk and
 *                    dv hold the sum over each group's query heads.
 *   window         : 0 for no window.  window = w >= 1 requires causal != 0
 *                    (FA_ERR_UNSUPPORTED otherwise): key j is visible to
 *                    query i iff i - w < j <= i, i.e. the w most recent keys,
 *                    the query's own position included.  w >= N is the same
 *                    as no window.  window < 0 is FA_ERR_SHAPE.
 *   H_kv < 1 or H not a multiple of H_kv is FA_ERR_SHAPE.
 * Workspace sizes are those of fa_bwd_workspace_bytes(B, H, N, d) and
 * fa_decode_workspace_bytes(B, H, d, num_splits), with H the query heads.
 * Every other convention (dtypes, alignment, lse, ownership, errors,
 * streams, determinism) is that of fa_fwd / fa_bwd / fa_decode.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int H_kv, int N, int d, float scale, int causal, int window,
                    fa_dtype dt, void* stream);
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int H, int H_kv, int N,
                    int d, float scale, int causal, int window, fa_dtype dt, void* stream);
fa_status fa_decode_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int H_kv, int Nkv, int d, float scale, int num_splits,
                       void* workspace, size_t workspace_bytes, fa_dtype dt, void* stream);

/*
 * Decode over a padded cache of ragged histories: every sequence of the batch
 * has its own history length ("FlashAttention ontleed", § "Interactie met de
 * KV-cache tijdens inferentie": K and V span each conversation's history).
 * As fa_decode_ex, plus
 *   kv_lens : device int32 [B], 4-byte aligned, read by the kernels:
 *             sequence b attends to its first kv_lens[b] keys of the cache
 *             (values are clamped to [0, Nkv]); its history is cut into
 *             num_splits chunks of ceil(kv_lens[b] / num_splits) keys.  A
 *             sequence with no keys gets o = 0 and lse = -inf.
 *   k, v    : [B, H_kv, Nkv, d], Nkv the cache length (the longest history).
 * kv_lens NULL is FA_ERR_NULL.
 */
fa_status fa_decode_varlen(const void* q, const void* k, const void* v, const int* kv_lens,
                           void* o, float* lse, int B, int H, int H_kv, int Nkv, int d,
                           float scale, int num_splits, void* workspace, size_t workspace_bytes,
                           fa_dtype dt, void* stream);

/*
 * Decode without any device allocation, for callers that cannot allocate:
 * code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  The same computation and kernels as fa_decode_ex (same
 * arguments, minus the workspace), with the per-chunk partial outputs and
 * log-sum-exps held in a static device array of FA_NOALLOC_SCRATCH_BYTES
 * inside the library instead of a caller workspace; the results are bitwise
 * those of fa_decode_ex.
 *   - The call needs fa_decode_workspace_bytes(B, H, d, num_splits) bytes of
 *     it; more is FA_ERR_SCRATCH (checked before any HIP call).  For
 *     example B = 64, H = 32, d = 128, 16 chunks need 16.1 MiB.
 *   - Every GPU the library runs on holds its own copy of the array until the
 *     process ends.  The first call on a device (with that device current)
 *     looks up the array's address there with hipGetSymbolAddress; a failure
 *     of that lookup is FA_ERR_HIP.
 *   - Nothing in the array needs to start at zero: every chunk slot the merge
 *     reads is written by the same call.
 *   - All calls on one device share the array: calls whose kernels may run at
 *     the same time on one device (other streams, other threads) race and
 *     give undefined results.  Calls in order on one stream are safe.
 *   - No allocation of any kind: no hipMalloc, hipFree or allocating library
 *     routine is called.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int Nkv, int d, float scale, int num_splits,
                            fa_dtype dt, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(fa_status s);

/* Library version as "major.minor.patch" (static string). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
