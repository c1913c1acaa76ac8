// fa_decode.hip -- split-history single-token decode for gfx950.
//
// With one query token per head the score "matrix" is a single row and the
// cost is reading the key/value history ("FlashAttention ontleed",
// § "Interactie met de KV-cache tijdens inferentie"; Lensa ML explainer,
// question on decoding).  To keep every CU busy the history of each head is
// cut into `splits` contiguous chunks ("03. FlashAttention", § "Variantes et
// extensions": the decode variant spreads the history read over many
// workgroups).  Kernel 1 turns each chunk into its normalised partial output
// and log-sum-exp; kernel 2 merges the chunks with the online-softmax
// rescaling rule applied to whole chunks (Lensa ML explainer, Step 4).
//
// The path is HBM-bound (about 1 flop per byte), so the kernels are written
// for bandwidth: 16-byte coalesced loads (a run of d/8 lanes reads one
// 2*d-byte key row), several loads in flight per lane, fp32 FMAs on the
// VALU (the matrix cores would idle with one query column), and the chunk's
// scores kept in LDS between the K pass and the V pass.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int DEC_THREADS = 256;
constexpr int DEC_SUB = 1024;  // keys whose scores are held in LDS at a time
constexpr int DEC_UNROLL = 8;  // key rows in flight per lane

template <typename T>
__device__ __forceinline__ void widen8(const typename Vec<T>::v8& x, float* f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)x[i];
}

// x + (x of the lane chosen by the DPP pattern), all in registers.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the WIDTH consecutive lanes (8 or 16, aligned) that share a key
// row, with DPP lane moves instead of LDS permutes: swap neighbours and
// pairs inside each quad (quad_perm 1,0,3,2 and 2,3,0,1), then mirror within
// each 8-lane half-row (every lane now holds its 8-lane sum) and, for 16,
// within the 16-lane row.
template <int WIDTH>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(WIDTH == 8 || WIDTH == 16, "8- or 16-lane rows");
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_add<0x141>(x);  // row_half_mirror
  if (WIDTH == 16) x = dpp_add<0x140>(x);  // row_mirror
  return x;
}

// Streaming 16-byte load (each K/V byte is read exactly once).
template <typename V>
__device__ __forceinline__ V ld16_stream(const void* p) {
  return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Kernel 1: one workgroup per (head, chunk).
template <typename T, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ part_o, float* __restrict__ part_lse, int Nkv, int splits, int chunk,
    int group, float c) {
  using v8 = typename Vec<T>::v8;
  constexpr int LPK = D / 8;                 // lanes per key row
  constexpr int KPI = DEC_THREADS / LPK;     // key rows per workgroup step
  __shared__ float sc[DEC_SUB];
  __shared__ float red[DEC_THREADS / 64];
  __shared__ float oacc_s[KPI][D + 4];

  const int bh = blockIdx.x / splits, split = blockIdx.x % splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = tid / LPK, col = tid % LPK;
  const int k_lo = split * chunk;
  const int k_hi = min(Nkv, k_lo + chunk);
  float* __restrict__ po = part_o + ((size_t)bh * splits + split) * D;

  if (k_lo >= k_hi) {  // empty chunk: weight zero in the merge
    for (int i = tid; i < D; i += DEC_THREADS) po[i] = 0.f;
    if (tid == 0) part_lse[(size_t)bh * splits + split] = -INFINITY;
    return;
  }

  // Query head bh reads key/value head bh / group ("FlashAttention ontleed",
  // § "Interactie met de KV-cache tijdens inferentie": query heads may share
  // key/value heads).  The group's heads have the same chunk index and
  // grid positions that differ by a multiple of `splits`, so they run close
  // together on one XCD and share the chunk through its L2.
  const size_t hoff = (size_t)(bh / group) * Nkv * D;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;
  float qv[8];
  widen8<T>(ld16<v8>(Q + (size_t)bh * D + 8 * col), qv);
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] *= c;  // scores come out in log2 units

  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int s0 = k_lo; s0 < k_hi; s0 += DEC_SUB) {
    const int s1 = min(k_hi, s0 + DEC_SUB);
    // K pass: scores of keys s0..s1-1 into LDS.
    for (int kk = s0 + slot; kk < s1; kk += KPI * DEC_UNROLL) {
      // Rows past the sub-chunk are clamped to its last row (always valid);
      // their scores are never stored.
      v8 kr[DEC_UNROLL];
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        const int key = min(kk + u * KPI, s1 - 1);
        kr[u] = ld16_stream<v8>(Kh + (size_t)key * D + 8 * col);
      }
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        float kf[8];
        widen8<T>(kr[u], kf);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = __builtin_fmaf(qv[i], kf[i], dot);
        dot = row_sum<LPK>(dot);
        const int key = kk + u * KPI;
        if (col == 0 && key < s1) sc[key - s0] = dot;
      }
    }
    __syncthreads();
    // Chunk maximum.
    float mx = -INFINITY;
    for (int i = tid; i < s1 - s0; i += DEC_THREADS) mx = fmaxf(mx, sc[i]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int wv = 1; wv < DEC_THREADS / 64; ++wv) mx = fmaxf(mx, red[wv]);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    __syncthreads();  // everyone has read red[]
    // Probabilities (unnormalised) in place, and their sum.
    float ps = 0.f;
    for (int i = tid; i < s1 - s0; i += DEC_THREADS) {
      const float pe = fast_exp2(sc[i] - m_new);
      sc[i] = pe;
      ps += pe;
    }
    ps = wave_sum(ps);
    if (lane == 0) red[wave] = ps;
    __syncthreads();
    ps = 0.f;
#pragma unroll
    for (int wv = 0; wv < DEC_THREADS / 64; ++wv) ps += red[wv];
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
    // V pass: o += p * v over this lane's key rows.
    for (int kk = s0 + slot; kk < s1; kk += KPI * DEC_UNROLL) {
      // Clamped rows as in the K pass; they get weight 0 below.
      v8 vr[DEC_UNROLL];
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        const int key = min(kk + u * KPI, s1 - 1);
        vr[u] = ld16_stream<v8>(Vh + (size_t)key * D + 8 * col);
      }
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        const int key = kk + u * KPI;
        const float pe = (key < s1) ? sc[key - s0] : 0.f;
        float vf[8];
        widen8<T>(vr[u], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = __builtin_fmaf(pe, vf[i], o[i]);
      }
    }
    __syncthreads();  // sc[] and red[] are reused by the next sub-chunk
  }

  // Sum the per-slot partial outputs, normalise, write the chunk summary.
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc_s[slot][8 * col + i] = o[i];
  __syncthreads();
  const float inv = 1.f / l_run;
  for (int x = tid; x < D; x += DEC_THREADS) {
    float s = 0.f;
#pragma unroll 4
    for (int sl = 0; sl < KPI; ++sl) s += oacc_s[sl][x];
    po[x] = s * inv;
  }
  if (tid == 0)
    part_lse[(size_t)bh * splits + split] = (m_run + log2f(l_run)) * 0.69314718055994531f;
}

// Kernel 2: one wave per head merges its chunk summaries.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          T* __restrict__ O, float* __restrict__ LSE,
                                                          int splits) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* __restrict__ pl = part_lse + (size_t)bh * splits;
  const float* __restrict__ po = part_o + (size_t)bh * splits * D;
  float big = -INFINITY;
  for (int s = lane; s < splits; s += 64) big = fmaxf(big, pl[s]);
  big = wave_max(big);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = expf(pl[s] - big);  // exp(-inf) = 0 for empty chunks
    wsum += w;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w, po[(size_t)s * D + lane + 64 * i], acc[i]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) O[(size_t)bh * D + lane + 64 * i] = (T)(acc[i] * inv);
  if (LSE && lane == 0) LSE[bh] = big + logf(wsum);
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int chunk = (a.Nkv + a.splits - 1) / a.splits;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(BH * a.splits), dim3(DEC_THREADS), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.part_o, a.part_lse, a.Nkv, a.splits, chunk,
                     a.H / a.Hkv, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(BH), dim3(64), 0, s, a.part_o, a.part_lse,
                     static_cast<T*>(a.o), a.lse, a.splits);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_decode_t<T, 64>(a, s) : launch_decode_t<T, 128>(a, s);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_decode_dt<__bf16>(a, s) : launch_decode_dt<_Float16>(a, s);
}

size_t decode_part_o_bytes(int B, int H, int d, int splits) {
  return align256((size_t)B * H * splits * d * sizeof(float));
}
size_t decode_part_lse_bytes(int B, int H, int splits) {
  return align256((size_t)B * H * splits * sizeof(float));
}

}  // namespace fa
