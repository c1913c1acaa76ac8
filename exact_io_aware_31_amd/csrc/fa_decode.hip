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
// 2*d-byte key row), several loads in flight per lane, packed dot products
// on the VALU (the matrix cores would idle with one query column), and the
// chunk's scores kept in LDS between the K pass and the V pass.  Scores are
// v_dot2_f32 over pairs of stored elements (exact products, fp32 sums);
// the probabilities are rounded to the storage type, as the fused forward
// pass rounds P for its P V product, and the output accumulates
// v_dot2_f32 over pairs of keys: (v_a[i], v_b[i]) . (p_a, p_b).
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"
#include "../../include/fa.h"

namespace fa {

constexpr int DEC_THREADS = 256;
constexpr int DEC_SUB = 1024;  // keys whose scores are held in LDS at a time
constexpr int DEC_UNROLL = 8;  // key rows in flight per lane

// acc + a.x b.x + a.y b.y in fp32 (v_dot2_f32_bf16 / v_dot2_f32_f16).
__device__ __forceinline__ float dot2(__bf16 __attribute__((ext_vector_type(2))) a,
                                      __bf16 __attribute__((ext_vector_type(2))) b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}
__device__ __forceinline__ float dot2(_Float16 __attribute__((ext_vector_type(2))) a,
                                      _Float16 __attribute__((ext_vector_type(2))) b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}
// sum_i a[i] b[i] over 8 elements: four packed dot products.  The pairs are
// taken with element shuffles: fed bit casts of the packed 32-bit words
// instead, this compiler keeps only the first of several such dot products.
template <typename V8>
__device__ __forceinline__ float dot8(V8 a, V8 b) {
  float acc = dot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), 0.f);
  acc = dot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc);
  acc = dot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc);
  return dot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc);
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
  static_assert(WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "4-, 8- or 16-lane rows");
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  if (WIDTH >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
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

// Kernel 1: one workgroup per (G query heads, chunk).  The G heads share one
// key/value head ("FlashAttention ontleed", § "Interactie met de KV-cache
// tijdens inferentie": query heads may share key/value heads), so the chunk
// of K and V is read once for all of them: each key row is dotted with G
// queries and each value row accumulated into G outputs.  G = 1 is plain
// multi-head decode.  Query heads h0 .. h0 + G - 1 (over B x H) with
// h0 = kvbh * group + G * (workgroup index within the group).
template <typename T, int D, int G>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int* __restrict__ kv_lens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Nkv, int splits, int Hkv, int group, float c) {
  using v8 = typename Vec<T>::v8;
  constexpr int LPK = D / 8;                 // lanes per value row (V pass)
  constexpr int KPI = DEC_THREADS / LPK;     // value rows per workgroup step
  // K pass: with one query head each lane dots 16 elements (two 16-byte
  // loads) of a key row, so a row is summed over D / 16 lanes, one DPP step
  // fewer per score (+1.3% at B64 H32 Nkv16384); with several heads the
  // extra query registers would cost occupancy, so 8 elements per lane.
  constexpr int KP = (G == 1) ? 2 : 1;       // 16-byte parts of a key row per lane
  constexpr int LPKK = D / (8 * KP);         // lanes per key row (K pass)
  constexpr int KPIK = DEC_THREADS / LPKK;   // key rows per workgroup step (K pass)
  constexpr int UNK = DEC_UNROLL / KP;       // key rows in flight per lane
  constexpr int NWV = DEC_THREADS / 64;      // waves
  __shared__ float sc[G][DEC_SUB];
  __shared__ float red[G][NWV];
  __shared__ float oacc_s[KPI][D + 4];

  const int wg = blockIdx.x / splits, split = blockIdx.x % splits;
  const int per_kv = group / G;                      // workgroups per key/value head
  const int kvbh = wg / per_kv;                      // key/value head (over B x H_kv)
  const int h0 = kvbh * group + G * (wg % per_kv);   // first query head (over B x H)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = tid / LPK, col = tid % LPK;
  const int kslot = tid / LPKK, kcol = tid % LPKK;
  // This sequence's history: its first kv_lens[b] keys (clamped to the cache),
  // cut into `splits` chunks of ceil(len / splits) keys.
  const int len = kv_lens ? min(max(kv_lens[kvbh / Hkv], 0), Nkv) : Nkv;
  const int chunk = (len + splits - 1) / splits;
  const int k_lo = split * chunk;
  const int k_hi = min(len, k_lo + chunk);

  if (k_lo >= k_hi) {  // empty chunk: weight zero in the merge
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      float* __restrict__ po = part_o + ((size_t)(h0 + gh) * splits + split) * D;
      for (int i = tid; i < D; i += DEC_THREADS) po[i] = 0.f;
      if (tid == 0) part_lse[(size_t)(h0 + gh) * splits + split] = -INFINITY;
    }
    return;
  }

  const size_t hoff = (size_t)kvbh * Nkv * D;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;
  // The query elements stay packed; scores are scaled by c after the sum,
  // so they come out in log2 units.
  v8 qv[G][KP];
#pragma unroll
  for (int gh = 0; gh < G; ++gh)
#pragma unroll
    for (int pp = 0; pp < KP; ++pp) qv[gh][pp] = ld16<v8>(Q + (size_t)(h0 + gh) * D + 8 * (KP * kcol + pp));

  float o[G][8], m_run[G], l_run[G];
#pragma unroll
  for (int gh = 0; gh < G; ++gh) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[gh][i] = 0.f;
    m_run[gh] = -INFINITY;
    l_run[gh] = 0.f;
  }

  for (int s0 = k_lo; s0 < k_hi; s0 += DEC_SUB) {
    const int s1 = min(k_hi, s0 + DEC_SUB);
    // K pass: scores of keys s0..s1-1 for the G heads into LDS.
    for (int kk = s0 + kslot; kk < s1; kk += KPIK * UNK) {
      // Rows past the sub-chunk are clamped to its last row (always valid);
      // their scores are never stored.
      v8 kr[UNK][KP];
#pragma unroll
      for (int u = 0; u < UNK; ++u) {
        const int key = min(kk + u * KPIK, s1 - 1);
#pragma unroll
        for (int pp = 0; pp < KP; ++pp)
          kr[u][pp] = ld16_stream<v8>(Kh + (size_t)key * D + 8 * (KP * kcol + pp));
      }
#pragma unroll
      for (int u = 0; u < UNK; ++u) {
        const int key = kk + u * KPIK;
#pragma unroll
        for (int gh = 0; gh < G; ++gh) {
          float part = dot8(kr[u][0], qv[gh][0]);
#pragma unroll
          for (int pp = 1; pp < KP; ++pp) part += dot8(kr[u][pp], qv[gh][pp]);
          const float dot = row_sum<LPKK>(part) * c;
          if (kcol == 0 && key < s1) sc[gh][key - s0] = dot;
        }
      }
    }
    __syncthreads();
    // Chunk maxima, one per head.
    float mx[G];
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      mx[gh] = -INFINITY;
      for (int i = tid; i < s1 - s0; i += DEC_THREADS) mx[gh] = fmaxf(mx[gh], sc[gh][i]);
      mx[gh] = wave_max(mx[gh]);
      if (lane == 0) red[gh][wave] = mx[gh];
    }
    __syncthreads();
    float alpha[G], m_new[G];
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      float m = red[gh][0];
#pragma unroll
      for (int wv = 1; wv < NWV; ++wv) m = fmaxf(m, red[gh][wv]);
      m_new[gh] = fmaxf(m_run[gh], m);
      alpha[gh] = fast_exp2(m_run[gh] - m_new[gh]);
    }
    __syncthreads();  // everyone has read red[]
    // Probabilities (unnormalised, rounded to the storage type: the weights
    // the V pass uses) in place, and their sums.
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      float ps = 0.f;
      for (int i = tid; i < s1 - s0; i += DEC_THREADS) {
        const float pe = (float)(T)fast_exp2(sc[gh][i] - m_new[gh]);
        sc[gh][i] = pe;
        ps += pe;
      }
      ps = wave_sum(ps);
      if (lane == 0) red[gh][wave] = ps;
    }
    __syncthreads();
#pragma unroll
    for (int gh = 0; gh < G; ++gh) {
      float ps = 0.f;
#pragma unroll
      for (int wv = 0; wv < NWV; ++wv) ps += red[gh][wv];
      l_run[gh] = l_run[gh] * alpha[gh] + ps;
      m_run[gh] = m_new[gh];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[gh][i] *= alpha[gh];
    }
    // V pass: o += p * v over this lane's key rows, for every head.
    for (int kk = s0 + slot; kk < s1; kk += KPI * DEC_UNROLL) {
      // Clamped rows as in the K pass; they get weight 0 below.
      v8 vr[DEC_UNROLL];
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        const int key = min(kk + u * KPI, s1 - 1);
        vr[u] = ld16_stream<v8>(Vh + (size_t)key * D + 8 * col);
      }
      // Keys in pairs (u, u+1): element i of the two value rows against the
      // two probabilities, one packed dot product per element and head.
      typedef T t2 __attribute__((ext_vector_type(2)));
      static_assert(DEC_UNROLL % 2 == 0, "value rows are taken in pairs");
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; u += 2) {
        const int ka = kk + u * KPI, kb = ka + KPI;
        const v8 va = vr[u], vb = vr[u + 1];
        t2 vp[8];
        vp[0] = __builtin_shufflevector(va, vb, 0, 8);
        vp[1] = __builtin_shufflevector(va, vb, 1, 9);
        vp[2] = __builtin_shufflevector(va, vb, 2, 10);
        vp[3] = __builtin_shufflevector(va, vb, 3, 11);
        vp[4] = __builtin_shufflevector(va, vb, 4, 12);
        vp[5] = __builtin_shufflevector(va, vb, 5, 13);
        vp[6] = __builtin_shufflevector(va, vb, 6, 14);
        vp[7] = __builtin_shufflevector(va, vb, 7, 15);
#pragma unroll
        for (int gh = 0; gh < G; ++gh) {
          const t2 pp = {(T)((ka < s1) ? sc[gh][ka - s0] : 0.f), (T)((kb < s1) ? sc[gh][kb - s0] : 0.f)};
#pragma unroll
          for (int i = 0; i < 8; ++i) o[gh][i] = dot2(vp[i], pp, o[gh][i]);
        }
      }
    }
    __syncthreads();  // sc[] and red[] are reused by the next sub-chunk
  }

  // Per head: sum the per-slot partial outputs, normalise, write the chunk summary.
#pragma unroll
  for (int gh = 0; gh < G; ++gh) {
#pragma unroll
    for (int i = 0; i < 8; ++i) oacc_s[slot][8 * col + i] = o[gh][i];
    __syncthreads();
    float* __restrict__ po = part_o + ((size_t)(h0 + gh) * splits + split) * D;
    const float inv = 1.f / l_run[gh];
    for (int x = tid; x < D; x += DEC_THREADS) {
      float sum = 0.f;
#pragma unroll 4
      for (int sl = 0; sl < KPI; ++sl) sum += oacc_s[sl][x];
      po[x] = sum * inv;
    }
    if (tid == 0)
      part_lse[(size_t)(h0 + gh) * splits + split] =
          (m_run[gh] + log2f(l_run[gh])) * 0.69314718055994531f;
    __syncthreads();  // oacc_s is reused by the next head
  }
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
  if (big == -INFINITY) {  // no key at all (an empty history): O = 0, lse = -inf
    for (int i = lane; i < D; i += 64) O[(size_t)bh * D + i] = (T)0.f;
    if (LSE && lane == 0) LSE[bh] = -INFINITY;
    return;
  }
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

template <typename T, int D, int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
  const float c = a.scale * 1.4426950408889634f;
  return launch_kernel(decode_split_kernel<T, D, G>, dim3(a.B * a.H / G * a.splits),
                       dim3(DEC_THREADS), s, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.kv_lens, a.part_o,
                       a.part_lse, a.Nkv, a.splits, a.Hkv, a.H / a.Hkv, c);
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  // Query heads per workgroup: the largest of 4, 2, 1 dividing the group.
  // (Eight heads need more than 256 registers per lane: one wave per SIMD,
  // too few loads in flight for the HBM stream.)
  const int group = a.H / a.Hkv;
  hipError_t e = (group % 4 == 0)   ? launch_decode_g<T, D, 4>(a, s)
                 : (group % 2 == 0) ? launch_decode_g<T, D, 2>(a, s)
                                    : launch_decode_g<T, D, 1>(a, s);
  if (e != hipSuccess) return e;
  return launch_kernel(decode_merge_kernel<T, D>, dim3(a.B * a.H), dim3(64), s, a.part_o,
                       a.part_lse, static_cast<T*>(a.o), a.lse, a.splits);
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_decode_t<T, 64>(a, s) : launch_decode_t<T, 128>(a, s);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_decode_dt<__bf16>(a, s) : launch_decode_dt<_Float16>(a, s);
}

// Scratch of fa_decode_noalloc, for callers that cannot allocate device
// memory: the per-chunk partial outputs and log-sum-exps live in this
// file-scope array, which every device the library runs on holds (its own
// copy) until the process ends.  Host code never uses the array's name as an
// address: the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Every chunk slot
// the merge reads is written by the split kernel of the same call (empty
// chunks included), so nothing needs clearing between calls; calls that
// overlap on one device share the array and race.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
