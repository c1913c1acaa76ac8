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
// The path is HBM-bound (about 1 flop per byte per query head), so the
// kernels are written for bandwidth: 16-byte coalesced non-temporal loads
// (every K/V byte is read once), several loads in flight per lane, and no
// arithmetic unit that the stream has to wait for.  Two chunk kernels:
//   * one query head per key/value head: packed dot products on the VALU
//     (the matrix cores would idle with one query column).  Scores are
//     v_dot2_f32 over pairs of stored elements (exact products, fp32 sums),
//     kept in LDS between a K pass and a V pass; the probabilities are
//     rounded to the storage type, as the fused forward pass rounds P for its
//     P V product, and the output accumulates v_dot2_f32 over pairs of keys:
//     (v_a[i], v_b[i]) . (p_a, p_b).
//   * several query heads per key/value head: the G heads' scores and
//     outputs are matrix products, done on the matrix cores with the heads
//     as columns (up to 16 per workgroup), so each chunk of K and V is read
//     once for all of them.
#include <mutex>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_tile.h"
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
// Sum over the WIDTH consecutive lanes (4 or 8, aligned) that share a key
// row, with DPP lane moves instead of LDS permutes: swap neighbours and
// pairs inside each quad (quad_perm 1,0,3,2 and 2,3,0,1), then, for 8,
// mirror within each 8-lane half-row (every lane now holds its 8-lane sum).
template <int WIDTH>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(WIDTH == 4 || WIDTH == 8, "4- or 8-lane rows");
  x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
  if (WIDTH == 8) x = dpp_add<0x141>(x);  // row_half_mirror
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

// Kernel 1, one query head per key/value head: one workgroup per (head,
// chunk).  A K pass puts the chunk's scores into LDS, the chunk maximum and
// sum are reduced over the workgroup, and a V pass accumulates the output,
// 1024 keys at a time.
template <typename T, int D>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int* __restrict__ kv_lens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Nkv, int splits, int H, float c) {
  using v8 = typename Vec<T>::v8;
  constexpr int LPK = D / 8;                 // lanes per value row (V pass)
  constexpr int KPI = DEC_THREADS / LPK;     // value rows per workgroup step
  // K pass: each lane dots 16 elements (two 16-byte loads) of a key row, so
  // a row is summed over D / 16 lanes, one DPP step fewer per score than
  // with 8 elements per lane (+1.3% at B64 H32 Nkv16384).
  constexpr int KP = 2;                      // 16-byte parts of a key row per lane
  constexpr int LPKK = D / (8 * KP);         // lanes per key row (K pass)
  constexpr int KPIK = DEC_THREADS / LPKK;   // key rows per workgroup step (K pass)
  constexpr int UNK = DEC_UNROLL / KP;       // key rows in flight per lane
  constexpr int NWV = DEC_THREADS / 64;      // waves
  __shared__ float sc[DEC_SUB];
  __shared__ float red[NWV];
  __shared__ float oacc_s[KPI][D + 4];

  const int bh = blockIdx.x / splits, split = blockIdx.x % splits;  // head over B x H
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = tid / LPK, col = tid % LPK;
  const int kslot = tid / LPKK, kcol = tid % LPKK;
  // This sequence's history: its first kv_lens[b] keys (clamped to the cache),
  // cut into `splits` chunks of ceil(len / splits) keys.
  const int len = kv_lens ? min(max(kv_lens[bh / H], 0), Nkv) : Nkv;
  const int chunk = (len + splits - 1) / splits;
  const int k_lo = split * chunk;
  const int k_hi = min(len, k_lo + chunk);
  float* __restrict__ po = part_o + ((size_t)bh * splits + split) * D;

  if (k_lo >= k_hi) {  // empty chunk: weight zero in the merge
    for (int i = tid; i < D; i += DEC_THREADS) po[i] = 0.f;
    if (tid == 0) part_lse[(size_t)bh * splits + split] = -INFINITY;
    return;
  }

  const size_t hoff = (size_t)bh * Nkv * D;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;
  // The query elements stay packed; scores are scaled by c after the sum,
  // so they come out in log2 units.
  v8 qv[KP];
#pragma unroll
  for (int pp = 0; pp < KP; ++pp) qv[pp] = ld16<v8>(Q + (size_t)bh * D + 8 * (KP * kcol + pp));

  float o[8], m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  for (int s0 = k_lo; s0 < k_hi; s0 += DEC_SUB) {
    const int s1 = min(k_hi, s0 + DEC_SUB);
    // K pass: scores of keys s0..s1-1 into LDS.
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
        float part = dot8(kr[u][0], qv[0]);
#pragma unroll
        for (int pp = 1; pp < KP; ++pp) part += dot8(kr[u][pp], qv[pp]);
        const float dot = row_sum<LPKK>(part) * c;
        if (kcol == 0 && key < s1) sc[key - s0] = dot;
      }
    }
    __syncthreads();
    // Chunk maximum.
    float mx = -INFINITY;
    for (int i = tid; i < s1 - s0; i += DEC_THREADS) mx = fmaxf(mx, sc[i]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int wv = 1; wv < NWV; ++wv) m = fmaxf(m, red[wv]);
    const float m_new = fmaxf(m_run, m);
    const float alpha = fast_exp2(m_run - m_new);
    __syncthreads();  // everyone has read red[]
    // Probabilities (unnormalised, rounded to the storage type: the weights
    // the V pass uses) in place, and their sum.
    float ps = 0.f;
    for (int i = tid; i < s1 - s0; i += DEC_THREADS) {
      const float pe = (float)(T)fast_exp2(sc[i] - m_new);
      sc[i] = pe;
      ps += pe;
    }
    ps = wave_sum(ps);
    if (lane == 0) red[wave] = ps;
    __syncthreads();
    ps = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWV; ++wv) ps += red[wv];
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
      // Keys in pairs (u, u+1): element i of the two value rows against the
      // two probabilities, one packed dot product per element.
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
        const t2 pp = {(T)((ka < s1) ? sc[ka - s0] : 0.f), (T)((kb < s1) ? sc[kb - s0] : 0.f)};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = dot2(vp[i], pp, o[i]);
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
    float sum = 0.f;
#pragma unroll 4
    for (int sl = 0; sl < KPI; ++sl) sum += oacc_s[sl][x];
    po[x] = sum * inv;
  }
  if (tid == 0) part_lse[(size_t)bh * splits + split] = (m_run + log2f(l_run)) * 0.69314718055994531f;
}

// Kernel 1, grouped heads on the matrix cores.  With G >= 2 query heads per
// key/value head ("FlashAttention ontleed", § "Interactie met de KV-cache
// tijdens inferentie") the chunk's scores are a G x keys matrix product and
// its output a G x d one, so both go to v_mfma_f32_16x16x32 with the query
// heads as the sixteen matrix columns (G <= 16; the unused columns hold zero
// queries and are never written out).  Per lane the VALU then only does the
// softmax of its head: the packed dot products and row sums of the kernel
// above are gone.
//   * One workgroup of four waves per (key/value head, G query heads, chunk).
//     Wave w takes the chunk's 32-key tiles w, w + 4, w + 8, ... and keeps its
//     own running maximum, running sum and output; the four are merged by the
//     online-softmax rule in LDS at the end (Lensa ML explainer, Step 4).
//   * S^T = K Q^T: the key rows are the A operand, read straight from HBM
//     into registers (16-byte buffer loads, one tile ahead); lane l supplies
//     key l % 16 of a 16-key block and elements 32 t + 8 (l / 16) .. + 7 of
//     its row, and Q^T (held for the whole chunk) the same elements of query
//     head l % 16.  Accumulator register r of lane l is then the score of key
//     4 (l / 16) + r against head l % 16.
//   * The probabilities of a 32-key tile stay in registers as the B operand
//     of O^T += V^T P^T: lane l's eight values are keys 4 (l / 16) .. + 3 of
//     the first 16-key block and the same four of the second, a permutation
//     of the 32 reduction indices that the A operand V^T repeats.  V^T comes
//     from transpose reads (ds_read_b64_tr_b16) of the row-major V tile, which
//     each wave loads into its own two-deep LDS ring with direct buffer-to-LDS
//     loads.  Rows past the chunk read as zero (buffer range check) and their
//     scores are masked.
//   * Running maximum in log2 units with the lazy rescale of the fused forward
//     pass (the reference maximum is moved only when a tile's maximum exceeds
//     it by more than 2^8), so the probabilities stay below 2^8.
constexpr int DGM_WAVES = 4;
constexpr int DGM_MAX_G = 16;
constexpr int DGM_TK = 32;   // keys per tile

// Swizzle of the decode's V tiles: 16-byte chunk c of row r at c ^ sw(r).
// A transpose read touches rows 4 g .. 4 g + 3 (g the lane's 16-lane group)
// at two neighbouring chunks; with these XORs the 32 lanes of groups 0-1 (and
// of groups 2-3) address 16 different 16-byte bank groups.
template <int D>
struct DecodeSwizzle {
  static __device__ __forceinline__ int sw(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Max / sum over the four lanes l % 16 + 16 g (g = 0..3): v_permlane16_swap
// then v_permlane32_swap on (x, x), each giving every lane its own value and
// its partner's.
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  return half_pair_max(x);
}
__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  return half_pair_sum(x);
}

template <typename T, int D>
__global__ __launch_bounds__(DGM_WAVES * 64) void decode_group_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int* __restrict__ kv_lens, float* __restrict__ part_o, float* __restrict__ part_lse,
    int Nkv, int splits, int Hkv, int group, int G, float c) {
  using v8 = typename Vec<T>::v8;
  constexpr int TK = DGM_TK;
  constexpr int NKB = TK / 16;               // 16-key blocks per tile
  constexpr int NT = D / 32;                 // k-steps of S^T = K Q^T
  constexpr int NB = D / 16;                 // 16-row blocks of O^T
  constexpr int TILE = TK * D;               // elements of a V tile
  constexpr int LPT = NKB * NT + TILE * 2 / 1024;  // loads per tile and lane (vmcnt units)
  static_assert(NKB == 2, "32-key tiles: two 16-key blocks");
  static_assert(D * DGM_MAX_G * 4 <= TILE * 2, "a wave's output fits in its first ring slot");
  // The two ring slots are separate arrays, so the compiler can tell the
  // loads into one slot from the reads of the other and waits only for the
  // loads a read depends on.
  __shared__ __attribute__((aligned(1024))) T Vs0[DGM_WAVES][TILE];
  __shared__ __attribute__((aligned(1024))) T Vs1[DGM_WAVES][TILE];
  __shared__ float ms[DGM_WAVES][DGM_MAX_G], ls[DGM_WAVES][DGM_MAX_G];

  const int wg = blockIdx.x / splits, split = blockIdx.x % splits;
  const int per_kv = group / G;                      // workgroups per key/value head
  const int kvbh = wg / per_kv;                      // key/value head (over B x H_kv)
  const int h0 = kvbh * group + G * (wg % per_kv);   // first query head (over B x H)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_int(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int len = kv_lens ? min(max(kv_lens[kvbh / Hkv], 0), Nkv) : Nkv;
  const int chunk = (len + splits - 1) / splits;
  const int k_lo = split * chunk;
  const int k_hi = min(len, k_lo + chunk);

  if (k_lo >= k_hi) {  // empty chunk: weight zero in the merge
    for (int i = tid; i < G * D; i += DGM_WAVES * 64)
      part_o[((size_t)(h0 + i / D) * splits + split) * D + i % D] = 0.f;
    if (tid < G) part_lse[(size_t)(h0 + tid) * splits + split] = -INFINITY;
    return;
  }

  const size_t hoff = (size_t)kvbh * Nkv * D;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;
  // Q^T as the B operand: lane l holds elements 32 t + 8 (l / 16) .. + 7 of
  // query head h0 + l % 16 (zero for the unused columns).
  v8 qop[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    qop[t] = (n16 < G) ? ld16<v8>(Q + (size_t)(h0 + n16) * D + 32 * t + 8 * g4) : v8{};

  // Byte offsets inside a tile: the K row elements of the A operand, and the
  // transpose reads of V (lane a of group g addresses row 4 g + a / 4 of a
  // 16-key block, columns 16 nb + 4 (a mod 4) .. + 3).
  uint32_t koff[NKB][NT];
#pragma unroll
  for (int b = 0; b < NKB; ++b)
#pragma unroll
    for (int t = 0; t < NT; ++t) koff[b][t] = 2u * (uint32_t)((16 * b + n16) * D + 32 * t + 8 * g4);
  uint32_t voff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    voff[nb] = 2u * (uint32_t)tile_off<D, DecodeSwizzle<D>>(4 * g4 + (n16 >> 2), 16 * nb + 4 * (n16 & 3));
  const TileLoader<D, TK, 1, DecodeSwizzle<D>> vload(0, lane);

  const int ntile = (k_hi - k_lo + TK - 1) / TK;
  const int nmine = ntile > wave ? (ntile - wave + DGM_WAVES - 1) / DGM_WAVES : 0;

  // Tile i of this wave: K rows into kr, V rows into ring slot `slot`.  Both
  // are read once, so the loads are non-temporal.  A tile past the chunk gets
  // a descriptor of zero bytes: its loads read nothing (the range check
  // returns zeros) but count like any other, so the loop below issues the
  // same loads on every step and needs no branch around them (the compiler's
  // wait counting is exact only without one).
  auto load_tile = [&](int i, u32x4 (&kr)[NKB][NT], T* slot) {
    const int kb = min(k_lo + TK * (wave + DGM_WAVES * i), k_hi);
    const int rows = min(k_hi - kb, TK);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(Kh + (size_t)kb * D), 0, rows * D * 2, 0x00020000);
#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        kr[b][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)koff[b][t], 0, FA_CPOL_NT);
    vload.template load<FA_CPOL_NT>(Vh, kb + rows, kb, slot, 0);
  };

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f, nref = -0.f;

  auto tile = [&](int i, const u32x4 (&kr)[NKB][NT], const T* vt) {
    const int kb = k_lo + TK * (wave + DGM_WAVES * i);
    f32x4 s[NKB];
#pragma unroll
    for (int b = 0; b < NKB; ++b) s[b] = f32x4{};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int b = 0; b < NKB; ++b) s[b] = mfma16x16x32(__builtin_bit_cast(v8, kr[b][t]), qop[t], s[b]);
    if (kb + TK > k_hi) {  // keys past the chunk: -inf
      const int lim = k_hi - kb - 4 * g4;
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * b + r >= lim) s[b][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = group4_max(mx);
    const float m_cand = mx * c;
    if (__ballot(m_cand > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb] *= alpha;
      m_run = m_new;
      nref = (m_new == -INFINITY) ? -0.f : -m_new;
    }
    float p[4 * NKB];
#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[4 * b + r] = fast_exp2(__builtin_fmaf(s[b][r], c, nref));
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    const v8 pb = to_v8<T>(p);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x2 lo = lds_tr_at(vt, voff[nb]);
      const u32x2 hi = lds_tr_at(vt, voff[nb] + 16 * D * 2);
      const u32x4 cat = {lo[0], lo[1], hi[0], hi[1]};
      oacc[nb] = mfma16x16x32(__builtin_bit_cast(v8, cat), pb, oacc[nb]);
    }
  };

  // Two register sets for the K rows and two ring slots for V: tile i + 1
  // loads while tile i is computed.
  // (The rows stay 32-bit words until the MFMA: moved as bf16 vectors they
  // are repacked per 16-bit half, which reads each load as soon as it is
  // issued and so waits for it.)
  u32x4 ka[NKB][NT], kn[NKB][NT];
  if (nmine > 0) load_tile(0, ka, Vs0[wave]);
  for (int i = 0; i < nmine; i += 2) {
    load_tile(i + 1, kn, Vs1[wave]);
    wait_counts<FA_VMCNT_LGKM0(LPT)>();
    tile(i, ka, Vs0[wave]);
    if (i + 1 >= nmine) break;
    load_tile(i + 2, ka, Vs0[wave]);
    wait_counts<FA_VMCNT_LGKM0(LPT)>();
    tile(i + 1, kn, Vs1[wave]);
  }

  // Merge the four waves.  Each wave's output goes into its own first ring
  // slot (its last transpose reads have returned and its loads have landed),
  // its maximum and sum into ms / ls.
  const float l_tot = group4_sum(l_run);
  wait_counts<FA_VMCNT_LGKM0(0)>();
  float* __restrict__ ow = reinterpret_cast<float*>(Vs0[wave]);
  if (n16 < G) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4*>(ow + n16 * D + 16 * nb + 4 * g4) = oacc[nb];
    if (g4 == 0) {
      ms[wave][n16] = m_run;
      ls[wave][n16] = l_tot;
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += DGM_WAVES * 64) {
    const int h = i / D, d = i % D;
    float big = -INFINITY;
#pragma unroll
    for (int w = 0; w < DGM_WAVES; ++w) big = fmaxf(big, ms[w][h]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < DGM_WAVES; ++w) {
      if (ms[w][h] == -INFINITY) continue;  // a wave with no tile
      const float a = fast_exp2(ms[w][h] - big);
      lsum = __builtin_fmaf(a, ls[w][h], lsum);
      acc = __builtin_fmaf(a, reinterpret_cast<const float*>(Vs0[w])[h * D + d], acc);
    }
    part_o[((size_t)(h0 + h) * splits + split) * D + d] = acc / lsum;
    if (d == 0) part_lse[(size_t)(h0 + h) * splits + split] = (big + log2f(lsum)) * 0.69314718055994531f;
  }
}

// Kernel 2: one wave per head merges its chunk summaries.  The partial
// outputs of the first MERGE_PRE chunks are loaded together with the chunks'
// log-sum-exps, before their maximum is known, so that a merge of up to that
// many chunks waits for memory once.
constexpr int MERGE_PRE = 16;
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          T* __restrict__ O, float* __restrict__ LSE,
                                                          int splits) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* __restrict__ pl = part_lse + (size_t)bh * splits;
  const float* __restrict__ po = part_o + (size_t)bh * splits * D;
  constexpr int PER = D / 64;
  // Chunks past the last read the last one again (no branch around the
  // loads); their values are never used.
  float pre[MERGE_PRE][PER];
#pragma unroll
  for (int s = 0; s < MERGE_PRE; ++s)
#pragma unroll
    for (int i = 0; i < PER; ++i)
      pre[s][i] = po[(size_t)min(s, splits - 1) * D + lane + 64 * i];
  // Lane s holds the log-sum-exp of chunk s (of the first 64).
  const float lsev = lane < splits ? pl[lane] : -INFINITY;
  float big = lsev;
  for (int s = lane + 64; s < splits; s += 64) big = fmaxf(big, pl[s]);
  big = wave_max(big);
  if (big == -INFINITY) {  // no key at all (an empty history): O = 0, lse = -inf
    for (int i = lane; i < D; i += 64) O[(size_t)bh * D + i] = (T)0.f;
    if (LSE && lane == 0) LSE[bh] = -INFINITY;
    return;
  }
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  static_assert(MERGE_PRE <= 64, "the prefetched chunks' log-sum-exps are lanes of one wave");
#pragma unroll
  for (int s = 0; s < MERGE_PRE; ++s) {
    if (s < splits) {
      const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsev), s));
      const float w = expf(ls - big);  // exp(-inf) = 0 for empty chunks
      wsum += w;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w, pre[s][i], acc[i]);
    }
  }
  for (int s = MERGE_PRE; s < splits; ++s) {
    const float w = expf(pl[s] - big);
    wsum += w;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(w, po[(size_t)s * D + lane + 64 * i], acc[i]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int i = 0; i < PER; ++i) O[(size_t)bh * D + lane + 64 * i] = (T)(acc[i] * inv);
  if (LSE && lane == 0) LSE[bh] = big + logf(wsum);
}

// Query heads per workgroup of the matrix-core kernel: the largest divisor
// of the group that is at most 16.
static int decode_heads_per_wg(int group) {
  for (int g = group < DGM_MAX_G ? group : DGM_MAX_G; g > 1; --g)
    if (group % g == 0) return g;
  return 1;
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  // One query head per key/value head: the packed-dot-product kernel, which
  // streams at the chip's read rate.  Several: the matrix-core kernel, which
  // reads each chunk of K and V once for up to 16 of them.
  const int group = a.H / a.Hkv;
  hipError_t e;
  const float c = a.scale * 1.4426950408889634f;
  if (group == 1) {
    e = launch_kernel(decode_split_kernel<T, D>, dim3(a.B * a.H * a.splits), dim3(DEC_THREADS), s,
                      static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                      static_cast<const T*>(a.v), a.kv_lens, a.part_o, a.part_lse, a.Nkv, a.splits,
                      a.H, c);
  } else {
    const int g = decode_heads_per_wg(group);
    e = launch_kernel(decode_group_kernel<T, D>, dim3(a.B * a.H / g * a.splits),
                      dim3(DGM_WAVES * 64), s, static_cast<const T*>(a.q),
                      static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.kv_lens, a.part_o,
                      a.part_lse, a.Nkv, a.splits, a.Hkv, group, g, c);
  }
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
