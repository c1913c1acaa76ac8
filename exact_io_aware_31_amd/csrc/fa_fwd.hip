// fa_fwd.hip -- fused exact attention forward for gfx950 (CDNA4).
//
// Method ("FlashAttention ontleed", § "Algoritmische kern in pseudocode";
// "03. FlashAttention", § "Mécanisme"; Lensa ML explainer, Steps 3-4): one
// workgroup owns a block of query rows; key/value tiles stream through LDS;
// for each tile the scores, the causal mask, the running max m and running
// sum l (with rescaling of the partial output) and the P V product all happen
// on chip, so neither S nor P is ever written to HBM.  After the last tile
// the output is divided by l and written once, together with
// lse = m + ln(l).
//
// MI355X mapping (not the pages' A100 tile rule):
//   * 4 waves x 32 query rows = 128 rows per workgroup, 64-key tiles.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//     each lane then owns ONE query row (column l % 32) and 16 of its scores
//     per 32-key block, so the row max / row sum are in-lane reductions plus
//     one v_permlane32_swap between the two wave halves.
//   * The probabilities stay in registers and feed O^T += V^T P^T directly
//     as the B operand: the accumulator layout of S^T is used as the operand
//     layout with a consistent permutation of the reduction index, and the
//     V tile is stored transposed in LDS in that same key order.
//   * exp2 with log2(e) folded into the scale (v_exp_f32).
//   * Causal: tiles entirely above the diagonal are never loaded; per wave,
//     tiles entirely above its 32 rows are skipped; only tiles that cross the
//     diagonal (or the ragged end) are masked element-wise.
//   * Grid: consecutive work items of one head are placed on one XCD (the
//     hardware deals workgroups round-robin over the 8 XCDs) so the head's
//     K/V stay in that XCD's L2; causal query blocks run heaviest first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 256;

// Position of key k (0 <= k < FWD_BC) inside a transposed V tile row.  Within
// each group of 16 keys the four quads are stored in the order 0, 2, 1, 3,
// which is the order in which the S^T accumulator hands probabilities to the
// two wave halves (see fa_common.h).
__device__ __forceinline__ int vt_pos_of_quad(int kq) {
  const int quad = kq & 3;
  const int perm = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
  return (kq >> 2) * 16 + perm * 4;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS, 2) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int N, int nqb, int total, float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  constexpr int BR = FWD_BR, BC = FWD_BC;
  constexpr int KSTR = D + 8;   // K tile row stride (elements); +16 B against bank conflicts
  constexpr int VSTR = BC + 8;  // V^T tile row stride (elements)
  __shared__ __attribute__((aligned(16))) T Ks[BC * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

  // Work item: XCD-local heads, heaviest causal query blocks first.
  const int p = blockIdx.x;
  const int w = (total % 8 == 0) ? (p % 8) * (total / 8) + p / 8 : p;
  const int bh = w / nqb;
  const int qb = CAUSAL ? nqb - 1 - (w % nqb) : (w % nqb);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * N * D;
  const T* __restrict__ Qh = Q + hoff;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;

  const int q0 = qb * BR + wave * 32;  // first query row of this wave
  const int myq = q0 + l32;            // the query row this lane owns

  // Q as the B operand of S^T = K Q^T: lane holds Q[myq][16 kk + 8 hh + 0..7].
  v8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (myq < N) qf[kk] = ld16<v8>(Qh + (size_t)myq * D + 16 * kk + 8 * hh);
    else qf[kk] = v8{};
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // running sum over this wave half's keys

  const int kv_end = CAUSAL ? min(N, qb * BR + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  for (int j = 0; j < ntiles; ++j) {
    const int kb = j * BC;
    __syncthreads();  // every wave is done reading the previous tile
    // K tile, row-major, 16-byte chunks (a wave covers 4 rows contiguously).
    constexpr int KCH = BC * D / 8;
#pragma unroll
    for (int e = tid; e < KCH; e += FWD_THREADS) {
      const int row = e / (D / 8), c8 = e % (D / 8);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (kb + row < N) val = *reinterpret_cast<const u32x4*>(Kh + (size_t)(kb + row) * D + 8 * c8);
      *reinterpret_cast<u32x4*>(&Ks[row * KSTR + 8 * c8]) = val;
    }
    // V tile, transposed: a thread moves 4 keys x 8 columns.
    constexpr int VUNITS = (BC / 4) * (D / 8);
#pragma unroll
    for (int u = tid; u < VUNITS; u += FWD_THREADS) {
      const int c8 = u % (D / 8), kq = u / (D / 8);
      v8 rows[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 4 * kq + i;
        rows[i] = (key < N) ? ld16<v8>(Vh + (size_t)key * D + 8 * c8) : v8{};
      }
      const int pos = vt_pos_of_quad(kq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v4 col = {rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
        *reinterpret_cast<u32x2*>(&Vt[(8 * c8 + e) * VSTR + pos]) = __builtin_bit_cast(u32x2, col);
      }
    }
    __syncthreads();
    if (CAUSAL && kb > q0 + 31) continue;  // whole tile above this wave's rows

    // S^T = K Q^T for BC/32 blocks of 32 keys.
    f32x16 sacc[BC / 32];
#pragma unroll
    for (int sb = 0; sb < BC / 32; ++sb) {
      sacc[sb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const v8 a = *reinterpret_cast<const v8*>(&Ks[(32 * sb + l32) * KSTR + 16 * kk + 8 * hh]);
        sacc[sb] = mfma32x32x16(a, qf[kk], sacc[sb]);
      }
    }

    // Mask keys past the end and, on diagonal tiles, keys after the query.
    const bool need_mask = (CAUSAL && kb + BC - 1 > q0) || (kb + BC > N);
    if (need_mask) {
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= N || (CAUSAL && key > myq)) sacc[sb][r] = -INFINITY;
        }
    }

    // Online softmax update for this lane's query row.
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
    mx = fmaxf(mx, other_half(mx));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = fast_exp2(m_run - m_new);
    float rs = 0.f;
    v8 pb[BC / 16];
#pragma unroll
    for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = fast_exp2(__builtin_fmaf(sacc[sb][8 * hf + e], c, -m_new));
          rs += pe;
          pv[e] = pe;
        }
        pb[2 * sb + hf] = to_v8<T>(pv);
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) oacc[nb] *= alpha;

    // O^T += V^T P^T.
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        const v8 a = *reinterpret_cast<const v8*>(&Vt[(32 * nb + l32) * VSTR + 16 * kc + 8 * hh]);
        oacc[nb] = mfma32x32x16(a, pb[kc], oacc[nb]);
      }
    m_run = m_new;
  }

  // Epilogue: O = O / l, lse = (m + log2 l) ln 2.
  const float l_tot = l_run + other_half(l_run);
  const float inv = 1.f / l_tot;
  if (myq < N) {
    T* __restrict__ orow = O + hoff + (size_t)myq * D;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v4 vals;
#pragma unroll
        for (int q = 0; q < 4; ++q) vals[q] = (T)(oacc[nb][4 * g + q] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * nb + 8 * g + 4 * hh) = __builtin_bit_cast(u32x2, vals);
      }
    if (hh == 0) LSE[(size_t)bh * N + myq] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.N + FWD_BR - 1) / FWD_BR;
  const int total = a.B * a.H * nqb;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3(total), dim3(FWD_THREADS), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, a.N, nqb, total, c);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_dt(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_fwd_t<T, 64, true>(a, s) : launch_fwd_t<T, 64, false>(a, s);
  return a.causal ? launch_fwd_t<T, 128, true>(a, s) : launch_fwd_t<T, 128, false>(a, s);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_fwd_dt<__bf16>(a, s) : launch_fwd_dt<_Float16>(a, s);
}

}  // namespace fa
