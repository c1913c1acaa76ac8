// fa_bwd.hip -- exact attention backward by recomputation, gfx950.
//
// Only O and the per-row log-sum-exp L are kept from the forward pass; the
// probabilities are rebuilt on chip from Q, K and L instead of being read
// back ("FlashAttention ontleed", § "Geheugencomplexiteit: van O(N²) naar
// O(N)"; "03. FlashAttention", § "Backward pass"; Lensa ML explainer, Step 5:
// recomputation adds arithmetic but moves fewer bytes).  The gradients are
// the plain calculus of O = softmax(scale Q K^T) V:
//     P  = exp(scale Q K^T - L)            dV = P^T dO
//     dP = dO V^T                           D_i = sum_k dO_ik O_ik
//     dS = P o (dP - D)                     dK = scale dS^T Q,  dQ = scale dS K
// (D_i equals sum_j P_ij dP_ij because each row of O is P_i V.)
//
// Three kernels on one stream:
//   1. bwd_pre:  D = rowsum(dO o O) in fp32 and a zeroed fp32 dQ accumulator.
//   2. bwd_main: one workgroup per (head, block of 128 keys); wave w owns 32
//      keys and keeps K_w, V_w and its dK, dV accumulators in registers while
//      it walks the query blocks (only blocks at or below the diagonal when
//      causal).  Per 64-query block: S and dP with v_mfma_f32_32x32x16 (keys
//      on the lanes), P and dS in registers, dV += P^T dO and dK += dS^T Q
//      straight from those registers (the same reduction-index permutation as
//      the forward), dS through LDS once so the four waves can form
//      dQ = dS K for the whole 128-key block, added to fp32 dQ with atomics.
//   3. bwd_dq:   dQ = scale * accumulator, rounded to the storage type.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int BWD_BK = 128;  // keys per workgroup (4 waves x 32)
constexpr int BWD_BQ = 64;   // query rows per inner step
constexpr int BWD_THREADS = 256;

// Same quad order as the forward's transposed V tile (see fa_fwd.hip).
__device__ __forceinline__ int tr_pos_of_quad(int kq) {
  const int quad = kq & 3;
  const int perm = (quad == 1) ? 2 : (quad == 2) ? 1 : quad;
  return (kq >> 2) * 16 + perm * 4;
}

// ---------------------------------------------------------------- kernel 1
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      float* __restrict__ drow,
                                                      float* __restrict__ dq_acc, long rows) {
  using v8 = typename Vec<T>::v8;
  constexpr int LPR = D / 8;  // lanes per row
  const long gt = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gt / LPR;
  const int col = (int)(gt % LPR);
  float s = 0.f;
  if (row < rows) {
    const v8 a = ld16<v8>(O + row * D + 8 * col);
    const v8 b = ld16<v8>(dO + row * D + 8 * col);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = __builtin_fmaf((float)a[i], (float)b[i], s);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dq_acc + row * D + 8 * col) = z;
    *reinterpret_cast<f32x4*>(dq_acc + row * D + 8 * col + 4) = z;
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < rows && col == 0) drow[row] = s;
}

// ---------------------------------------------------------------- kernel 2
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, 1) void bwd_main_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ drow,
    float* __restrict__ dq_acc, T* __restrict__ dK, T* __restrict__ dV, int N, int nkb,
    float scale, float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  constexpr int BK = BWD_BK, BQ = BWD_BQ;
  constexpr int RSTR = D + 8;    // row-major Q / dO tiles
  constexpr int TSTR = BQ + 8;   // transposed Q / dO tiles
  constexpr int SSTR = BK + 8;   // dS tile [query][key]
  __shared__ __attribute__((aligned(16))) T Qs[BQ * RSTR];
  __shared__ __attribute__((aligned(16))) T dOs[BQ * RSTR];
  __shared__ __attribute__((aligned(16))) T QsT[D * TSTR];
  __shared__ __attribute__((aligned(16))) T dOsT[D * TSTR];
  __shared__ __attribute__((aligned(16))) T dSs[BQ * SSTR];
  __shared__ float Ls2[BQ];
  __shared__ float Dsh[BQ];

  const int bh = blockIdx.x / nkb;
  const int kblk = CAUSAL ? nkb - 1 - (blockIdx.x % nkb) : (blockIdx.x % nkb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * N * D;
  const T* __restrict__ Qh = Q + hoff;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;
  const T* __restrict__ dOh = dO + hoff;
  const float* __restrict__ Lh = LSE + (size_t)bh * N;
  const float* __restrict__ Dh = drow + (size_t)bh * N;
  float* __restrict__ dQh = dq_acc + hoff;

  const int kj0 = kblk * BK;
  const int mykey = kj0 + 32 * wave + l32;  // key this lane owns in S, dP, dS
  const bool key_ok = mykey < N;

  // K_w and V_w as B operands of S = Q K^T and dP = dO V^T.
  v8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kf[kk] = key_ok ? ld16<v8>(Kh + (size_t)mykey * D + 16 * kk + 8 * hh) : v8{};
    vf[kk] = key_ok ? ld16<v8>(Vh + (size_t)mykey * D + 16 * kk + 8 * hh) : v8{};
  }
  // K as the B operand of dQ = dS K for this wave's column block(s) of dQ:
  // lane holds K[kj0 + 16 ch + 8 hh + e][32 nb + l32], e = 0..7.
  constexpr int NB = D / 32;          // column blocks of dQ
  constexpr int QB = BQ / 32;         // row blocks of dQ
  constexpr int PER_WAVE = NB * QB / 4;
  const int nb_q = wave % NB;
  v8 ktf[BK / 16];
#pragma unroll
  for (int ch = 0; ch < BK / 16; ++ch) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kj0 + 16 * ch + 8 * hh + e;
      ktf[ch][e] = (key < N) ? Kh[(size_t)key * D + 32 * nb_q + l32] : (T)0.f;
    }
  }

  f32x16 dvacc[NB], dkacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) { dvacc[i] = f32x16{}; dkacc[i] = f32x16{}; }

  const int qstart = CAUSAL ? kj0 : 0;
  for (int qi0 = qstart; qi0 < N; qi0 += BQ) {
    __syncthreads();  // previous step's readers of the shared tiles are done
    // Stage Q_i and dO_i, row-major and transposed; L (log2 units) and D.
    constexpr int UNITS = (BQ / 4) * (D / 8);
#pragma unroll
    for (int u = tid; u < UNITS; u += BWD_THREADS) {
      const int c8 = u % (D / 8), kq = u / (D / 8);
      v8 qr[4], dr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qrow = qi0 + 4 * kq + i;
        qr[i] = (qrow < N) ? ld16<v8>(Qh + (size_t)qrow * D + 8 * c8) : v8{};
        dr[i] = (qrow < N) ? ld16<v8>(dOh + (size_t)qrow * D + 8 * c8) : v8{};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<v8*>(&Qs[(4 * kq + i) * RSTR + 8 * c8]) = qr[i];
        *reinterpret_cast<v8*>(&dOs[(4 * kq + i) * RSTR + 8 * c8]) = dr[i];
      }
      const int pos = tr_pos_of_quad(kq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v4 qc = {qr[0][e], qr[1][e], qr[2][e], qr[3][e]};
        v4 dc = {dr[0][e], dr[1][e], dr[2][e], dr[3][e]};
        *reinterpret_cast<u32x2*>(&QsT[(8 * c8 + e) * TSTR + pos]) = __builtin_bit_cast(u32x2, qc);
        *reinterpret_cast<u32x2*>(&dOsT[(8 * c8 + e) * TSTR + pos]) = __builtin_bit_cast(u32x2, dc);
      }
    }
    if (tid < BQ) {
      const int qrow = qi0 + tid;
      Ls2[tid] = (qrow < N) ? Lh[qrow] * 1.4426950408889634f : 0.f;
      Dsh[tid] = (qrow < N) ? Dh[qrow] : 0.f;
    }
    __syncthreads();

    // S = Q K_w^T and dP = dO V_w^T; P and dS stay in registers.
    v8 pA[BQ / 16], dsA[BQ / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const v8 aq = *reinterpret_cast<const v8*>(&Qs[(32 * qb + l32) * RSTR + 16 * kk + 8 * hh]);
        s = mfma32x32x16(aq, kf[kk], s);
        const v8 ad = *reinterpret_cast<const v8*>(&dOs[(32 * qb + l32) * RSTR + 16 * kk + 8 * hh]);
        dp = mfma32x32x16(ad, vf[kk], dp);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);  // query row in the block
        const int qrow = qi0 + ql;
        const bool ok = key_ok && qrow < N && (!CAUSAL || mykey <= qrow);
        const float pe = ok ? fast_exp2(__builtin_fmaf(s[r], c, -Ls2[ql])) : 0.f;
        pv[r] = pe;
        dsv[r] = pe * (dp[r] - Dsh[ql]);
        dSs[ql * SSTR + 32 * wave + l32] = (T)dsv[r];
      }
      pA[2 * qb] = to_v8<T>(pv);
      pA[2 * qb + 1] = to_v8<T>(pv + 8);
      dsA[2 * qb] = to_v8<T>(dsv);
      dsA[2 * qb + 1] = to_v8<T>(dsv + 8);
    }

    // dV_w += P^T dO_i and dK_w += dS^T Q_i (scale applied at the end).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kc = 0; kc < BQ / 16; ++kc) {
        const v8 bd = *reinterpret_cast<const v8*>(&dOsT[(32 * nb + l32) * TSTR + 16 * kc + 8 * hh]);
        dvacc[nb] = mfma32x32x16(pA[kc], bd, dvacc[nb]);
        const v8 bq = *reinterpret_cast<const v8*>(&QsT[(32 * nb + l32) * TSTR + 16 * kc + 8 * hh]);
        dkacc[nb] = mfma32x32x16(dsA[kc], bq, dkacc[nb]);
      }
    __syncthreads();  // the whole dS block is in LDS

    // dQ_i += dS K over all 128 keys, this wave's output blocks.
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int qb = wave / NB + j * (4 / NB);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ch = 0; ch < BK / 16; ++ch) {
        const v8 a = *reinterpret_cast<const v8*>(&dSs[(32 * qb + l32) * SSTR + 16 * ch + 8 * hh]);
        acc = mfma32x32x16(a, ktf[ch], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = qi0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (qrow < N) unsafeAtomicAdd(dQh + (size_t)qrow * D + 32 * nb_q + l32, acc[r]);
      }
    }
  }

  // Write dK = scale * sum dS^T Q and dV = sum P^T dO for this wave's keys.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kj0 + 32 * wave + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key < N) {
        dK[hoff + (size_t)key * D + 32 * nb + l32] = (T)(dkacc[nb][r] * scale);
        dV[hoff + (size_t)key * D + 32 * nb + l32] = (T)dvacc[nb][r];
      }
    }
}

// ---------------------------------------------------------------- kernel 3
template <typename T>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc,
                                                     T* __restrict__ dQ, long n8, float scale) {
  using v8 = typename Vec<T>::v8;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(acc + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(acc + 8 * i + 4);
  v8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = (T)(a[e] * scale); r[4 + e] = (T)(b[e] * scale); }
  st16<v8>(dQ + 8 * i, r);
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.H * a.N;
  const long pre_threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256),
                     0, s, static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.drow,
                     a.dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.N + BWD_BK - 1) / BWD_BK;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL>), dim3(a.B * a.H * nkb), dim3(BWD_THREADS), 0,
                     s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.drow,
                     a.dq_acc, static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, nkb, a.scale, c);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n8 = rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_kernel<T>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     a.dq_acc, static_cast<T*>(a.dq), n8, a.scale);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_dt(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch_bwd_t<T, 64, true>(a, s) : launch_bwd_t<T, 64, false>(a, s);
  return a.causal ? launch_bwd_t<T, 128, true>(a, s) : launch_bwd_t<T, 128, false>(a, s);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_bwd_dt<__bf16>(a, s) : launch_bwd_dt<_Float16>(a, s);
}

size_t bwd_dq_acc_bytes(int B, int H, int N, int d) {
  return align256((size_t)B * H * N * d * sizeof(float));
}
size_t bwd_drow_bytes(int B, int H, int N) { return align256((size_t)B * H * N * sizeof(float)); }

}  // namespace fa
