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
//      straight from those registers (the B operands dO^T and Q^T come from
//      the row-major tiles through the LDS transpose read), dS^T through LDS
//      once so the four waves can form dQ = dS K for the whole 128-key block,
//      added to the fp32 dQ accumulator with atomics.
//   3. bwd_dq:   dQ = scale * accumulator, rounded to the storage type.
//
// Pipelining in bwd_main: the next query block's Q, dO, L and D are loaded
// into registers while the current block is computed; tiles and the dS^T
// block are double-buffered in LDS, and the dQ product of a block runs one
// step later, so each step needs a single barrier.
//
// LDS layout: row-major tiles without padding, 16-byte chunk c of row r
// stored at chunk c ^ sw(r), sw(r) = 2 (r mod 4) + (r / 4 mod 2).  Eight
// consecutive rows then hit eight different chunks (16-byte row reads are
// conflict-free) and four consecutive rows hit four different chunk pairs
// (transpose reads are conflict-free).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int BWD_BK = 128;  // keys per workgroup (4 waves x 32)
constexpr int BWD_BQ = 64;   // query rows per step
constexpr int BWD_THREADS = 256;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 bwd_read_tr16(const void* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Element offset of (row, col) in a swizzled row-major tile of ROWLEN elements.
template <int ROWLEN>
__device__ __forceinline__ int sw_off(int row, int col) {
  return row * ROWLEN + ((((col >> 3) ^ swz(row)) << 3) | (col & 7));
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
    int total, float scale, float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  constexpr int BK = BWD_BK, BQ = BWD_BQ;
  constexpr int NB = D / 32;          // 32-column blocks of D
  constexpr int QB = BQ / 32;         // 32-row blocks of a query step
  constexpr int CH = BQ * D / 8;      // 16-byte chunks per Q (or dO) tile
  constexpr int CPT = CH / BWD_THREADS;
  static_assert(CH % BWD_THREADS == 0, "tile chunks must divide evenly");
  __shared__ __attribute__((aligned(16))) T Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T dSt[2][BK * BQ];  // dS^T: [key][query]
  __shared__ __attribute__((aligned(16))) float Ls2[2][BQ];
  __shared__ __attribute__((aligned(16))) float Dsh[2][BQ];

  // Work item: XCD-local heads; causal key blocks heaviest (first) first.
  const int p = blockIdx.x;
  const int w = (total % 8 == 0) ? (p % 8) * (total / 8) + p / 8 : p;
  const int bh = w / nkb;
  const int kblk = w % nkb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int li = lane & 15, grp = lane >> 4;
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
  // K as the B operand of dQ = dS K, in the key order the transpose read of
  // dS^T produces: element e of lane half hh is key 8 (e / 4) + 4 hh + (e % 4)
  // of each 16-key chunk; column 32 nb_q + l32.
  constexpr int PER_WAVE = NB * QB / 4;  // dQ output blocks per wave
  const int nb_q = wave % NB;
  v8 ktf[BK / 16];
#pragma unroll
  for (int ch = 0; ch < BK / 16; ++ch)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kj0 + 16 * ch + 8 * (e >> 2) + 4 * hh + (e & 3);
      ktf[ch][e] = (key < N) ? Kh[(size_t)key * D + 32 * nb_q + l32] : (T)0.f;
    }

  f32x16 dvacc[NB], dkacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) { dvacc[i] = f32x16{}; dkacc[i] = f32x16{}; }

  // Per-lane LDS offsets (elements).
  //  * 16-byte row reads of Q / dO (A operands of S and dP): row 32 qb + l32,
  //    chunk 2 kk + hh; the swizzle only changes the low 3 chunk bits, so the
  //    offset is rowoff[kk mod 4] plus 8 chunks for kk >= 4.
  int rowoff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) rowoff[m] = sw_off<D>(l32, 16 * m + 8 * hh);
  //  * transpose reads of Q / dO (B operands of dK / dV): rows 16 kc + 8 t +
  //    4 hh + li / 4, columns 32 nb + 16 (grp mod 2) + 4 (li mod 4).
  const int trrow = 4 * hh + (li >> 2);
  const int trcol = 16 * (grp & 1) + 4 * (li & 3);
  //  * transpose reads of dS^T (A operand of dQ): rows (keys) 16 ch + 8 t +
  //    4 hh + li / 4, columns (queries) 32 qb + 16 (grp mod 2) + 4 (li mod 4).
  // Swizzle of a row depends only on row mod 8 = 8 t + trrow mod 8 = trrow + 8t.

  u32x4 qpre[CPT], dpre[CPT];
  float lpre = 0.f, dpre_row = 0.f;
  auto load_step = [&](int qi0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int e = tid + i * BWD_THREADS;
      const int row = min(qi0 + e / (D / 8), N - 1), c8 = e % (D / 8);
      const size_t off = (size_t)row * D + 8 * c8;
      qpre[i] = *reinterpret_cast<const u32x4*>(Qh + off);
      dpre[i] = *reinterpret_cast<const u32x4*>(dOh + off);
    }
    if (tid < BQ) {
      const int qrow = qi0 + tid;
      lpre = (qrow < N) ? Lh[qrow] * 1.4426950408889634f : 0.f;
      dpre_row = (qrow < N) ? Dh[qrow] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int e = tid + i * BWD_THREADS;
      const int row = e / (D / 8), col = 8 * (e % (D / 8));
      *reinterpret_cast<u32x4*>(&Qs[buf][sw_off<D>(row, col)]) = qpre[i];
      *reinterpret_cast<u32x4*>(&dOs[buf][sw_off<D>(row, col)]) = dpre[i];
    }
    if (tid < BQ) {
      Ls2[buf][tid] = lpre;
      Dsh[buf][tid] = dpre_row;
    }
  };

  // dQ for the query block whose dS^T sits in dSt[buf], starting at row qi0.
  auto dq_step = [&](int buf, int qi0) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int qb = wave / NB + j * (4 / NB);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ch = 0; ch < BK / 16; ++ch) {
        u32x2 part[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = 16 * ch + 8 * t + trrow;
          part[t] = bwd_read_tr16(&dSt[buf][sw_off<BQ>(row, 32 * qb + trcol)]);
        }
        const u32x4 cat = {part[0][0], part[0][1], part[1][0], part[1][1]};
        acc = mfma32x32x16(__builtin_bit_cast(v8, cat), ktf[ch], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = qi0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (qrow < N) unsafeAtomicAdd(dQh + (size_t)qrow * D + 32 * nb_q + l32, acc[r]);
      }
    }
  };

  const int qstart = CAUSAL ? kj0 : 0;
  const int nsteps = (N - qstart + BQ - 1) / BQ;
  load_step(qstart);
  store_step(0);
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    const int qi0 = qstart + it * BQ, buf = it & 1;
    if (it + 1 < nsteps) load_step(qi0 + BQ);

    const T* __restrict__ qt = Qs[buf];
    const T* __restrict__ dt = dOs[buf];
    // S = Q K_w^T and dP = dO V_w^T (keys on the lanes), then P and dS.
    v8 pA[BQ / 16], dsA[BQ / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int o = 32 * qb * D + rowoff[kk & 3] + 64 * (kk >> 2);
        const v8 aq = *reinterpret_cast<const v8*>(&qt[o]);
        const v8 ad = *reinterpret_cast<const v8*>(&dt[o]);
        s = mfma32x32x16(aq, kf[kk], s);
        dp = mfma32x32x16(ad, vf[kk], dp);
      }
      // Visibility: query qi0 + ql sees key mykey iff ql >= mykey - qi0 (causal),
      // the query exists (ql < N - qi0) and the key exists.
      const int lo = CAUSAL ? mykey - qi0 - 4 * hh : -(1 << 30);
      const int hi = (key_ok ? N - qi0 : 0) - 4 * hh;
      f32x4 lrow[4], drw[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lrow[g] = *reinterpret_cast<const f32x4*>(&Ls2[buf][32 * qb + 8 * g + 4 * hh]);
        drw[g] = *reinterpret_cast<const f32x4*>(&Dsh[buf][32 * qb + 8 * g + 4 * hh]);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qc = 32 * qb + 8 * (r >> 2) + (r & 3);  // query offset minus 4 hh
        const float pe = fast_exp2(__builtin_fmaf(s[r], c, -lrow[r >> 2][r & 3]));
        pv[r] = (qc >= lo && qc < hi) ? pe : 0.f;
        dsv[r] = pv[r] * (dp[r] - drw[r >> 2][r & 3]);
      }
      pA[2 * qb] = to_v8<T>(pv);
      pA[2 * qb + 1] = to_v8<T>(pv + 8);
      dsA[2 * qb] = to_v8<T>(dsv);
      dsA[2 * qb + 1] = to_v8<T>(dsv + 8);
      // dS^T row mykey, queries 32 qb + 8 g + 4 hh + 0..3 (8-byte writes).
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v4 q4;
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] = (T)dsv[4 * g + e];
        *reinterpret_cast<u32x2*>(&dSt[buf][sw_off<BQ>(32 * wave + l32, 32 * qb + 8 * g + 4 * hh)]) =
            __builtin_bit_cast(u32x2, q4);
      }
    }

    // dV_w += P^T dO_i and dK_w += dS^T Q_i (scale applied at the end); the
    // B operands come from transpose reads of the row-major tiles.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kc = 0; kc < BQ / 16; ++kc) {
        u32x2 pd[2], pq[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int o = sw_off<D>(16 * kc + 8 * t + trrow, 32 * nb + trcol);
          pd[t] = bwd_read_tr16(&dt[o]);
          pq[t] = bwd_read_tr16(&qt[o]);
        }
        const u32x4 cd = {pd[0][0], pd[0][1], pd[1][0], pd[1][1]};
        const u32x4 cq = {pq[0][0], pq[0][1], pq[1][0], pq[1][1]};
        dvacc[nb] = mfma32x32x16(pA[kc], __builtin_bit_cast(v8, cd), dvacc[nb]);
        dkacc[nb] = mfma32x32x16(dsA[kc], __builtin_bit_cast(v8, cq), dkacc[nb]);
      }

    if (it > 0) dq_step(buf ^ 1, qi0 - BQ);  // previous block's dS^T is complete
    if (it + 1 < nsteps) store_step(buf ^ 1);
    __syncthreads();
  }
  if (nsteps > 0) dq_step((nsteps - 1) & 1, qstart + (nsteps - 1) * BQ);

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
  const int total = a.B * a.H * nkb;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL>), dim3(total), dim3(BWD_THREADS), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.drow,
                     a.dq_acc, static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, nkb, total,
                     a.scale, c);
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
