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
// block are double-buffered in LDS, and the dQ product of a block runs at the
// start of the next step, so each step needs a single barrier.  The dQ
// atomics are issued before the step's matrix work: vector-memory counters
// track stores and atomics together with loads, so the wait for the
// prefetched tile at the end of the step would otherwise also wait for a
// fresh round trip of every atomic.
//
// LDS layout: row-major tiles without padding, 16-byte chunk c of row r
// stored at chunk c ^ sw(r).  For rows of 8 or more chunks sw(r) =
// 2 (r mod 4) + (r / 4 mod 2): eight consecutive rows then hit eight
// different chunks (16-byte row reads are conflict-free) and four consecutive
// rows hit four different chunk pairs (transpose reads are conflict-free).
// Rows of 4 chunks (the dS^T tile at 32 queries per step) use a 2-bit swizzle
// with the same transpose-read property.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int BWD_THREADS = 256;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 bwd_read_tr16(const void* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Chunk swizzle of row r for rows of at least 8 chunks (3 bits) and for rows
// of 4 chunks (2 bits: r bit 1 spreads the rows a transpose read touches,
// r bit 2 halves the conflicts of column writes).
template <int ROWLEN>
__device__ __forceinline__ int swz(int r) {
  static_assert(ROWLEN == 32 || ROWLEN % 64 == 0, "swizzle defined for 4 or >= 8 chunks per row");
  if (ROWLEN == 32) return (r & 2) | ((r >> 2) & 1);
  return ((r & 3) << 1) | ((r >> 2) & 1);
}

// Element offset of (row, col) in a swizzled row-major tile of ROWLEN elements.
template <int ROWLEN>
__device__ __forceinline__ int sw_off(int row, int col) {
  return row * ROWLEN + ((((col >> 3) ^ swz<ROWLEN>(row)) << 3) | (col & 7));
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
// KH = 32-key groups per wave (the workgroup owns BK = 128 KH keys), BQ =
// query rows per step.  Larger BK means fewer dQ atomics in total (each
// element of dQ receives one atomic add per key block).
template <typename T, int D, bool CAUSAL, int KH, int BQ>
__global__ __launch_bounds__(BWD_THREADS, 1) void bwd_main_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ drow,
    float* __restrict__ dq_acc, T* __restrict__ dK, T* __restrict__ dV, int N, int nkb,
    int total, float scale, float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  constexpr int BK = 128 * KH;
  constexpr int NB = D / 32;          // 32-column blocks of D
  constexpr int QB = BQ / 32;         // 32-row blocks of a query step
  constexpr int NDQ = NB * QB;        // 32x32 dQ output blocks per step
  __shared__ __attribute__((aligned(16))) T Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) T dSt[2][BK * BQ];  // dS^T: [key][query]
  __shared__ __attribute__((aligned(16))) T Kt[BK * D];       // this block's keys
  __shared__ __attribute__((aligned(16))) float Ls2[2][BQ];
  __shared__ __attribute__((aligned(16))) float Dsh[2][BQ];

  // Work item: XCD-local heads; causal key blocks heaviest (first) first.
  const int p = blockIdx.x;
  const int w = (total % 8 == 0) ? (p % 8) * (total / 8) + p / 8 : p;
  const int bh = w / nkb;
  const int kblk = w % nkb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_int(tid >> 6);  // wave-uniform
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
  const int kw0 = kj0 + 32 * KH * wave;  // first key of this wave
  int mykey[KH];                         // keys this lane owns in S, dP, dS
  bool key_ok[KH];
#pragma unroll
  for (int h = 0; h < KH; ++h) {
    mykey[h] = kw0 + 32 * h + l32;
    key_ok[h] = mykey[h] < N;
  }

  // K_w and V_w as B operands of S = Q K^T and dP = dO V^T.  With two key
  // groups per wave the register file holds the dK / dV accumulators and V_w
  // only, and the K_w operand is read from the block's K tile in LDS instead.
  constexpr bool KF_LDS = KH >= 2;
  v8 kf[KF_LDS ? 1 : KH][D / 16], vf[KH][D / 16];
#pragma unroll
  for (int h = 0; h < KH; ++h)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (!KF_LDS)
        kf[h][kk] = key_ok[h] ? ld16<v8>(Kh + (size_t)mykey[h] * D + 16 * kk + 8 * hh) : v8{};
      vf[h][kk] = key_ok[h] ? ld16<v8>(Vh + (size_t)mykey[h] * D + 16 * kk + 8 * hh) : v8{};
    }
  // The block's K rows in LDS (swizzled): the B operand of dQ = dS K comes
  // from transpose reads of it.  Rows past the end are zero.
  for (int e = tid; e < BK * D / 8; e += BWD_THREADS) {
    const int row = e / (D / 8), col = 8 * (e % (D / 8));
    u32x4 val = {0u, 0u, 0u, 0u};
    if (kj0 + row < N) val = *reinterpret_cast<const u32x4*>(Kh + (size_t)(kj0 + row) * D + col);
    *reinterpret_cast<u32x4*>(&Kt[sw_off<D>(row, col)]) = val;
  }

  f32x16 dvacc[KH][NB], dkacc[KH][NB];
#pragma unroll
  for (int h = 0; h < KH; ++h)
#pragma unroll
    for (int i = 0; i < NB; ++i) { dvacc[h][i] = f32x16{}; dkacc[h][i] = f32x16{}; }

  // Per-lane LDS offsets (elements).
  //  * 16-byte row reads of Q / dO (A operands of S and dP): row 32 qb + l32,
  //    chunk 2 kk + hh; the swizzle only changes the low 3 chunk bits, so the
  //    offset is rowoff[kk mod 4] plus 8 chunks for kk >= 4.
  int rowoff[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) rowoff[m] = sw_off<D>(l32, 16 * m + 8 * hh);
  //  * transpose reads (B operands of dK / dV from the Q / dO tiles, of dQ from
  //    the K tile, and the A operand of dQ from the dS^T tile): lane li of
  //    16-lane group grp addresses row 16 c + 8 t + trrow, column 32 b + trcol.
  //    In every case the reduction index (rows) comes out in the order the
  //    32x32 accumulator layout hands values to the other operand.
  const int trrow = 4 * hh + (li >> 2);
  const int trcol = 16 * (grp & 1) + 4 * (li & 3);

  // Q and dO tiles of a query step go straight from global memory into LDS
  // buffer `buf` (global_load_lds_dwordx4, no staging registers): wave w
  // fills 1 KiB segments w SPW .. w SPW + SPW - 1 of each tile, lane l of
  // segment g the LDS chunk slot l, i.e. tile row g RPS + l / (D / 8),
  // physical chunk l mod (D / 8), with the logical chunk the swizzle puts
  // there.  Rows past the end are clamped to row N-1 (their probabilities
  // are masked to 0).  L and D for the step's rows go through registers.
  constexpr int RPS = 512 / D;              // tile rows per 1 KiB segment
  constexpr int NSEG = BQ * D * 2 / 1024;   // segments per Q (or dO) tile
  constexpr int SPW = NSEG / 4;             // segments each wave loads
  static_assert(NSEG % 4 == 0 && BWD_THREADS == 256, "tile segments split evenly over the waves");
  float lpre = 0.f, dpre_row = 0.f;
  auto load_step = [&](int qi0, int buf) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int g = wave * SPW + i;
      const int row = g * RPS + lane / (D / 8);
      const int chunk = (lane % (D / 8)) ^ swz<D>(row);
      const size_t off = (size_t)min(qi0 + row, N - 1) * D + 8 * chunk;
      lds_load16(Qh + off, &Qs[buf][g * 512]);
      lds_load16(dOh + off, &dOs[buf][g * 512]);
    }
    if (tid < BQ) {
      const int qrow = qi0 + tid;
      lpre = (qrow < N) ? Lh[qrow] * 1.4426950408889634f : 0.f;
      dpre_row = (qrow < N) ? Dh[qrow] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
    if (tid < BQ) {
      Ls2[buf][tid] = lpre;
      Dsh[buf][tid] = dpre_row;
    }
  };

  // dQ for the query block whose dS^T sits in dSt[buf], starting at row qi0:
  // 32x32 output blocks wave, wave + 4, ... of the BQ x D block.
  auto dq_step = [&](int buf, int qi0) {
#pragma unroll
    for (int blk = wave; blk < NDQ; blk += 4) {
      const int nb = blk % NB, qb = blk / NB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ch = 0; ch < BK / 16; ++ch) {
        u32x2 pa[2], pk[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int row = 16 * ch + 8 * t + trrow;
          pa[t] = bwd_read_tr16(&dSt[buf][sw_off<BQ>(row, 32 * qb + trcol)]);
          pk[t] = bwd_read_tr16(&Kt[sw_off<D>(row, 32 * nb + trcol)]);
        }
        const u32x4 ca = {pa[0][0], pa[0][1], pa[1][0], pa[1][1]};
        const u32x4 ck = {pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
        acc = mfma32x32x16(__builtin_bit_cast(v8, ca), __builtin_bit_cast(v8, ck), acc);
      }
      // Element (row qrow, column 32 nb + l32) of this head's dQ accumulator,
      // addressed by a 32-bit offset from the head base (a head holds fewer
      // than 2^31 elements, which the host checks).
      const int off0 = (qi0 + 32 * qb + 4 * hh) * D + 32 * nb + l32;
      if (qi0 + BQ <= N) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          unsafeAtomicAdd(dQh + off0 + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = qi0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (qrow < N) unsafeAtomicAdd(dQh + off0 + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
        }
      }
    }
  };

  const int qstart = CAUSAL ? kj0 : 0;
  const int nsteps = (N - qstart + BQ - 1) / BQ;
  load_step(qstart, 0);
  store_step(0);
  wait_counts<FA_VMCNT_LGKM0(0)>();  // this wave's direct loads have landed
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    const int qi0 = qstart + it * BQ, buf = it & 1;
    // The previous block's dQ first: its atomics then drain while this block
    // is computed (the wait for the prefetched tile below also covers them).
    if (it > 0) dq_step(buf ^ 1, qi0 - BQ);
    if (it + 1 < nsteps) load_step(qi0 + BQ, buf ^ 1);  // buffer the previous step read

    const T* __restrict__ qt = Qs[buf];
    const T* __restrict__ dt = dOs[buf];
    // Let the scheduler interleave the LDS reads with the matrix products.
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      // S = Q K_w^T and dP = dO V_w^T (keys on the lanes), then P and dS.
      v8 pA[BQ / 16], dsA[BQ / 16];
      const bool need_mask = (CAUSAL && qi0 < kw0 + 32 * h + 31) || (qi0 + BQ > N) ||
                             (kw0 + 32 * h + 32 > N);
      // Visibility: query qi0 + ql sees key mykey iff ql >= mykey - qi0 (causal),
      // the query exists (ql < N - qi0) and the key exists.
      const int lo = CAUSAL ? mykey[h] - qi0 - 4 * hh : -(1 << 30);
      const int hi = (key_ok[h] ? N - qi0 : 0) - 4 * hh;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // Phase 1: S = Q K_w^T, then P (kept only in the storage type).
        f32x16 sa = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const int o = 32 * qb * D + rowoff[kk & 3] + 64 * (kk >> 2);
          const v8 aq = *reinterpret_cast<const v8*>(&qt[o]);
          const v8 bk = KF_LDS ? *reinterpret_cast<const v8*>(
                                     &Kt[(32 * KH * wave + 32 * h) * D + rowoff[kk & 3] + 64 * (kk >> 2)])
                               : kf[KF_LDS ? 0 : h][kk];
          sa = mfma32x32x16(aq, bk, sa);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls2[buf][32 * qb + 16 * hf + 8 * g2 + 4 * hh]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * hf + 4 * g2 + e;
              float pe = fast_exp2(__builtin_fmaf(sa[r], c, -l4[e]));
              if (need_mask) {
                const int qc = 32 * qb + 8 * (r >> 2) + (r & 3);  // query offset minus 4 hh
                pe = (qc >= lo && qc < hi) ? pe : 0.f;
              }
              pv[4 * g2 + e] = pe;
            }
          }
          pA[2 * qb + hf] = to_v8<T>(pv);
        }
        // Phase 2: dP = dO V_w^T, then dS = P o (dP - D) with P as rounded for
        // the P^T dO product (dS is rounded to the storage type as well).
        f32x16 dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const int o = 32 * qb * D + rowoff[kk & 3] + 64 * (kk >> 2);
          const v8 ad = *reinterpret_cast<const v8*>(&dt[o]);
          dp = mfma32x32x16(ad, vf[h][kk], dp);
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float dsv[8];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dsh[buf][32 * qb + 16 * hf + 8 * g2 + 4 * hh]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * hf + 4 * g2 + e;
              dsv[4 * g2 + e] = (float)pA[2 * qb + hf][4 * g2 + e] * (dp[r] - d4[e]);
            }
          }
          dsA[2 * qb + hf] = to_v8<T>(dsv);
          // dS^T row of this lane's key, queries 32 qb + 8 g + 4 hh + 0..3 (8-byte writes).
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            v4 q4;
#pragma unroll
            for (int e = 0; e < 4; ++e) q4[e] = dsA[2 * qb + hf][4 * g2 + e];
            *reinterpret_cast<u32x2*>(&dSt[buf][sw_off<BQ>(32 * KH * wave + 32 * h + l32,
                                                           32 * qb + 16 * hf + 8 * g2 + 4 * hh)]) =
                __builtin_bit_cast(u32x2, q4);
          }
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
          dvacc[h][nb] = mfma32x32x16(pA[kc], __builtin_bit_cast(v8, cd), dvacc[h][nb]);
          dkacc[h][nb] = mfma32x32x16(dsA[kc], __builtin_bit_cast(v8, cq), dkacc[h][nb]);
        }
    }

    if (it + 1 < nsteps) store_step(buf ^ 1);
    wait_counts<FA_VMCNT_LGKM0(0)>();  // this wave's direct loads have landed
    __syncthreads();
  }
  if (nsteps > 0) dq_step((nsteps - 1) & 1, qstart + (nsteps - 1) * BQ);

  // Write dK = scale * sum dS^T Q and dV = sum P^T dO for this wave's keys.
#pragma unroll
  for (int h = 0; h < KH; ++h)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kw0 + 32 * h + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key < N) {
          dK[hoff + (size_t)key * D + 32 * nb + l32] = (T)(dkacc[h][nb][r] * scale);
          dV[hoff + (size_t)key * D + 32 * nb + l32] = (T)dvacc[h][nb][r];
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

// Two shapes of the main kernel: 256 keys per workgroup halves the dQ atomics
// (the dominant cost at long sequence lengths) but makes each workgroup twice
// as long, which a short causal sequence cannot balance across the CUs.  The
// wider shape is used when it still yields at least four workgroups per CU.
#ifndef FA_BWD_FORCE_KH
#define FA_BWD_FORCE_KH 0
#endif

template <typename T, int D, bool CAUSAL, int KH, int BQ>
static hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t s) {
  const int nkb = (a.N + 128 * KH - 1) / (128 * KH);
  const int total = a.B * a.H * nkb;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL, KH, BQ>), dim3(total), dim3(BWD_THREADS), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.drow,
                     a.dq_acc, static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, nkb, total,
                     a.scale, c);
  return hipGetLastError();
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
  const long wide_blocks = (long)a.B * a.H * ((a.N + 255) / 256);
  const bool wide = FA_BWD_FORCE_KH ? FA_BWD_FORCE_KH == 2 : wide_blocks >= 4L * 256;
  e = wide ? launch_bwd_main<T, D, CAUSAL, 2, 32>(a, s) : launch_bwd_main<T, D, CAUSAL, 1, 64>(a, s);
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
