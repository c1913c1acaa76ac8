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
// Three kernels, none of which uses atomics (every output element is written
// once, by one lane, and partial sums are added in a fixed order, so the
// results are deterministic); on small grids and with grouped heads the
// third runs on a second stream beside the second (see the launchers):
//   1. bwd_pre: D = rowsum(dO o O) in fp32.
//   2. bwd_kv:  dK and dV.  One workgroup of 4 waves per block of 128 keys;
//      wave w owns 32 keys and keeps V_w and its dK, dV accumulators in
//      registers while it walks the 32-query steps (only steps at or below the
//      diagonal when causal).  Per step: S = Q K_w^T and dP = dO V_w^T with
//      v_mfma_f32_32x32x16 (keys on the lanes), P and dS in registers, then
//      dV += P^T dO and dK += dS^T Q straight from those registers; the B
//      operands dO and Q come from transpose reads of the row-major tiles.
//      The kernel fits in 256 registers, so two workgroups share a CU (two
//      waves per SIMD hide each other's LDS and MFMA latencies).  On tiny
//      grids a block has 64 or 32 keys, and the two or four waves that own
//      the same keys take alternate query steps, then add their dK and dV
//      through LDS.
//   3. bwd_dq:  dQ, with the forward pass's shape: one workgroup of 8 waves
//      per block of 256 query rows, 64-key K and V tiles streaming through a
//      three-deep LDS ring, and transposed products so that each lane owns
//      one query row:
//          S^T  = K Q^T,    dP^T = V dO^T     (Q and dO rows in registers)
//          dS^T = P^T o (dP^T - D),  P^T = exp2(c S^T - L log2 e)
//          dQ^T += K^T dS^T                   (K^T by transpose reads)
//      dS^T never leaves the registers: its accumulator layout is used as the
//      B operand layout of the last product.
// Splitting dK/dV from dQ recomputes S and dP once more, but a fused kernel
// must either sum dQ over key blocks with atomics or sum dK, dV over query
// blocks the same way; the extra matrix work costs less than either.
//
// LDS tiles use the forward's unpadded, swizzled layout (fa_tile.h: 16-byte
// row reads and transpose reads conflict-free) and are filled by direct
// buffer-to-LDS loads (TileLoader).
#include <mutex>

#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

// ---------------------------------------------------------------- kernel 1
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O,
                                                      const T* __restrict__ dO,
                                                      float* __restrict__ drow, long rows) {
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
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < rows && col == 0) drow[row] = s;
}

// p, an address in LDS, with its provenance hidden from the compiler: it
// cannot tell which shared array the result points into.
template <typename T>
__device__ __forceinline__ T* opaque_lds(T* p) {
  uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
  asm volatile("" : "+s"(a));
  return (T*)(__attribute__((address_space(3))) T*)(uintptr_t)a;
}

// ---------------------------------------------------------------- kernel 2
constexpr int KV_WAVES = 4;
constexpr int KV_BK = 32 * KV_WAVES;  // keys per workgroup
constexpr int KV_BQ = 32;             // query rows per step
constexpr int KV_READ_AHEAD = 3;      // S / dP MFMAs whose LDS operands are read ahead

template <typename T, int D, bool CAUSAL, bool WIN, int QS>
__global__ __launch_bounds__(KV_WAVES * 64, QS == 1 ? 2 : 1) void bwd_kv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ drow,
    T* __restrict__ dK, T* __restrict__ dV, int N, int nkb, int total, int group, int window,
    float scale, float c) {
  using v8 = typename Vec<T>::v8;
  if constexpr (!WIN) window = 0;  // window code only in the WIN instantiation
  // QS > 1 splits the query steps inside the workgroup (tiny grids): the
  // QS waves that own the same 32 keys take every QS-th query step each
  // (QS = 2: waves w and w + 2, even and odd steps, 64 keys per block; QS =
  // 4: all four waves, 32 keys), then merge their dK and dV at the end.  The
  // Q / dO ring holds QS query tiles per step (81 / 138 KiB of LDS at d =
  // 128), so one such workgroup runs per CU, with registers to match.
  static_assert(QS == 1 || QS == 2 || QS == 4, "query steps split in 1, 2 or 4");
  constexpr int KWAVES = KV_WAVES / QS;  // waves per set of the block's keys
  constexpr int BK = 32 * KWAVES, BQ = KV_BQ, NB = D / 32;
  constexpr int SPW_Q = BQ * D * 2 / 1024 / KV_WAVES;  // load segments per wave per Q tile
  __shared__ __attribute__((aligned(1024))) T Qs[2][QS * BQ * D];
  __shared__ __attribute__((aligned(1024))) T dOs[2][QS * BQ * D];
  __shared__ __attribute__((aligned(1024))) T Ks[BK * D];  // this block's keys
  __shared__ __attribute__((aligned(16))) float Ls[2][QS * BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][QS * BQ];

  // Work item: XCD-local heads; causal key blocks heaviest (first) first.
  int kvbh, kblk;  // key/value head (over B x H_kv), key block
  work_item(blockIdx.x, total / nkb, nkb, CAUSAL && !WIN, kvbh, kblk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_int(tid >> 6);  // wave-uniform
  const int kw = QS == 1 ? wave : wave % KWAVES;  // the wave's set of 32 keys
  const int qp = QS == 1 ? 0 : wave / KWAVES;     // the wave's step of each pair
  const int l32 = lane & 31, hh = lane >> 5;
  const int li = lane & 15, grp = lane >> 4;
  // K, V, dK, dV of key/value head kvbh; the query heads of its group are
  // kvbh * group .. kvbh * group + group - 1, and this block's dK, dV sum
  // over all of them.
  const size_t hoff = (size_t)kvbh * N * D;
  const int qh0 = kvbh * group;
  const T* __restrict__ Kh = K + hoff;
  const T* __restrict__ Vh = V + hoff;

  const int kj0 = kblk * BK;
  const int kw0 = kj0 + 32 * kw;  // first key of this wave
  const int mykey = kw0 + l32;      // the key this lane owns in S, dP, dS
  const bool key_ok = mykey < N;

  // V_w as the B operand of dP = dO V_w^T.  K_w, the B operand of S = Q K_w^T,
  // is read from the block's K tile in LDS (registers hold the accumulators).
  v8 vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    vf[kk] = key_ok ? ld16<v8>(Vh + (size_t)mykey * D + 16 * kk + 8 * hh) : v8{};
  // Rows past the end read as zero; those keys' scores are masked.
  TileLoader<D, BK, KV_WAVES>(wave, lane).load(Kh, N, kj0, Ks, wave);

  f32x16 dvacc[NB], dkacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) { dvacc[i] = f32x16{}; dkacc[i] = f32x16{}; }

  // LDS byte offsets by XOR addressing (fa_tile.h): 16-byte row reads (row
  // l32, columns 16 kk + 8 hh: A operands Q and dO of S and dP, B operand K_w
  // of S) and transpose reads (B operands of dK / dV from the Q / dO tiles:
  // row 16 kc + 8 t + 4 hh + li / 4, column 32 nb + 16 (grp mod 2) +
  // 4 (li mod 4)).  Three base registers and one XOR per read replace a table
  // of sixteen offsets, which this kernel has no registers for.  The
  // transpose reads hand the reduction index (query) over in the order the
  // 32x32 accumulator layout gives P and dS to the A operand.
  const uint32_t rb = tile_row_base<D>(l32, hh);
  const uint32_t tb = tile_tr_base<D>(4 * hh + (li >> 2), 16 * (grp & 1) + 4 * (li & 3));
  const uint32_t kwb = rb + 64 * D * kw;  // this wave's 32 K rows: 32 D * 2 bytes per wave

  // Q and dO tiles of a step go straight into LDS buffer `buf` (rows past the
  // end read as zero, their probabilities masked to 0); L and D of the step's
  // rows go through registers.
  // Steps run over the group's query heads, each over query rows qstart ..
  // qend - 1: causal blocks start at their first key; with a window, queries
  // from the block's last key + window on see none of its keys.
  const int qstart = CAUSAL ? kj0 : 0;
  const int qend = (CAUSAL && window > 0) ? min(N, kj0 + BK - 1 + window) : N;
  const int nsh = (qend - qstart + BQ - 1) / BQ;  // steps per query head
  const int nsteps = group * nsh;
  // (query head, first row) of a step, advanced step by step (no divisions).
  auto advance = [&](int& qh, int& q0) {
    q0 += BQ;
    if (q0 >= qend) {
      q0 = qstart;
      ++qh;
    }
  };
  float lraw = 0.f, draw = 0.f;
  const TileLoader<D, BQ, KV_WAVES> step_loader(wave, lane);
  // Loads the QS query tiles of the steps from index si on (head qh, first
  // row qi0) into ring slot buf; a tile past the last step reads nothing
  // (first row N: its slot fills with zeros and no wave computes it).
  auto load_step = [&](int qh, int qi0, int buf, int si) {
    if constexpr (QS == 1) {
      const size_t qoff = (size_t)qh * N * D;
      step_loader.load(Q + qoff, N, qi0, opaque_lds(Qs[buf]), wave);
      step_loader.load(dO + qoff, N, qi0, opaque_lds(dOs[buf]), wave);
      const uint32_t bytes = (uint32_t)(N - qi0) * 4u;
      lraw = buffer_load_f32(LSE + (size_t)qh * N + qi0, bytes, 4u * l32);
      draw = buffer_load_f32(drow + (size_t)qh * N + qi0, bytes, 4u * l32);
      return;
    }
#pragma unroll
    for (int tq = 0; tq < QS; ++tq) {
      if (tq > 0) advance(qh, qi0);
      const bool ok = QS == 1 || si + tq < nsteps;
      const int h = ok ? qh : qh0, r0 = ok ? qi0 : N;
      const size_t qoff = (size_t)h * N * D;
      // The direct loads name their ring slot through an opaque LDS address.
      // Loads into a slot the compiler can trace (the Qs / dOs arrays) make it
      // wait for them before every later read of the same array, including
      // the reads of the other slot, which is this step's: the next step's
      // tiles would have to arrive before this step could start.  The slots
      // are ordered by the wait and the barrier that end every step instead.
      step_loader.load(Q + qoff, N, r0, opaque_lds(Qs[buf] + tq * BQ * D), wave);
      step_loader.load(dO + qoff, N, r0, opaque_lds(dOs[buf] + tq * BQ * D), wave);
      // Rows r0 + l32 of the head's L and D (for this wave's own step)
      // through a buffer descriptor of the rows from r0 on: rows past the end
      // read as zero (their probabilities are masked), and no lane holds a
      // 64-bit address.  Every lane loads (no branch around loads); the
      // values are used only when stored at the end of the step, so nothing
      // waits for them before.
      if (tq == qp) {
        const uint32_t bytes = (uint32_t)(N - r0) * 4u;
        lraw = buffer_load_f32(LSE + (size_t)h * N + r0, bytes, 4u * l32);
        draw = buffer_load_f32(drow + (size_t)h * N + r0, bytes, 4u * l32);
      }
    }
  };
  auto store_step = [&](int buf) {
    if constexpr (QS == 1) {
      if (tid < BQ) {
        Ls[buf][tid] = lraw * 1.4426950408889634f;
        Ds[buf][tid] = draw;
      }
    } else if (kw == 0 && lane < BQ) {
      Ls[buf][qp * BQ + lane] = lraw * 1.4426950408889634f;
      Ds[buf][qp * BQ + lane] = draw;
    }
  };
  static_assert(SPW_Q >= 1, "each wave loads part of every tile");

  const int nss = (nsteps + QS - 1) / QS;  // steps of the ring (QS query steps each)
  int ld_h = qh0, ld_q = qstart;  // first query step being loaded
  int cu_h = qh0, cu_q = qstart;  // first query step being computed
  load_step(ld_h, ld_q, 0, 0);
  store_step(0);
  wait_counts<FA_VMCNT_LGKM0(0)>();  // this wave's direct loads (K tile included) have landed
  __syncthreads();

  for (int it = 0; it < nss; ++it) {
    int qi0 = cu_q;
    const int buf = it & 1;
    if constexpr (QS > 1) {  // this wave's step: qp steps after the pair's (group's) first
      int h1 = cu_h;
      for (int tq = 0; tq < qp; ++tq) advance(h1, qi0);
      (void)h1;
    }
    if (it + 1 < nss) {  // into the buffer the previous step read
#pragma unroll
      for (int tq = 0; tq < QS; ++tq) advance(ld_h, ld_q);
      load_step(ld_h, ld_q, buf ^ 1, QS * (it + 1));
    }
    // (QS = 2: a wave whose step is past the last one computes nothing.)
    if (QS == 1 || QS * it + qp < nsteps) {

    // This step's buffer: tiles are 32 D * 2 bytes apart, above every in-tile
    // offset, so adding the buffer offset commutes with the XORs.  The empty
    // asm makes the bases opaque, so the XORs stay in the loop rather than
    // being hoisted into sixteen loop-invariant registers.
    uint32_t rbs = rb + buf * (QS * BQ * D * 2) + qp * (BQ * D * 2),
             tbs = tb + buf * (QS * BQ * D * 2) + qp * (BQ * D * 2), kws = kwb;
    asm volatile("" : "+v"(rbs), "+v"(tbs), "+v"(kws));
    // Visibility: query qi0 + ql sees key mykey iff ql >= mykey - qi0 (causal),
    // the query exists (ql < N - qi0) and the key exists.
    // Window: query qi0 + ql also needs ql < mykey + window - qi0.
    const bool need_mask = (CAUSAL && qi0 < kw0 + 31) || (qi0 + BQ > N) || (kw0 + 32 > N) ||
                           (CAUSAL && window > 0 && qi0 + BQ - 1 >= kw0 + window);
    const int lo = CAUSAL ? mykey - qi0 - 4 * hh : -(1 << 30);
    const int hi = (key_ok ? min(N - qi0, (CAUSAL && window > 0) ? mykey + window - qi0 : N) : 0) -
                   4 * hh;

    // Issue order within the step: both score-shaped products first (S =
    // Q K_w^T and dP = dO V_w^T, keys on the lanes), so the exponentials of P
    // run beside the dP MFMAs; then dV += P^T dO, beside which the dS
    // arithmetic runs; then dK += dS^T Q.  Within one wave a few VALU
    // instructions per MFMA are nearly free, so each VALU phase hides behind
    // independent matrix work instead of stalling between two products.
    v8 pA[BQ / 16], dsA[BQ / 16];
    f32x16 sa = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const v8 aq = lds_at<v8>(Qs[0], rbs ^ (32 * kk));
      const v8 bk = lds_at<v8>(Ks, kws ^ (32 * kk));
      sa = mfma32x32x16(aq, bk, sa);
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const v8 ad = lds_at<v8>(dOs[0], rbs ^ (32 * kk));
      dp = mfma32x32x16(ad, vf[kk], dp);
    }
    // Issue order of the two products: each MFMA's LDS operands are read
    // KV_READ_AHEAD MFMAs ahead of it (two reads per S MFMA, one per dP MFMA),
    // instead of the scheduler's read-wait-use pairs, which expose the LDS
    // latency at every MFMA of the S chain.
    {
      constexpr int NS = D / 16, L = NS < KV_READ_AHEAD ? NS : KV_READ_AHEAD;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * L, 0);
#pragma unroll
      for (int i = 0; i < NS - L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
    }
    // P = exp2(c S - L log2 e) for every element, then, on the few steps that
    // need it (the wave's diagonal step and the ragged ends), the masked
    // elements are zeroed.  The empty volatile asm keeps that a real branch:
    // flattened into selects it would cost five instructions per score on
    // every step.  Unmasked garbage never reaches a product.  P is kept only
    // in the storage type.
    float pv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][qp * BQ + 8 * g + 4 * hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[4 * g + e] = fast_exp2(__builtin_fmaf(sa[4 * g + e], c, -l4[e]));
    }
    if (need_mask) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qc = 8 * (r >> 2) + (r & 3);  // query offset minus 4 hh
        pv[r] = (qc >= lo && qc < hi) ? pv[r] : 0.f;
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) pA[hf] = to_v8<T>(&pv[8 * hf]);

    // dV_w += P^T dO_i; the B operand comes from transpose reads of the dO tile.
#pragma unroll
    for (int kc = 0; kc < BQ / 16; ++kc)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2 d0 = lds_tr_at(dOs[0], (tbs ^ tile_tr_xor<D>(0, nb)) + 32 * D * kc);
        const u32x2 d1 = lds_tr_at(dOs[0], (tbs ^ tile_tr_xor<D>(1, nb)) + 32 * D * kc);
        const u32x4 cd = {d0[0], d0[1], d1[0], d1[1]};
        dvacc[nb] = mfma32x32x16(pA[kc], __builtin_bit_cast(v8, cd), dvacc[nb]);
      }
    // dS = P o (dP - D), rounded to the storage type.  For bfloat16, P as
    // rounded for the P^T dO product (unpacked from the packed words); for
    // fp16, the fp32 P, as in the dQ pass (the fp16 unpacking costs the
    // registers that keep this kernel out of scratch memory).
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      float pr[8], dsv[8];
      if constexpr (__is_same(T, __bf16)) {
        from_v8(pA[hf], pr);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = pv[8 * hf + e];
      }
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const f32x4 d4 =
            *reinterpret_cast<const f32x4*>(&Ds[buf][qp * BQ + 16 * hf + 8 * g2 + 4 * hh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dsv[4 * g2 + e] = pr[4 * g2 + e] * (dp[8 * hf + 4 * g2 + e] - d4[e]);
      }
      dsA[hf] = to_v8<T>(dsv);
    }
    // dK_w += dS^T Q_i (scale applied at the end), Q^T by transpose reads.
#pragma unroll
    for (int kc = 0; kc < BQ / 16; ++kc)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2 q0 = lds_tr_at(Qs[0], (tbs ^ tile_tr_xor<D>(0, nb)) + 32 * D * kc);
        const u32x2 q1 = lds_tr_at(Qs[0], (tbs ^ tile_tr_xor<D>(1, nb)) + 32 * D * kc);
        const u32x4 cq = {q0[0], q0[1], q1[0], q1[1]};
        dkacc[nb] = mfma32x32x16(dsA[kc], __builtin_bit_cast(v8, cq), dkacc[nb]);
      }

    }
    if (it + 1 < nss) store_step(buf ^ 1);
#pragma unroll
    for (int tq = 0; tq < QS; ++tq) advance(cu_h, cu_q);
    wait_counts<FA_VMCNT_LGKM0(0)>();  // this wave's direct loads have landed
    __syncthreads();
  }

  if constexpr (QS > 1) {
    // Merge the parts of the query steps: each wave with qp > 0 leaves its
    // dK and dV accumulators in a region of the Q / dO ring (free after the
    // last barrier), in its own lane order, and the qp = 0 wave of the same
    // keys adds them in, in qp order.
    constexpr int RF = 2 * NB * 16 * 64;                    // floats per region
    constexpr int RPA = (int)sizeof(Qs) / (RF * 4);          // regions per array
    static_assert(RPA >= 1 && 2 * RPA >= (QS - 1) * KWAVES, "partials fit in the ring");
    auto region = [&](int p) {  // region of the wave (key set kw, step part p)
      const int ri = (p - 1) * KWAVES + kw;
      return ri < RPA ? reinterpret_cast<float*>(&Qs[0][0]) + ri * RF
                      : reinterpret_cast<float*>(&dOs[0][0]) + (ri - RPA) * RF;
    };
    if (qp > 0) {
      float* const xa = region(qp);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xa[(16 * nb + r) * 64 + lane] = dkacc[nb][r];
          xa[(16 * (NB + nb) + r) * 64 + lane] = dvacc[nb][r];
        }
    }
    __syncthreads();
    if (qp > 0) return;
    for (int p = 1; p < QS; ++p) {
      const float* const xa = region(p);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dkacc[nb][r] += xa[(16 * nb + r) * 64 + lane];
          dvacc[nb][r] += xa[(16 * (NB + nb) + r) * 64 + lane];
        }
    }
  }

  // Write dK = scale * sum dS^T Q and dV = sum P^T dO for this wave's keys,
  // through LDS: in the accumulator layout a lane holds one column of 16 keys,
  // so direct stores would be 2-byte pieces; staged row-major in the wave's
  // own 32 rows of the K tile (free after the last step's barrier), every
  // store instruction writes whole rows, 1 KiB contiguous.  dK first, then dV
  // through the same rows.
  T* const stage = Ks + 32 * D * kw;
  constexpr int LPR = D / 8;    // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;  // rows per store instruction
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        stage[tile_off<D>(8 * (r >> 2) + 4 * hh + (r & 3), 32 * nb + l32)] =
            t2 == 0 ? (T)(dkacc[nb][r] * scale) : (T)dvacc[nb][r];
    T* __restrict__ dst = t2 == 0 ? dK : dV;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / LPR, ch = lane % LPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + tile_off<D>(row, 8 * ch));
      if (kw0 + row < N) st16(dst + hoff + (size_t)(kw0 + row) * D + 8 * ch, w);
    }
  }
}

// ---------------------------------------------------------------- kernel 3
// NW waves x 32 query rows per workgroup: eight waves (one workgroup per CU,
// a three-deep ring) or four (two workgroups per CU, a two-deep ring); the
// launcher picks by the number of 256-row blocks.
constexpr int DQ_BC = 64;  // keys per tile
constexpr int DQ_READ_AHEAD = 6;  // S / dP MFMAs whose LDS operands are read ahead
constexpr long DQ_SMALL_GRID = 256;   // 256-row blocks below which dQ runs four-wave workgroups
constexpr long DQ_LARGE_GRID = 1024;  // ... and from which on it runs them again

template <typename T, int D, bool CAUSAL, bool WIN, int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ drow,
    T* __restrict__ dQ, int N, int nqb, int total, int group, int window, float scale, float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  if constexpr (!WIN) window = 0;  // window code only in the WIN instantiation
  constexpr int BR = 32 * NW, BC = DQ_BC, NB = D / 32;
  constexpr int SPW = BC * D * 2 / 1024 / NW;  // tile load segments per wave (vmcnt units)
  constexpr int RING = NW == 8 ? 3 : 2;         // tiles in the LDS ring
  static_assert(NW == 8 || NW == 4, "one eight-wave or two four-wave workgroups per CU");
  __shared__ __attribute__((aligned(1024))) T K0[BC * D], K1[BC * D], K2[RING > 2 ? BC * D : 1];
  __shared__ __attribute__((aligned(1024))) T V0[BC * D], V1[BC * D], V2[RING > 2 ? BC * D : 1];

  // Work item: XCD-local heads, heaviest causal query blocks first.
  int bh, rank;
  work_item(blockIdx.x, total / nqb, nqb, CAUSAL && !WIN, bh, rank);
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_int(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int li = lane & 15, grp = lane >> 4;
  const size_t hoff = (size_t)bh * N * D;
  const size_t kvoff = (size_t)(bh / group) * N * D;  // the group's key/value head
  const T* __restrict__ Kh = K + kvoff;
  const T* __restrict__ Vh = V + kvoff;

  const int qw0 = qb * BR + 32 * wave;  // first query row of this wave
  const int myq = qw0 + l32;
  const bool q_ok = myq < N;
  f32x16 dqacc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) dqacc[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, (qb + 1) * BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  // Sliding window: tiles before the block's first visible key are skipped.
  const int kbase = (CAUSAL && window > 0) ? (max(0, qb * BR - window + 1) / BC) * BC : 0;
  const int nt = ntiles - kbase / BC;
  // Rows past the end of a tile read as zero and are masked.
  const TileLoader<D, BC, NW> loader(wave, lane);
  auto load_kv = [&](const T* __restrict__ src, T* dst, int kb) {
    loader.load(src, N, kb, dst, wave);
  };
  // LDS byte offsets by XOR addressing (fa_tile.h): K and V rows (A operands
  // of S^T and dP^T) at row l32, columns 16 kk + 8 hh; K^T (A operand of
  // dQ^T += K^T dS^T) by transpose reads, lane li of group grp at key
  // 8 t + 4 hh + li / 4, columns 32 nb + 16 (grp mod 2) + 4 (li mod 4).
  const uint32_t rb = tile_row_base<D>(l32, hh);
  const uint32_t tb = tile_tr_base<D>(4 * hh + (li >> 2), 16 * (grp & 1) + 4 * (li & 3));

  // Tiles 0 .. RING-2 start loading first, then the rows of Q, dO, L and D:
  // scaling L waits for its load and, the counter being in order, for every
  // load issued before it, so issued the other way round the tiles' loads
  // would start only once the rows had arrived.
  load_kv(Kh, K0, kbase);
  load_kv(Vh, V0, kbase);
  if (RING > 2 && nt > 1) {
    load_kv(Kh, K1, kbase + BC);
    load_kv(Vh, V1, kbase + BC);
  }
  asm volatile("" ::: "memory");  // keeps the row loads after the tiles' loads
  // Q and dO rows as the B operands of S^T = K Q^T and dP^T = V dO^T: lane
  // holds row myq, columns 16 kk + 8 hh + 0..7.  Rows past the end are zero
  // (with L = D = 0 their dS is exactly 0).
  v8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const size_t off = hoff + (size_t)myq * D + 16 * kk + 8 * hh;
    qf[kk] = q_ok ? ld16<v8>(Q + off) : v8{};
    dof[kk] = q_ok ? ld16<v8>(dO + off) : v8{};
  }
  const float lq = q_ok ? LSE[(size_t)bh * N + myq] * 1.4426950408889634f : 0.f;
  const float dq_row = q_ok ? drow[(size_t)bh * N + myq] : 0.f;

  // Wait for tile 0.  The row loads are younger than tile 1's, so in a wave
  // that loads rows this also waits for tile 1.
  if (RING > 2 && nt > 1)
    wait_counts<FA_VMCNT_LGKM0(2 * SPW)>();
  else
    wait_counts<FA_VMCNT_LGKM0(0)>();
  bare_barrier();

  // One tile: tile j + RING - 1 starts loading into the buffer tile j-1 used,
  // tile j is computed, and before the barrier this wave's loads of tile j+1
  // are done.
  auto tile_step = [&](int j, const T* __restrict__ kt, const T* __restrict__ vt, T* kn, T* vn) {
    const int kb = kbase + j * BC;
    const bool more = j + RING - 1 < nt;
    if (more) {
      load_kv(Kh, kn, kb + (RING - 1) * BC);
      load_kv(Vh, vn, kb + (RING - 1) * BC);
    }
    if (!CAUSAL || (kb <= qw0 + 31 && (window == 0 || kb + BC - 1 > qw0 - window))) {
      // Keys past the end and, on diagonal tiles, keys after the query are
      // dropped: key kb + 32 sb + 8 (r / 4) + 4 hh + (r % 4) is kept iff its
      // offset within the tile is <= lim.
      const bool need_mask = (CAUSAL && kb + BC - 1 > qw0) || (kb + BC > N) ||
                             (CAUSAL && window > 0 && kb <= qw0 + 31 - window);
      int lim = N - 1 - kb;
      if (CAUSAL) lim = min(lim, myq - kb);
      lim -= 4 * hh;
      // Window: keys at tile offset < llim are too old for this row.
      const int llim = (window > 0 ? myq - window + 1 - kb : -(1 << 30)) - 4 * hh;
      // Opaque copies of the bases keep the XORs per tile instead of hoisted
      // into sixteen loop-invariant registers.
      uint32_t rbs = rb, tbs = tb;
      asm volatile("" : "+v"(rbs), "+v"(tbs));
      // Both halves' S and dP first, then one mask branch (taken on diagonal
      // and ragged tiles only), then per 32 keys the exponentials and dS
      // followed by that half's dQ products: the second half's VALU work can
      // then run beside the first half's dQ MFMAs.
      {
        f32x16 s[BC / 32], dp[BC / 32];
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb) {
          s[sb] = f32x16{};
          dp[sb] = f32x16{};
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            const v8 ak = lds_at<v8>(kt, (rbs ^ (32 * kk)) + 64 * D * sb);
            const v8 av = lds_at<v8>(vt, (rbs ^ (32 * kk)) + 64 * D * sb);
            s[sb] = mfma32x32x16(ak, qf[kk], s[sb]);
            dp[sb] = mfma32x32x16(av, dof[kk], dp[sb]);
          }
        }
        // Issue order: each K or V row read runs DQ_READ_AHEAD MFMAs ahead of
        // the MFMA that uses it (the scheduler's read-wait-use pairs expose
        // the LDS latency at every one of these MFMAs).
        {
          constexpr int NM = 2 * (BC / 32) * (D / 16), L = DQ_READ_AHEAD;
          __builtin_amdgcn_sched_group_barrier(0x100, L, 0);
#pragma unroll
          for (int i = 0; i < NM - L; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
        }
        if (need_mask) {
#pragma unroll
          for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * sb + 8 * (r >> 2) + (r & 3) > lim || 32 * sb + 8 * (r >> 2) + (r & 3) < llim)
                s[sb][r] = -INFINITY;
        }
        // Per 32 keys: dS^T = P^T o (dP^T - D), then dQ^T += K^T dS^T for
        // those keys (K^T from two transpose reads per MFMA).
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb) {
          v8 dsb[2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float dsv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int r = 8 * hf + e;
              dsv[e] = fast_exp2(__builtin_fmaf(s[sb][r], c, -lq)) * (dp[sb][r] - dq_row);
            }
            dsb[hf] = to_v8<T>(dsv);
          }
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const int kc = 2 * sb + hf;
              const u32x2 lo = lds_tr_at(kt, (tbs ^ tile_tr_xor<D>(0, nb)) + 32 * D * kc);
              const u32x2 hi = lds_tr_at(kt, (tbs ^ tile_tr_xor<D>(1, nb)) + 32 * D * kc);
              const u32x4 cat = {lo[0], lo[1], hi[0], hi[1]};
              dqacc[nb] = mfma32x32x16(__builtin_bit_cast(v8, cat), dsb[hf], dqacc[nb]);
            }
        }
      }
    }
    // Tile j+1 has landed (this wave's share) and every LDS read of tile j
    // has returned; after the barrier no wave reads tile j's buffer again.
    if (RING > 2 && more) wait_counts<FA_VMCNT_LGKM0(2 * SPW)>();
    else wait_counts<FA_VMCNT_LGKM0(0)>();
    bare_barrier();
  };
  // Unrolled by the ring depth so each step names its ring buffers statically.
  if constexpr (RING == 3) {
    for (int j = 0; j < nt; j += 3) {
      tile_step(j, K0, V0, K2, V2);
      if (j + 1 < nt) tile_step(j + 1, K1, V1, K0, V0);
      if (j + 2 < nt) tile_step(j + 2, K2, V2, K1, V1);
    }
  } else {
    for (int j = 0; j < nt; j += 2) {
      tile_step(j, K0, V0, K1, V1);
      if (j + 1 < nt) tile_step(j + 1, K1, V1, K0, V0);
    }
  }

  // dQ = scale * dQ^T, transposed back through LDS as in the forward pass: in
  // the accumulator layout a lane holds 8-byte pieces of one row, so a store
  // instruction would touch 32 rows; staged in a swizzled row-major tile (the
  // ring is free after the last tile's barrier, half a ring buffer per wave),
  // every store instruction writes whole rows, 1 KiB contiguous.
  T* const stage = (wave < 2 ? K0 : wave < 4 ? K1 : wave < 6 ? K2 : V0) + (wave & 1) * 32 * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      v4 vals;
#pragma unroll
      for (int q = 0; q < 4; ++q) vals[q] = (T)(dqacc[nb][4 * gg + q] * scale);
      *reinterpret_cast<u32x2*>(stage + tile_off<D>(l32, 32 * nb + 8 * gg + 4 * hh)) =
          __builtin_bit_cast(u32x2, vals);
    }
  constexpr int LPR = D / 8;    // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / LPR, ch = lane % LPR;
    const u32x4 w = *reinterpret_cast<const u32x4*>(stage + tile_off<D>(row, 8 * ch));
    if (qw0 + row < N) st16(dQ + hoff + (size_t)(qw0 + row) * D + 8 * ch, w);
  }
}

// ---------------------------------------------------------------- launchers
// On small grids, and with grouped key/value heads, the dQ pass runs on a
// second stream beside the dK/dV pass (both read only what bwd_pre wrote):
// each pass alone leaves most CUs idle while its heaviest blocks finish, and
// grouped heads make the dK/dV blocks long (each walks every query head of
// its group).  The caller's stream forks to the second
// stream after bwd_pre and joins it after the dQ pass, through two events,
// so work later queued on the caller's stream still follows the whole
// backward; kernels and results are the same as on one stream.  Measured
// against one stream (causal unless noted, d = 128, blocks of 128 keys):
// B1 H4 N2048 (64 blocks) 0.1158 -> 0.0827 ms, B1 H8 N2048 0.1185 ->
// 0.0902, B1 H4 N8192 (256) 0.4312 -> 0.3157, B4 H8 N1024 0.0705 -> 0.0654,
// B1 H8 N4096 non-causal 0.2475 -> 0.2193, B1 H32 N2048 (512) 0.1658 ->
// 0.1492, B1 H16 N4096 0.3063 -> 0.2624, B1 H64 N1024 0.0964 -> 0.0950; from
// 1024 blocks on it loses: B4 H16 N2048 0.2571 -> 0.2631, B2 H16 N4096
// 0.4596 -> 0.4656, B8 H16 N1024 0.1587 -> 0.1664, B1 H32 N8192 1.663 ->
// 1.685.  Grouped heads (H / H_kv query heads per key/value head): B1 H32
// H_kv8 N8192 (512) 2.031 -> 1.715, B2 H16 H_kv4 N4096 (256) 0.7213 ->
// 0.5861, and past 512 blocks B2 H32 H_kv8 N8192 (1024) 3.518 -> 3.373,
// B2 H16 H_kv8 N8192 (1024) 1.761 -> 1.697, B4 H32 H_kv8 N4096 (1024) 1.823
// -> 1.761, B8 H32 H_kv8 N2048 (2048) 0.9832 -> 0.9678.
constexpr long BWD_SIDE_MAX_BLOCKS = 512;
// At most 128 blocks of 64 keys (half the CUs): blocks of 64 keys whose two
// pairs of waves split the query steps, one workgroup per CU, with the other
// CUs free for the dQ pass beside them.  Measured against 128-key blocks,
// interleaved on one box (causal, d = 128): B1 H4 N2048 0.0848 -> 0.0744
// ms, non-causal 0.0896 -> 0.0766, B1 H2 N4096 0.1464 -> 0.1283, B1 H1
// N8192 0.2742 -> 0.2360, B2 H4 N1024 0.0554 -> 0.0495, B1 H8 H_kv2 N2048
// 0.2804 -> 0.2368.  At 256 blocks the dK/dV workgroups take every CU and
// the dQ ones no longer fit beside them: B1 H8 N2048 0.0887 -> 0.0910, B1
// H4 N4096 0.1536 -> 0.2051.  Where even 32-key blocks number at most 128,
// four waves own each block's keys and take every fourth step, against the
// two-way split: grouped B1 H8 H_kv2 N2048 0.2396 -> 0.1506, B1 H16 H_kv2
// N2048 0.4609 -> 0.2787, B1 H8 H_kv1 N4096 0.8974 -> 0.5287; B1 H1 N4096
// 0.1282 -> 0.1066, B1 H2 N2048 0.0738 -> 0.0677, B1 H4 N1024 0.0480 ->
// 0.0491.
constexpr long BWD_Q_SPLIT_MAX = 128;  // blocks (of 64, or of 32, keys)
// With grouped heads every block walks its whole group, so its walk is long
// enough for the split to pay on up to 256 blocks, against 128-key blocks
// (two-way) or the two-way split (four-way): B1 H16 H_kv4 N4096 0.5492 ->
// 0.4602 ms, B1 H8 H_kv2 N8192 1.0667 -> 0.9599, B2 H16 H_kv4 N2048 0.2847
// -> 0.2417, B1 H32 H_kv4 N4096 1.0800 -> 0.9043, B1 H32 H_kv8 N2048 0.2848
// -> 0.2427; four-way at 256 blocks of 32 keys, B1 H16 H_kv4 N2048 0.2397
// -> 0.1631.
constexpr long BWD_Q_SPLIT4_MAX_GROUPED = 256;
constexpr long BWD_Q_SPLIT2_MAX_GROUPED = 256;

namespace {
// The second stream and the fork / join events of one device, created on
// the first small-grid call on it (never inside a stream capture) and kept
// until the process ends.  The lock makes each call's fork, launches and
// join one unit, so concurrent calls on one device never pair one call's
// event with another's wait (they share the second stream and run its dQ
// passes in order).
struct SideStream {
  hipStream_t s2;
  hipEvent_t fork, join;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// The current device's set, or null for one stream: s belongs to another
// device, or the set does not exist yet and s is capturing.  Called with
// g_side_mu held.
hipError_t side_stream(hipStream_t s, SideStream*& out) {
  out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipDevice_t sdev = -1;
  if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess) return e;
  if (sdev != dev || dev < 0 || dev >= kMaxSideDevices) return hipSuccess;
  SideStream& ss = g_side[dev];
  if (!ss.s2) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(s, &st)) != hipSuccess) return e;
    if (st != hipStreamCaptureStatusNone) return hipSuccess;
    SideStream n{};
    if ((e = hipStreamCreateWithFlags(&n.s2, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) != hipSuccess) {
      if (n.fork) (void)hipEventDestroy(n.fork);
      (void)hipStreamDestroy(n.s2);
      return e;
    }
    ss = n;
  }
  out = &ss;
  return hipSuccess;
}
}  // namespace

template <typename T, int D, bool CAUSAL, bool WIN>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.H * a.N;
  const long pre_threads = rows * (D / 8);
  hipError_t e = launch_kernel(bwd_pre_kernel<T, D>, dim3((unsigned)((pre_threads + 255) / 256)),
                               dim3(256), s, static_cast<const T*>(a.o),
                               static_cast<const T*>(a.dout), a.drow, rows);
  if (e != hipSuccess) return e;
  const float c = a.scale * 1.4426950408889634f;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  const T* dout = static_cast<const T*>(a.dout);

  const int group = a.H / a.Hkv;
  const int window = WIN ? a.window : 0;
  // Tiny grids: blocks of 64 (32) keys whose waves split the query steps in
  // two (four).
  const long kvh = (long)a.B * a.Hkv;
  const long max4 = group > 1 ? BWD_Q_SPLIT4_MAX_GROUPED : BWD_Q_SPLIT_MAX;
  // (At d = 64 the two-way split workgroup needs half the LDS and fewer
  // registers, so a dQ workgroup still fits beside it: B1 H2 N8192 0.2061
  // -> 0.1812 ms, B1 H4 N4096 0.1140 -> 0.1079, B1 H8 N2048 0.0700 ->
  // 0.0688, non-causal 0.0671 -> 0.0679, at 256 blocks.)
  const long max2 = (group > 1 || D == 64) ? BWD_Q_SPLIT2_MAX_GROUPED : BWD_Q_SPLIT_MAX;
  const int qs = kvh * ((a.N + 31) / 32) <= max4 ? 4 : kvh * ((a.N + 63) / 64) <= max2 ? 2 : 1;
  const int bk = KV_BK / qs;
  const int nkb = (a.N + bk - 1) / bk;
  const int kv_total = a.B * a.Hkv * nkb;

  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  if (kv_total <= BWD_SIDE_MAX_BLOCKS || group > 1) {
    lock.lock();
    if ((e = side_stream(s, side)) != hipSuccess) return e;
    if (side) {
      if ((e = hipEventRecord(side->fork, s)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side->s2, side->fork, 0)) != hipSuccess) return e;
    }
  }
  if (qs == 4)
    e = launch_kernel(bwd_kv_kernel<T, D, CAUSAL, WIN, 4>, dim3(kv_total), dim3(KV_WAVES * 64), s,
                      q, k, v, dout, a.lse, a.drow, static_cast<T*>(a.dk), static_cast<T*>(a.dv),
                      a.N, nkb, kv_total, group, window, a.scale, c);
  else if (qs == 2)
    e = launch_kernel(bwd_kv_kernel<T, D, CAUSAL, WIN, 2>, dim3(kv_total), dim3(KV_WAVES * 64), s,
                      q, k, v, dout, a.lse, a.drow, static_cast<T*>(a.dk), static_cast<T*>(a.dv),
                      a.N, nkb, kv_total, group, window, a.scale, c);
  else
    e = launch_kernel(bwd_kv_kernel<T, D, CAUSAL, WIN, 1>, dim3(kv_total), dim3(KV_WAVES * 64), s,
                      q, k, v, dout, a.lse, a.drow, static_cast<T*>(a.dk), static_cast<T*>(a.dv),
                      a.N, nkb, kv_total, group, window, a.scale, c);
  if (e != hipSuccess) return e;

  // dQ: four-wave workgroups, two per CU, below one 256-row block per CU and
  // from four per CU on; eight-wave ones in between.  Measured, gradients
  // bitwise identical (eight-wave against four-wave): 512 blocks, B2 H16
  // N4096 0.4509 / 0.4533 ms and B1 H16 N16384 3.3205 / 3.3228; 1024
  // blocks, B1 H32 N8192 1.6776 / 1.6619 and B8 H16 N2048 0.5229 / 0.5103;
  // 2048 blocks, B4 H32 N4096 1.8679 / 1.8611 and B2 H32 N8192 3.4116 /
  // 3.3883.  Beside the dK/dV pass without grouped heads (at most 256 such
  // blocks), four-wave workgroups share CUs with dK/dV ones, where the
  // eight-wave ones do not fit beside them: at 256 blocks B1 H32 N2048
  // 0.1538 -> 0.1448 ms, B1 H16 N4096 0.2725 -> 0.2522, B1 H64 N1024 0.0978
  // -> 0.0923.  With grouped heads the rule stands (B2 H16 H_kv4 N4096,
  // 512 blocks: 0.5912 eight-wave against 0.6672 four-wave).
  const long blocks256 = (long)a.B * a.H * ((a.N + 255) / 256);
  const bool four_wave = blocks256 < DQ_SMALL_GRID || blocks256 >= DQ_LARGE_GRID ||
                         (side && group == 1);
  const int br = four_wave ? 128 : 256;
  const int nqb = (a.N + br - 1) / br;
  const int dq_total = a.B * a.H * nqb;
  const hipStream_t sq = side ? side->s2 : s;
  if (four_wave)
    e = launch_kernel(bwd_dq_kernel<T, D, CAUSAL, WIN, 4>, dim3(dq_total), dim3(4 * 64), sq, q, k,
                      v, dout, a.lse, a.drow, static_cast<T*>(a.dq), a.N, nqb, dq_total, group,
                      window, a.scale, c);
  else
    e = launch_kernel(bwd_dq_kernel<T, D, CAUSAL, WIN, 8>, dim3(dq_total), dim3(8 * 64), sq, q, k,
                      v, dout, a.lse, a.drow, static_cast<T*>(a.dq), a.N, nqb, dq_total, group,
                      window, a.scale, c);
  if (e != hipSuccess || !side) return e;
  if ((e = hipEventRecord(side->join, side->s2)) != hipSuccess) return e;
  return hipStreamWaitEvent(s, side->join, 0);
}

template <typename T, int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  if (!a.causal) return launch_bwd_t<T, D, false, false>(a, s);
  return a.window > 0 ? launch_bwd_t<T, D, true, true>(a, s) : launch_bwd_t<T, D, true, false>(a, s);
}

template <typename T>
static hipError_t launch_bwd_dt(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_bwd_d<T, 64>(a, s) : launch_bwd_d<T, 128>(a, s);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_bwd_dt<__bf16>(a, s) : launch_bwd_dt<_Float16>(a, s);
}

}  // namespace fa
