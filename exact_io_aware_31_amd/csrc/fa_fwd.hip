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
//   * NW waves x 32 query rows per workgroup, two waves per SIMD; 64-key
//     tiles.  Eight-wave workgroups (one per CU) are the default; for small
//     grids and short sequences four-wave workgroups run two per CU instead.
//     On grids of at most one 64-row block per CU, a four-wave workgroup
//     takes 64 rows and its two pairs of waves split the keys (even and odd
//     tiles of each step, merged at the end), so the longest block's tiles
//     are shared by two waves (the rules and their measurements are at the
//     launcher).
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//     each lane then owns ONE query row per 32-row group (column l % 32) and
//     16 of its scores per 32-key block, so the row max / row sum are in-lane
//     reductions plus one v_permlane32_swap between the two wave halves.
//   * The probabilities stay in registers and feed O^T += V^T P^T directly
//     as the B operand: the accumulator layout of S^T is used as the operand
//     layout with a consistent permutation of the reduction index.  The A
//     operand V^T is read from the row-major V tile with the LDS transpose
//     read (ds_read_b64_tr_b16), so V is never transposed in memory.
//   * K and V tiles reach LDS by direct buffer-to-LDS loads
//     (buffer_load_dwordx4 ... lds: each lane's 16 bytes land at the wave's
//     LDS base + 16 * lane) into a ring of tiles: three deep, two tiles ahead
//     of their use, for eight waves; two deep, one tile ahead, for four (so
//     that two workgroups fit in LDS).  A lane's offset inside a tile is fixed,
//     so the only per-tile work is a scalar buffer descriptor; its range
//     check returns zeros for rows past the end.
//     No registers hold staged data and no LDS store instructions are issued;
//     each wave waits for its own loads before the tile's barrier.  Tiles are
//     stored unpadded with 16-byte chunk c of row r at chunk c ^ sw(r), which
//     keeps the 16-byte row reads and the transpose reads conflict-free; the
//     loading lane picks the global chunk that belongs in its LDS slot.
//   * Running max in log2 units with log2(e) folded into the scale (v_exp_f32).
//     The output is rescaled only when a row's maximum grows by more than
//     2^8: until then the stale maximum is kept as the reference, which leaves
//     O / l and lse exact (both use the same reference) and keeps every
//     exponentiated score below 2^8.
//   * Causal: tiles entirely above the diagonal are never loaded; per
//     32-row group, tiles entirely above its rows are skipped; only tiles that
//     cross the diagonal (or the ragged end) are masked element-wise.  A
//     sliding window ("03. FlashAttention", § "Variantes et extensions") is
//     the same at the other end: tiles before the block's first window are
//     never loaded, tiles before a group's windows are skipped, and tiles
//     crossing a window's lower edge are masked.
//   * Grouped key/value heads ("FlashAttention ontleed", § "Interactie met
//     de KV-cache tijdens inferentie"): query head bh reads K/V head
//     bh / group; nothing else changes.
//   * Grid: consecutive work items of one head are placed on one XCD (the
//     hardware deals workgroups round-robin over the 8 XCDs) so the head's
//     K/V stay in that XCD's L2; causal query blocks run heaviest first.
#include "fa_launch.h"
#include "fa_tile.h"

namespace fa {

constexpr int FWD_QG = 1;  // 32-row query groups per wave
constexpr int FWD_BC = 64;
constexpr float FWD_RESCALE_SLACK = 8.0f;  // log2 units


template <typename T, int D, bool CAUSAL, bool WIN, int NW, int QG, int KS>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ LSE, int N, int nqb, int total, int group, int window,
    float c) {
  using v8 = typename Vec<T>::v8;
  using v4 = typename Vec<T>::v4;
  // The sliding-window code exists only in the WIN instantiation (window is
  // then >= 1 and the mask causal); elsewhere it folds away.
  if constexpr (!WIN) window = 0;
  // In the four-wave shape, the arguments used in and after the tile loop
  // load at the start (load_args_now): B4 H16 N2048 +1.4 to +2.0%, bitwise
  // identical.  The eight-wave shape measured 0.6-0.8% slower with them.
  if constexpr (NW == 4) load_args_now(O, LSE, c);
  // KS = 2 splits the keys inside the workgroup (tiny grids): waves w and
  // w + NW / 2 own the same 32 rows and take the even and the odd key tiles
  // of each step, then merge their partial results at the end.
  static_assert(KS == 1 || (KS == 2 && NW == 4), "key split only in four-wave workgroups");
  constexpr int BR = NW * 32 * QG / KS, BC = FWD_BC;
  constexpr int SPW = BC * D * 2 / 1024 / NW;  // tile load segments per wave (vmcnt units)
  constexpr int RING = NW == 8 ? 3 : 2;         // steps in the LDS ring
  static_assert(NW == 8 || NW == 4, "one eight-wave or two four-wave workgroups per CU");
  // The ring of K and V tiles (separate arrays, so every access names its
  // buffer statically and the compiler sees which loads it depends on); a
  // slot holds the KS tiles of one step.
  __shared__ __attribute__((aligned(1024))) T K0[KS * BC * D], K1[KS * BC * D],
      K2[RING > 2 ? BC * D : 1];
  __shared__ __attribute__((aligned(1024))) T V0[KS * BC * D], V1[KS * BC * D],
      V2[RING > 2 ? BC * D : 1];

  // Work item: XCD-local heads, heaviest causal query blocks first.
  int bh, rank;
  work_item(blockIdx.x, total / nqb, nqb, CAUSAL && !WIN, bh, rank);
  const int qb = CAUSAL ? nqb - 1 - rank : rank;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform_int(tid >> 6);  // wave-uniform
  const int rg = wave % (NW / KS), kh = wave / (NW / KS);  // row group, key tile parity
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t hoff = (size_t)bh * N * D;
  // Query head bh reads key/value head bh / group (groups of consecutive
  // query heads share one; group = 1 is plain multi-head attention).
  const size_t kvoff = (size_t)(bh / group) * N * D;
  const T* __restrict__ Qh = Q + hoff;
  const T* __restrict__ Kh = K + kvoff;
  const T* __restrict__ Vh = V + kvoff;

  const int qw0 = qb * BR + rg * 32 * QG;  // first query row of this wave
  int myq[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) myq[g] = qw0 + 32 * g + l32;

  // Q as the B operand of S^T = K Q^T: lane holds Q[myq][16 kk + 8 hh + 0..7].
  v8 qf[QG][D / 16];
#pragma unroll
  for (int g = 0; g < QG; ++g)
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[g][kk] = (myq[g] < N) ? ld16<v8>(Qh + (size_t)myq[g] * D + 16 * kk + 8 * hh) : v8{};

  f32x16 oacc[QG][D / 32];
  // m_run: running maximum (log2 units); nref: the negated reference the
  // probabilities are formed against, -m_run, or -0 while m_run is -inf (a
  // row that has seen no visible key yet: any finite reference gives its
  // -inf scores probability 0 rather than NaN).
  float m_run[QG], l_run[QG], nref[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[g][i] = f32x16{};
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
    nref[g] = -0.f;
  }

  const int kv_end = CAUSAL ? min(N, (qb + 1) * BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  // With a sliding window the block's first visible key is qb BR - window + 1:
  // tiles before the one holding it are never loaded.
  const int kbase = (CAUSAL && window > 0) ? (max(0, qb * BR - window + 1) / BC) * BC : 0;
  const int nt = ntiles - kbase / BC;  // tiles this workgroup streams
  const int nst = (nt + KS - 1) / KS;   // steps (KS tiles each)

  // Tile loads (TileLoader): rows past the end read as zero; those keys are
  // masked to -inf before the softmax, so their probabilities (and their V
  // rows' weight) are 0.
  const TileLoader<D, BC, NW> loader(wave, lane);
  auto load_kv = [&](const T* __restrict__ src, T* dst, int kb) {
    if constexpr (KS == 1) {
      loader.load(src, N, kb, dst, wave);  // kb < N
    } else {
      // A step's second tile can start past the end (an odd tile count):
      // from N on, nothing is read and the slot fills with zeros.
#pragma unroll
      for (int s = 0; s < KS; ++s) loader.load(src, N, min(kb + s * BC, N), dst + s * BC * D, wave);
    }
  };
  // Per-lane element offsets of the operand reads (the swizzle depends on the
  // row mod 16 only, so they hold for every 16- or 32-row block of a tile):
  //  * K rows (A operand of S^T = K Q^T): row l32, columns 16 kk + 8 hh.
  //  * V^T (A operand of O^T += V^T P^T) by transpose reads: lane i of 16-lane
  //    group G addresses key 8 t + 4 hh + i / 4, columns 32 nb + 16 (G mod 2)
  //    + 4 (i mod 4).
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = tile_off<D>(l32, 16 * kk + 8 * hh);
  const int grp = lane >> 4, li = lane & 15;
  int voff[2][D / 32];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
      voff[t][nb] = tile_off<D>(8 * t + 4 * hh + (li >> 2), 32 * nb + 16 * (grp & 1) + 4 * (li & 3));

  // Tiles 0 .. RING-2 in flight; wait for tile 0 (vmcnt counts this wave's loads).
  load_kv(Kh, K0, kbase);
  load_kv(Vh, V0, kbase);
  if (RING > 2 && nst > 1) {
    load_kv(Kh, K1, kbase + BC);
    load_kv(Vh, V1, kbase + BC);
    wait_counts<FA_VMCNT_LGKM0(2 * SPW)>();
  } else {
    wait_counts<FA_VMCNT_LGKM0(0)>();
  }
  // A bare barrier: the waits above already cover what it must publish (a
  // fenced barrier would also wait for the loads of the tile after next).
  bare_barrier();

  // One tile: tile j + RING - 1 starts loading into the buffer tile j-1
  // used, tile j is computed, and before the barrier this wave's loads of
  // tile j+1 are done.
  auto tile_step = [&](int j, const T* __restrict__ kslot, const T* __restrict__ vslot, T* kn,
                       T* vn) {
    const int kb0 = kbase + j * KS * BC;  // the step's first key
    const bool more = j + RING - 1 < nst;
    if (more) {
      load_kv(Kh, kn, kb0 + (RING - 1) * KS * BC);
      load_kv(Vh, vn, kb0 + (RING - 1) * KS * BC);
    }
    // This wave's tile of the step.
    const int kb = kb0 + kh * BC;
    const T* __restrict__ kt = kslot + kh * BC * D;
    const T* __restrict__ vt = vslot + kh * BC * D;
    bool active[QG];
    bool any_active = false;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      // Causal: tiles wholly after the group's last row, or (window) wholly
      // before its first row's window, are skipped.
      active[g] = (KS == 1 || j * KS + kh < nt) &&
                  (!CAUSAL || (kb <= qw0 + 32 * g + 31 &&
                               (window == 0 || kb + BC - 1 > qw0 + 32 * g - window)));
      any_active |= active[g];
    }
    if (any_active) {
      // S^T = K Q^T for BC/32 blocks of 32 keys; the blocks are interleaved so
      // consecutive MFMAs are independent, and each K operand is read from LDS
      // one step before the MFMA that uses it.
      f32x16 sacc[QG][BC / 32];
#pragma unroll
      for (int g = 0; g < QG; ++g)
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb) sacc[g][sb] = f32x16{};
      v8 ka[2][BC / 32];
#pragma unroll
      for (int sb = 0; sb < BC / 32; ++sb)
        ka[0][sb] = *reinterpret_cast<const v8*>(kt + 32 * sb * D + koff[0]);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + 1 < D / 16) {
#pragma unroll
          for (int sb = 0; sb < BC / 32; ++sb)
            ka[(kk + 1) & 1][sb] = *reinterpret_cast<const v8*>(kt + 32 * sb * D + koff[kk + 1]);
        }
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
          for (int g = 0; g < QG; ++g)
            if (active[g]) sacc[g][sb] = mfma32x32x16(ka[kk & 1][sb], qf[g][kk], sacc[g][sb]);
      }
      // Issue order of the score block: the K row reads run six reads (three
      // MFMA pairs) ahead of the MFMAs that use them, instead of the
      // scheduler's read-wait-use pairs.
      {
        constexpr int NM = (D / 16) * (BC / 32), PF = 6;
        __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
        for (int i = 0; i < (NM - PF) / 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      }

      v8 pb[QG][BC / 16];
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        if (!active[g]) {
#pragma unroll
          for (int kc = 0; kc < BC / 16; ++kc) pb[g][kc] = v8{};
          continue;
        }
        // Mask keys past the end and, on diagonal tiles, keys after the query:
        // key kb + 32 sb + 8 (r / 4) + 4 hh + (r % 4) is kept iff its offset
        // within the tile is <= lim (a per-lane bound, so 2 VALU ops per score).
        const bool need_mask = (CAUSAL && kb + BC - 1 > qw0 + 32 * g) || (kb + BC > N) ||
                               (CAUSAL && window > 0 && kb <= qw0 + 32 * g + 31 - window);
        if (need_mask) {
          int lim = N - 1 - kb;
          if (CAUSAL) lim = min(lim, myq[g] - kb);
          lim -= 4 * hh;
          // Window: keys at tile offset < llim are too old for this row.
          const int llim = (window > 0 ? myq[g] - window + 1 - kb : -(1 << 30)) - 4 * hh;
#pragma unroll
          for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * sb + 8 * (r >> 2) + (r & 3) > lim || 32 * sb + 8 * (r >> 2) + (r & 3) < llim)
                sacc[g][sb][r] = -INFINITY;
        }
        // Tile row max (3-input max tree), shared by the two halves of the wave.
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
          for (int r = 0; r < 16; r += 4)
            mx = fmaxf(fmaxf(mx, sacc[g][sb][r]),
                       fmaxf(fmaxf(sacc[g][sb][r + 1], sacc[g][sb][r + 2]), sacc[g][sb][r + 3]));
        mx = half_pair_max(mx);
        const float m_cand = mx * c;
        if (__ballot(m_cand > m_run[g] + FWD_RESCALE_SLACK)) {
          const float m_new = fmaxf(m_run[g], m_cand);
          const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[g] - m_new);
          l_run[g] *= alpha;
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) oacc[g][nb] *= alpha;
          m_run[g] = m_new;
          // (A window can hide every key so far from one row of an active
          // group, leaving its maximum at -inf.)
          nref[g] = (m_new == -INFINITY) ? -0.f : -m_new;
        }
        // Four independent partial row sums, started from the first four
        // probabilities (no additions of zero).
        float rs[4];
#pragma unroll
        for (int sb = 0; sb < BC / 32; ++sb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pv[e] = fast_exp2(__builtin_fmaf(sacc[g][sb][8 * hf + e], c, nref[g]));
              rs[e & 3] = (sb == 0 && hf == 0 && e < 4) ? pv[e] : rs[e & 3] + pv[e];
            }
            pb[g][2 * sb + hf] = to_v8<T>(pv);
          }
        l_run[g] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      }

      // O^T += V^T P^T; the V^T operand comes from two transpose reads.
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
          const u32x2 lo = lds_read_tr16(vt + 16 * kc * D + voff[0][nb]);
          const u32x2 hi = lds_read_tr16(vt + 16 * kc * D + voff[1][nb]);
          const u32x4 cat = {lo[0], lo[1], hi[0], hi[1]};
          const v8 a = __builtin_bit_cast(v8, cat);
#pragma unroll
          for (int g = 0; g < QG; ++g)
            if (active[g]) oacc[g][nb] = mfma32x32x16(a, pb[g][kc], oacc[g][nb]);
        }
    }

    // Tile j+1 has landed (this wave's share) and every LDS read of tile j
    // has returned; after the barrier no wave reads tile j's buffer again, so
    // the next step may start loading into it.
    if (RING > 2 && more) wait_counts<FA_VMCNT_LGKM0(2 * SPW)>();
    else wait_counts<FA_VMCNT_LGKM0(0)>();
    bare_barrier();
  };
  // Unrolled by the ring depth so each step names its ring buffers statically.
  if constexpr (RING == 3) {
    for (int j = 0; j < nst; j += 3) {
      tile_step(j, K0, V0, K2, V2);
      if (j + 1 < nst) tile_step(j + 1, K1, V1, K0, V0);
      if (j + 2 < nst) tile_step(j + 2, K2, V2, K1, V1);
    }
  } else {
    for (int j = 0; j < nst; j += 2) {
      tile_step(j, K0, V0, K1, V1);
      if (j + 1 < nst) tile_step(j + 1, K1, V1, K0, V0);
    }
  }

  if constexpr (KS == 2) {
    // Merge the two key halves of each row group: the odd-tile wave leaves
    // its reference maximum, its partial row sums and its output
    // accumulators in a V slot (free after the last barrier), in its own
    // lane order, and the even-tile wave of the same rows adds them in,
    // both rescaled to the larger reference.
    constexpr int NX = 2 + D / 32 * 16;  // floats per lane
    static_assert(NX * 64 * 4 <= KS * BC * D * (int)sizeof(T), "partials fit in a V slot");
    float* const xa = reinterpret_cast<float*>(rg == 0 ? V0 : V1);
    if (kh == 1) {
      xa[lane] = m_run[0];
      xa[64 + lane] = l_run[0];
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xa[(2 + 16 * nb + r) * 64 + lane] = oacc[0][nb][r];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xa[lane], l1 = xa[64 + lane];
    const float m = fmaxf(m_run[0], m1);
    const float a0 = (m == -INFINITY) ? 1.f : fast_exp2(m_run[0] - m);
    const float a1 = (m == -INFINITY) ? 0.f : fast_exp2(m1 - m);
    l_run[0] = l_run[0] * a0 + l1 * a1;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[0][nb][r] = oacc[0][nb][r] * a0 + xa[(2 + 16 * nb + r) * 64 + lane] * a1;
    m_run[0] = m;
  }

  // Epilogue: O = O / l, lse = (m + log2 l) ln 2.  The output goes through
  // LDS: in the accumulator layout a lane holds 8-byte pieces of one row, so
  // a store instruction would touch 32 rows with 16 bytes each; staged in a
  // swizzled row-major tile, every store instruction writes whole rows, 1 KiB
  // contiguous.  The K/V ring is free after the last tile's barrier; each
  // wave stages its own 32 rows in half of one ring buffer.
  static_assert(QG == 1, "one 32-row group per wave");
  T* const stage = (wave < 2 ? K0 : wave < 4 ? K1 : wave < 6 ? K2 : V0) + (wave & 1) * 32 * D;
  static_assert(KS == 1 || NW == 4, "with the key split, waves 0 and 1 stage their rows in K0");
  const float l_tot = half_pair_sum(l_run[0]);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      v4 vals;
#pragma unroll
      for (int q = 0; q < 4; ++q) vals[q] = (T)(oacc[0][nb][4 * gg + q] * inv);
      *reinterpret_cast<u32x2*>(stage + tile_off<D>(l32, 32 * nb + 8 * gg + 4 * hh)) =
          __builtin_bit_cast(u32x2, vals);
    }
  if (myq[0] < N && hh == 0)
    LSE[(size_t)bh * N + myq[0]] = (m_run[0] + log2f(l_tot)) * 0.69314718055994531f;
  constexpr int LPR = D / 8;    // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + lane / LPR, ch = lane % LPR;
    const u32x4 w = *reinterpret_cast<const u32x4*>(stage + tile_off<D>(row, 8 * ch));
    if (qw0 + row < N) st16(O + hoff + (size_t)(qw0 + row) * D + 8 * ch, w);
  }
}

template <typename T, int D, bool CAUSAL, bool WIN, int NW, int KS = 1>
static hipError_t launch_fwd_nw(const FwdArgs& a, hipStream_t s) {
  const int br = NW * 32 * FWD_QG / KS;
  const int nqb = (a.N + br - 1) / br;
  const int total = a.B * a.H * nqb;
  const float c = a.scale * 1.4426950408889634f;
  return launch_kernel(fwd_kernel<T, D, CAUSAL, WIN, NW, FWD_QG, KS>, dim3(total), dim3(NW * 64), s,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, a.N, nqb, total,
                       a.H / a.Hkv, WIN ? a.window : 0, c);
}

// Four-wave workgroups (two per CU) when the grid of 256-row blocks gives
// at most one per CU, or when blocks are short (N <= 2048) and there are at
// most four per CU; eight-wave workgroups otherwise, whose K/V tiles serve
// twice the rows.  Measured causal, interleaved on one box, eight-wave
// against four-wave (outputs bitwise identical):
//   256 blocks:  B1 H16 N4096 0.1075 / 0.0871 ms, B1 H8 N8192 0.1907 / 0.1596,
//                B4 H16 N1024 0.0333 / 0.0282;
//   512 blocks:  B4 H16 N2048 0.0792 / 0.0783, B2 H16 N4096 0.1350 / 0.1427,
//                B1 H16 N8192 0.2573 / 0.2726;
//   1024 blocks: B16 H16 N1024 0.1069 / 0.0993, B8 H16 N2048 0.1616 / 0.1471,
//                B4 H16 N4096 0.2754 / 0.2646, B1 H32 N8192 0.5135 / 0.5227;
//   2048 blocks: B16 H16 N2048 0.3373 / 0.3415, B4 H32 N4096 0.5635 / 0.5666,
//                B2 H32 N8192 1.0260 / 1.0452, B1 H32 N16384 1.9348 / 1.9684.
constexpr long FWD_ONE_PER_CU = 256;
constexpr long FWD_FOUR_PER_CU = 1024;
constexpr int FWD_SHORT_N = 2048;

// A sliding window of up to 2048 keys bounds each block's work to a few
// tiles, so the smaller blocks win there too (window 1024 at B1 H32 N8192:
// 0.1665 ms with eight-wave workgroups, 0.1483 with four-wave ones).
constexpr int FWD_SMALL_WINDOW = 2048;

// Grids of at most one 64-row block per CU: four-wave workgroups of 64 rows
// whose two pairs of waves split each step's keys (KS = 2), so the longest
// block's tiles are shared by two waves.  Each step then loads two tiles
// (a 128 KiB ring at d = 128: one workgroup per CU).  Measured against the
// four-wave shape, interleaved on one box (causal unless noted): B1 H8 N2048
// 0.0362 -> 0.0290 ms, non-causal 0.0352 -> 0.0297, B1 H4 N4096 0.0651 ->
// 0.0504, B1 H2 N8192 0.1246 -> 0.0985, B1 H16 N1024 0.0204 -> 0.0174, B1
// H1 N256 0.0086 / 0.0088.  Past 256 blocks it mostly loses (a second round
// of workgroups): B1 H16 N4096 0.0827 -> 0.1126, B1 H4 N8192 0.1263 ->
// 0.1440, B1 H32 N1024 0.0210 -> 0.0233; non-causal B1 H16 N2048 0.0379 ->
// 0.0548.  A window keeps the other shapes.  At d = 64 the ring takes 64
// KiB, two such workgroups fit on a CU, and the split runs up to 512 blocks:
// B1 H16 N2048 0.0274 -> 0.0208 ms, B1 H8 N4096 0.0472 -> 0.0340, B1 H4
// N8192 0.0878 -> 0.0652, B1 H32 N1024 0.0151 -> 0.0116, non-causal B1 H16
// N2048 0.0268 -> 0.0261.
constexpr long FWD_KEY_SPLIT_MAX = 256;

template <typename T, int D, bool CAUSAL, bool WIN>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  if constexpr (!WIN) {
    if ((long)a.B * a.H * ((a.N + 63) / 64) <= (D == 64 ? 2 : 1) * FWD_KEY_SPLIT_MAX)
      return launch_fwd_nw<T, D, CAUSAL, WIN, 4, 2>(a, s);
  }
  const long blocks256 = (long)a.B * a.H * ((a.N + 255) / 256);
  const bool small = blocks256 <= FWD_ONE_PER_CU ||
                     (a.N <= FWD_SHORT_N && blocks256 <= FWD_FOUR_PER_CU) ||
                     (WIN && a.window <= FWD_SMALL_WINDOW);
  return small ? launch_fwd_nw<T, D, CAUSAL, WIN, 4>(a, s) : launch_fwd_nw<T, D, CAUSAL, WIN, 8>(a, s);
}

template <typename T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  if (!a.causal) return launch_fwd_t<T, D, false, false>(a, s);
  return a.window > 0 ? launch_fwd_t<T, D, true, true>(a, s) : launch_fwd_t<T, D, true, false>(a, s);
}

template <typename T>
static hipError_t launch_fwd_dt(const FwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_fwd_d<T, 64>(a, s) : launch_fwd_d<T, 128>(a, s);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  return a.dt == DType::BF16 ? launch_fwd_dt<__bf16>(a, s) : launch_fwd_dt<_Float16>(a, s);
}

}  // namespace fa
