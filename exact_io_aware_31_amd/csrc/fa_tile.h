// fa_tile.h -- key / value tiles in LDS for the kernels that stream blocks of
// keys past a resident block of query rows (the forward pass and the dQ pass
// of the backward).
//
// A tile holds BC consecutive rows of a [N, D] head (D two-byte elements per
// row), unpadded, with 16-byte chunk c of row r stored at chunk c ^ sw(r).
// 256-byte rows use sw(r) = 4 (r mod 4) + (r / 4 mod 4), 128-byte rows
// sw(r) = r / 2 mod 8.  Either way sixteen consecutive rows read at one
// logical chunk touch every bank once, and the 4-row x 32-byte footprint of a
// transpose read is conflict-free.  The swizzle depends on r mod 16 only, so
// per-lane offsets computed for rows 0..15 (or 0..31) hold for every 16-row
// (32-row) block of a tile.
#pragma once

#include "fa_common.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i mod 4) of the 4-element rows addressed by lanes i/4, 4 + i/4, 8 + i/4
// and 12 + i/4 of its group.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

template <int D>
struct TileSwizzle {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static __device__ __forceinline__ int sw(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
  }
};
// Element offset of (row, col) in a tile of rows of D elements swizzled by SW.
template <int D, typename SW = TileSwizzle<D>>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ SW::sw(row)) << 3) | (col & 7));
}

// XOR addressing.  The swizzle only XORs chunk bits, so the byte offsets of
// a lane's reads are one base XOR a compile-time constant:
//   * 16-byte row read of row r, columns 16 kk + 8 h:
//       tile_row_base<D>(r, h) ^ (32 kk);
//   * transpose read of row 16 kc + 8 t + r0, columns 32 nb + c0 (r0 < 8,
//     c0 < 32, c0 a multiple of 4):
//       (tile_tr_base<D>(r0, c0) ^ tile_tr_xor<D>(t, nb)) + 32 D kc.
// A kernel short of registers keeps the two bases instead of a table of
// offsets (one XOR per read).  Bases may be offset by any multiple of the
// tile size: the XORs only touch bits below it.
template <int D>
__device__ __forceinline__ uint32_t tile_row_base(int r, int h) { return 2 * tile_off<D>(r, 8 * h); }
template <int D>
__device__ __forceinline__ uint32_t tile_tr_base(int r0, int c0) { return 2 * tile_off<D>(r0, c0); }
template <int D>
__device__ __forceinline__ uint32_t tile_tr_xor(int t, int nb) { return 2 * tile_off<D>(8 * t, 32 * nb); }

template <typename V>
__device__ __forceinline__ V lds_at(const void* tile, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(tile) + byte_off);
}
__device__ __forceinline__ u32x2 lds_tr_at(const void* tile, uint32_t byte_off) {
  return lds_read_tr16(reinterpret_cast<const char*>(tile) + byte_off);
}

// Direct buffer load of 16 bytes per lane into LDS: lane l's bytes, read at
// byte offset voff of a raw buffer of `bytes` bytes starting at base, land at
// lds_base + 16 l (lds_base wave-uniform).  Offsets at or past `bytes` read
// as zero.  base and bytes must be wave-uniform (they form the descriptor).
// CPOL is the load's cache policy (0, or FA_CPOL_NT for data read once).
#define FA_CPOL_NT 2
template <int CPOL = 0>
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t bytes, uint32_t voff,
                                                  void* lds_base) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, 0, 0, CPOL);
}

// One float through a raw buffer descriptor of `bytes` bytes at base (both
// wave-uniform): offsets voff at or past `bytes` read as zero.
__device__ __forceinline__ float buffer_load_f32(const float* base, uint32_t bytes, uint32_t voff) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}

// Direct load of rows kb .. kb + BC - 1 of a head into the tile at dst by NW
// waves (buffer_load_dwordx4 ... lds): the tile is cut into 1 KiB segments,
// wave w fills segments w SPW .. w SPW + SPW - 1, and lane l of segment g
// fills LDS chunk slot l of it, i.e. tile row g RPS + l / (D / 8), physical
// chunk l mod (D / 8), with the logical chunk the swizzle SW puts there.
// Each wave issues SPW loads per tile, counted by its vmcnt.  A lane's byte
// offset inside a tile (its row and swizzled chunk) is the same for every
// tile, so it is computed once; a tile's position enters only
// through the buffer descriptor, built in scalar registers per tile: base =
// the tile's first row, num_records = the bytes from there to the end of the
// head.  The hardware range check returns zeros for rows past the end (which
// callers mask), so no clamp is needed and no access can leave the head.
template <int D, int BC, int NW, typename SW = TileSwizzle<D>>
struct TileLoader {
  static constexpr int RPS = 512 / D;
  static constexpr int NSEG = BC * D * 2 / 1024;
  static constexpr int SPW = NSEG / NW;
  static_assert(NSEG % NW == 0, "tile segments split evenly over the waves");
  uint32_t voff[SPW];
  __device__ __forceinline__ TileLoader(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int row = (wave * SPW + i) * RPS + lane / (D / 8);
      voff[i] = 2u * (uint32_t)(row * D + 8 * ((lane % (D / 8)) ^ SW::sw(row)));
    }
  }
  // Rows kb .. kb + BC - 1 of a head of N rows (kb <= N; with kb = N nothing
  // is read and the loads land zeros) into the tile at dst.
  template <int CPOL = 0, typename T>
  __device__ __forceinline__ void load(const T* head, int N, int kb, T* dst, int wave) const {
    const uint32_t bytes = (uint32_t)(N - kb) * (uint32_t)(D * 2);
    const void* base = head + (size_t)kb * D;
#pragma unroll
    for (int i = 0; i < SPW; ++i)
      buffer_load_lds16<CPOL>(base, bytes, voff[i], dst + (wave * SPW + i) * 512);
  }
};

}  // namespace fa
