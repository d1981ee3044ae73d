// tile.hpp -- LDS tiles for gfx950: unpadded rows, 16-byte chunks XOR-swizzled, filled
// asynchronously by global_load_lds_dwordx4.
//
// A tile holds R rows of D bf16 (2*D bytes per row, no padding).  The 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r).  The swizzle makes the
// two read patterns the kernels use conflict-free on the 64 x 4-byte LDS banks:
//  * row-wise 16-byte reads (MFMA operand rows): 16 lanes read 16 consecutive rows
//    at the same logical chunk -> 16 distinct bank groups;
//  * transposing 8-byte reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive
//    rows (aligned to 4) x 4 consecutive chunks (aligned to 4) -> 16 distinct
//    16-byte bank groups.
// swz depends only on r & 15, so moving by a multiple of 16 rows keeps offsets.
//
// global_load_lds_dwordx4 writes lane l's 16 bytes to LDS at M0 + 16*l, i.e. one
// instruction fills 1 KiB of LDS contiguously; the swizzle is applied on the
// global side by choosing which chunk each lane fetches.
#pragma once
#include "common.hpp"

namespace attn {

typedef __attribute__((address_space(3))) void lds_void;

template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}

// Byte offset of (row r, logical 16-byte chunk c) inside a tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (2 * D) + ((c ^ swz<D>(r)) << 4);
}

// Byte offset of the 8-byte group holding elements [col, col+4) of row r (col % 4 == 0).
template <int D>
__device__ __forceinline__ int tile_off_tr(int r, int col) {
  return tile_off<D>(r, col >> 3) + 2 * (col & 7);
}

__device__ __forceinline__ bf16x8 lds_row16(const char* tile, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(tile + byte_off);
}

// A-operand of a 32x32x16 MFMA whose rows are the tile's columns (d) and whose
// reduction slots are 8 tile rows: two transposing reads (reduction slots 0-3 and
// 4-7), each at its own per-lane offset since the swizzle differs between them.
__device__ __forceinline__ bf16x8 lds_tr8(const char* tile, int off_lo, int off_hi) {
  return cat_tr(lds_read_tr16(reinterpret_cast<const bf16*>(tile + off_lo)),
                lds_read_tr16(reinterpret_cast<const bf16*>(tile + off_hi)));
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Asynchronously copy ROWS tile rows into `tile` with NW waves.  row_src(r) gives the
// global row index (already clamped into the tensor) holding tile row r; gbase points
// at (row 0, this head), rs is the row stride in elements.
template <int D, int ROWS, int NW, typename RowSrc>
__device__ __forceinline__ void tile_load_async(char* tile, const bf16* gbase, long rs, RowSrc row_src) {
  constexpr int CPR = D / 8;               // chunks per row
  constexpr int RPI = 1024 / (2 * D);      // rows per instruction (4 or 8)
  constexpr int NINST = ROWS * 2 * D / 1024;
  static_assert(NINST % NW == 0, "tile must split evenly over the waves");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < NINST / NW; ++i) {
    const int j = wave + i * NW;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(r);
    const bf16* src = gbase + (long)row_src(r) * rs + 8 * c;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + j * 1024), 16, 0, 0);
  }
}

// Wait until this wave's asynchronous tile copies have landed.
__device__ __forceinline__ void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace attn
