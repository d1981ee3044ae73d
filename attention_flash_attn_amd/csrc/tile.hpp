// tile.hpp -- LDS tiles for gfx950: unpadded rows, 16-byte chunks XOR-swizzled, filled
// asynchronously by buffer_load_dwordx4 ... lds.
//
// A tile holds R rows of D bf16 (2*D bytes per row, no padding).  The 16-byte
// chunk c of row r is stored at chunk position c ^ swz(r).  The LDS has 64 banks of 4
// bytes (256 bytes per bank row), and the swizzle keeps both read patterns of the
// 16x16x32 operands conflict-free under the way gfx950 serves them (measured with an
// in-bounds probe: a pair of lanes on one bank costs an extra cycle only inside one
// service group):
//  * ds_read_b128 (row reads of MFMA operands) is served in four groups of 16 lanes,
//    {0-3, 12-15, 20-23, 24-27}, {4-7, 8-11, 16-19, 28-31} and the same two plus 32; each
//    group must touch 16 distinct 16-byte bank groups.  The kernels' row reads put lane
//    16 g + c on row c (mod 16) at logical chunk 4 ks + g, so a group holds rows
//    {0-3, 12-15} of one g and rows {4-11} of g ^ 1: swz maps rows 4..11 onto whole
//    chunk pairs {2k, 2k+1} (positions 8..15 at D = 128) and rows {0-3, 12-15} onto the
//    other pairs; the two g of a group differ in bit 0 of the chunk, which maps every
//    pair onto itself, so the two halves of a group stay apart.  (The earlier swizzle, 2 (r & 7) + (r >> 3 & 1), was conflict-free for groups of
//    16 consecutive lanes and measured 8.2 instead of 4.7 cycles per read.)
//  * ds_read_b64_tr_b16 (transposing reads) is served as one 64-lane request in at least
//    two cycles, one more for each further distinct address on a bank.  Lane 16 g + c reads
//    row 4 g + c / 4 (mod 16) at logical chunks {2m, 2m + 1}, i.e. physical pair
//    m ^ (swz(r) >> 1); swz(r) >> 1 takes distinct values on rows 0..7 and on rows 8..15
//    (at D = 64 on the rows of one parity, which share a 256-byte bank row), so every bank
//    holds exactly two of the 512 bytes (this also holds if the request were split into
//    32-lane halves).
// At D = 64 two rows share one bank row (r & 1 selects its half), and the same
// construction applies to the rows of each parity.  swz depends only on r & 15, so moving
// by a multiple of 16 rows keeps offsets.
//
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes to LDS at M0 + 16*l, i.e. one
// instruction fills 1 KiB of LDS contiguously; the swizzle is applied on the
// global side by choosing which chunk each lane fetches.
#pragma once
#include "common.hpp"

namespace attn {

typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource (stride 0, byte-addressed, 32-bit data format).
constexpr int kBufferFlags = 0x00020000;

template <int D>
__host__ __device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  const int b = (r >> 3) & 1;
  const int pair = D == 128 ? ((r & 7) ^ (b << 2)) : (((r >> 1) & 3) ^ (b << 1));
  return (pair << 1) | b;
}

// Byte offset of (row r, logical 16-byte chunk c) inside a tile.
template <int D>
__host__ __device__ __forceinline__ int tile_off(int r, int c) {
  return r * (2 * D) + ((c ^ swz<D>(r)) << 4);
}

// Byte offset of the 8-byte group holding elements [col, col+4) of row r (col % 4 == 0).
template <int D>
__host__ __device__ __forceinline__ int tile_off_tr(int r, int col) {
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

// Asynchronous tile copy with NW waves, by buffer_load_dwordx4 ... lds: the tile's first
// row is the base of a buffer resource built per tile in scalar registers, so each lane
// keeps only 32-bit offsets.  Lane-dependent parts of the offsets are fixed per kernel,
// so they are computed once: off[i] is the byte offset, from the tile's first row, of the
// 16-byte chunk this lane fetches with its i-th instruction.  row_of(r) maps tile row r
// to its row offset within the tile (a permutation of 0..ROWS-1; the kernels use the
// identity).  In a tile that runs
// past the last valid row, the copies of the missing rows fall outside the buffer range
// and fill their LDS with zeros (issue() below): every access stays inside the tensor, and
// a tail tile costs no per-lane work.
template <int D, int ROWS, int NW>
struct TileLoader {
  static constexpr int CPR = D / 8;            // chunks per row
  static constexpr int RPI = 1024 / (2 * D);   // rows per instruction (4 or 8)
  static constexpr int NI = ROWS * 2 * D / 1024 / NW;
  static_assert(ROWS * 2 * D % (1024 * NW) == 0, "tile must split evenly over the waves");
  uint32_t off[NI];
  int wv;  // this wave's index among the NW copying waves (waves w0 .. w0 + NW - 1)

  template <typename RowOf>
  __device__ __forceinline__ void init(long rs, RowOf row_of, int w0 = 0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) - w0);
    wv = wave;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave + i * NW) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(r);
      off[i] = (uint32_t)(2 * ((long)row_of(r) * rs + 8 * c));
    }
  }

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, char* tile, int i, uint32_t o) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + (wv + i * NW) * 1024), 16, o, 0, 0, 0);
  }

  // Copy rows [row0, row0 + ROWS) of the tensor whose row 0 (this head) is at `base`; only
  // rows < nrows exist.  The buffer resource starts at row row0 and its byte range ends at
  // the last of them (min(ROWS, nrows - row0) rows of 2 rs bytes; the callers keep
  // ROWS * 2 * rs < 2^31), so the lanes of rows past the end read nothing and the hardware
  // writes zeros to their 16 bytes of LDS.
  __device__ __forceinline__ void issue(char* tile, const bf16* base, long rs, int row0, int nrows) const {
    const int n = min(ROWS, nrows - row0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(base + (long)row0 * rs), (short)0, (int)(n * 2 * rs), kBufferFlags);
#pragma unroll
    for (int i = 0; i < NI; ++i) load(r, tile, i, off[i]);
  }
};

// Key validity of the tiles of a loop over keys: bit i of a tile's word says that key
// k0 + i exists and is not excluded by the mask.  The mask bytes are read raw (index
// clamped, no arithmetic) one step before they are turned into a word, so the load never
// holds up the wave: a use right after it would wait for the tile copies issued with it.
struct KeyValidity {
  const uint8_t* mask;  // null: every existing key is valid
  int nk;
  __device__ __forceinline__ uint32_t load(int k0) const {
    uint32_t b = 1u;
    // nk = 0: no byte of the mask exists (the clamped index would be -1)
    if (mask && nk > 0) b = mask[min(k0 + (int)(threadIdx.x & 63), nk - 1)];
    return b;
  }
  __device__ __forceinline__ uint64_t word(int k0, uint32_t b) const {
    return __ballot(k0 + (int)(threadIdx.x & 63) < nk && b != 0u);
  }
};

// Wait until this wave's asynchronous tile copies have landed.
__device__ __forceinline__ void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace attn
