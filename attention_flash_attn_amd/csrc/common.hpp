// common.hpp -- device helpers shared by the libattn kernels (gfx950 only).
//
// MFMA: every product runs on v_mfma_f32_16x16x32_bf16 (wave64; layout verified on the
// GPU with an in-bounds probe):
//   A (16 x 32): lane l holds row l%16, reduction slots 8*(l/16) .. +7
//   B (32 x 16): lane l holds column l%16, reduction slots 8*(l/16) .. +7
//   C (16 x 16): lane l holds column l%16; register i holds row 4*(l/16) + i
// Any fixed assignment of reduction slots to a real index works as long as A and B agree,
// which is how score blocks are fed back in as operands without a shuffle: the kernels'
// transposing reads fetch the other operand in the order the score registers hold.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, four at a time.
__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) {
  bf16x4 b;
#pragma unroll
  for (int e = 0; e < 4; ++e) b[e] = (bf16)x[e];
  return b;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load / store as raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS transposing read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// destination lane j, element e receives element (j%4) of the 4-element chunk
// addressed by source lane 4*e + j/4 of the same group.
__device__ __forceinline__ i16x4 lds_read_tr16(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Eight fp32 values -> bf16x8 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[base + i];
  return r;
}

// Workgroups are dealt round-robin over the 8 XCDs; renumber them so that each
// XCD receives one contiguous range of logical tiles (neighbouring tiles share
// K/V and stay in that XCD's L2).  Bijective for any n.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;
// Ask the scheduler for a group of n instructions of class `mask` next in the
// current basic block (groups are filled in the order they are requested).
#define ATTN_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Placed first in a rarely taken, wave-uniform branch: an empty volatile asm has
// side effects, so the compiler keeps the branch instead of flattening its body
// into selects executed on every iteration.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

}  // namespace attn
