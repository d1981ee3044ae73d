// merge.hip -- merge of partial attention results over disjoint key chunks, and the
// fp32 -> bf16 rounding of gradients accumulated over such chunks.
//
// Ring (context-parallel) attention splits the keys of one attention into chunks; its
// backward is named as not yet implemented in diffusers PR #14834 (description) and left
// unverified in diffusers PR #14341 ("Not verified").  The forward of chunk c gives out_c,
// normalised over the chunk's own keys, and lse_c.  Since softmax over all keys is the
// chunk softmaxes reweighted by each chunk's share of the total exponential mass (a
// consequence of the definition; the pages print no formula):
//   LSE = log sum_c exp(lse_c),   out = sum_c exp(lse_c - LSE) out_c.
// A chunk with no key for a row has lse_c = -inf and weight 0; a row with no key in any
// chunk gets out = 0 and LSE = -inf, as the forward itself returns for it.
//
// Memory-bound: each lane owns 16 bytes of one (b, s, h) row (8 lanes per row at D=64,
// 16 at D=128) and reads those 16 bytes of every chunk once; all lanes of a row sit in
// one wave, so the row's LSE is read by all of them before one of them writes it, and
// the merge may run in place (out and lse aliasing chunk 0's, say).
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int CPR = D / 8;      // lanes per row
  constexpr int RPB = 256 / CPR;  // rows per workgroup
  const long row = (long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  if (row >= p.rows) return;
  const long h = row % p.H, bs = row / p.H;
  const long s = bs % p.S, b = bs / p.S;
  const long li = (b * p.H + h) * p.S + s;

  float l[kMaxMergeChunks];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeChunks; ++i)
    if (i < p.n) {
      l[i] = p.lse[i][li];
      m = fmaxf(m, l[i]);
    }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxMergeChunks; ++i)
    if (i < p.n) {
      l[i] = m == -INFINITY ? 0.f : expf(l[i] - m);  // exp(-inf) = 0 for empty chunks
      sum += l[i];
    }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kMaxMergeChunks; ++i)
    if (i < p.n) {
      const float w = l[i] * inv;
      const bf16x8 x = as_bf16x8(ld16(p.out[i] + row * D + 8 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, (float)x[e], acc[e]);
    }
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)acc[e];
  *reinterpret_cast<bf16x8*>(p.dst + row * D + 8 * c) = o;
  if (c == 0) p.dst_lse[li] = sum > 0.f ? m + logf(sum) : -INFINITY;
}

hipError_t launch_merge(int D, const MergeParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const long rpb = 256 / (D / 8);
  const long nb = (p.rows + rpb - 1) / rpb;
  void* args[] = {const_cast<MergeParams*>(&p)};
  const void* fn = D == 64 ? reinterpret_cast<const void*>(&merge_kernel<64>)
                           : reinterpret_cast<const void*>(&merge_kernel<128>);
  return hipLaunchKernel(fn, dim3((unsigned)nb), dim3(256), args, 0, stream);
}

// dst[i] = bf16(src[i]) (nearest even); each workgroup covers 2048 consecutive elements
// with lane-consecutive accesses.
__global__ __launch_bounds__(256) void cast_kernel(long n, const float* __restrict__ src,
                                                   bf16* __restrict__ dst) {
  const long base = (long)blockIdx.x * 2048 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const long i = base + 256 * j;
    if (i < n) dst[i] = (bf16)src[i];
  }
}

hipError_t launch_cast_bf16(long n, const float* src, bf16* dst, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const long nb = (n + 2047) / 2048;
  void* args[] = {&n, &src, &dst};
  return hipLaunchKernel(reinterpret_cast<const void*>(&cast_kernel), dim3((unsigned)nb), dim3(256),
                         args, 0, stream);
}

}  // namespace attn
