// fwd.hip -- attention forward for gfx950: out = softmax(scale * Q K^T) V and LSE.
//
// The forward op of the op pairs in diffusers PR #14341 (body): BSHD in, out in
// BSHD, log-sum-exp per query row (kept because the backward needs it, same
// PR, follow-up 1).  Keys excluded by the head-broadcast bool mask act as a
// -inf bias (same PR, follow-up 2; diffusers PR #14834, "Unsupported cases").
//
// Design (one workgroup = 4 waves = 128 query rows of one (batch|sequence, head)):
//  * Each wave keeps its 32 query rows in registers as the B operand of
//    S^T = K Q^T, so the score tile arrives with one query per lane and all
//    row statistics (max, sum, LSE) are per-lane values; the only cross-lane
//    step is one exchange between the two 32-lane halves.
//  * K/V tiles of 64 keys are double-buffered through LDS: the global loads of
//    tile j+1 are in flight while tile j is consumed; one barrier per tile.
//    K rows are stored permuted (kRowPerm) so that the exponentiated score
//    registers are directly the B operand of O^T += V^T P^T; V^T comes from
//    row-major V with the LDS transposing read.
//  * Online softmax in base 2 with scale*log2(e) folded into one FMA.  The
//    running max is only moved (and O, l rescaled) when the new tile max
//    exceeds it by more than 8 (log2 units), so the rescale is rare; the
//    unnormalised weights stay below 2^8 and the final division uses the
//    same reference max, so the result is the same softmax.
//  * Tiles whose keys are all masked are skipped; partially valid tiles (a
//    ragged tail or a mask edge) set the excluded scores to -inf.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

template <int D, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D + 8, VS = D + 8;  // LDS row strides (elements), 16 B of padding
  constexpr int NKS = D / 16;            // MFMA reduction steps over the head dim
  constexpr int NMB = D / 32;            // 32-row blocks of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;         // rows staged per pass
  constexpr int NPASS = BN / RPP;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * KS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][BN * VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, p.n_blocks);
  const int qt = logical % p.n_qtiles;
  const int rest = logical / p.n_qtiles;
  const int head = rest % p.H, outer = rest / p.H;
  int qrow0, krow0, nq, nk;
  long lse_base;
  const uint8_t* mask = nullptr;
  if (VARLEN) {
    const int s0 = p.cu[outer], s1 = p.cu[outer + 1];
    qrow0 = krow0 = s0;
    nq = nk = s1 - s0;
    lse_base = (long)head * p.Sq + s0;
  } else {
    qrow0 = outer * p.Sq;
    krow0 = outer * p.Sk;
    nq = p.Sq;
    nk = p.Sk;
    lse_base = ((long)outer * p.H + head) * p.Sq;
    if (p.mask) mask = p.mask + (long)outer * p.Sk;
  }
  const int qb = qt * BM;
  if (qb >= nq) return;  // block-uniform: a varlen tile past its sequence

  const long rs = (long)p.H * D;
  const bf16* kbase = p.k + (long)krow0 * rs + (long)head * D;
  const bf16* vbase = p.v + (long)krow0 * rs + (long)head * D;

  // Query rows of this wave, as B operand slices over the head dim.
  const int qrow = qb + wave * 32 + l32;
  bf16x8 qreg[NKS];
  {
    const bf16* qp = p.q + ((long)qrow0 + qrow) * rs + (long)head * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 z = {0, 0, 0, 0};
      qreg[ks] = as_bf16x8(qrow < nq ? ld16(qp + 16 * ks) : z);
    }
  }

  // Staging: thread -> (chunk c, rows r0 + i*RPP).
  const int sc = tid % CPR, sr0 = tid / CPR;
  u32x4 kr[NPASS], vr[NPASS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int key = k0 + sr0 + i * RPP;
      const u32x4 z = {0, 0, 0, 0};
      kr[i] = key < nk ? ld16(kbase + (long)key * rs + 8 * sc) : z;
      vr[i] = key < nk ? ld16(vbase + (long)key * rs + 8 * sc) : z;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int r = sr0 + i * RPP;
      const int rk = (r & ~31) | kRowPerm(r & 31);
      *reinterpret_cast<u32x4*>(&sK[buf][rk * KS + 8 * sc]) = kr[i];
      *reinterpret_cast<u32x4*>(&sV[buf][r * VS + 8 * sc]) = vr[i];
    }
  };
  auto tile_valid = [&](int k0) -> uint64_t {
    const int key = k0 + lane;
    bool ok = key < nk;
    if (ok && mask) ok = mask[key] != 0;
    return __ballot(ok);
  };

  // Per-lane offset of the transposing V read (see lds_read_tr16).
  const int g = lane >> 4, src = lane & 15;
  const int vt_off = (8 * (g >> 1) + (src >> 2)) * VS + 16 * (g & 1) + 4 * (src & 3);

  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.c2;

  const int ntiles = (nk + BN - 1) / BN;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  uint64_t vw = ntiles > 0 ? tile_valid(0) : 0;

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < ntiles;
    uint64_t vw_next = 0;
    if (more) {
      load_tile((j + 1) * BN);
      vw_next = tile_valid((j + 1) * BN);
    }
    if (vw != 0) {
      const bf16* sKb = sK[buf];
      const bf16* sVb = sV[buf];
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sKb[(32 * kb + l32) * KS + 16 * ks + 8 * hl]);
          sacc[kb] = mfma32(a, qreg[ks], sacc[kb]);
        }
      }
      if (vw != ~0ull) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((vw >> (32 * kb + c_row_permuted(r, hl))) & 1ull)) sacc[kb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = wave_max_halves(mx);
      const float mt = mx * c2;
      if (__ballot(mt > m_run + 8.0f)) {
        const float mnew = fmaxf(m_run, mt);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
        m_run = mnew;
      }
      const float muse = m_run == -INFINITY ? 0.f : m_run;
      bf16x8 pk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, -muse));
          sacc[kb][r] = x;
          l_run += x;
        }
        pk[kb][0] = pack8(sacc[kb], 0);
        pk[kb][1] = pack8(sacc[kb], 8);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16* vp = sVb + (32 * kb + 16 * t) * VS + 32 * mb + vt_off;
            const bf16x8 a = cat_tr(lds_read_tr16(vp), lds_read_tr16(vp + 4 * VS));
            oacc[mb] = mfma32(a, pk[kb][t], oacc[mb]);
          }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    vw = vw_next;
  }

  l_run = wave_sum_halves(l_run);
  if (qrow < nq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16* op = p.out + ((long)qrow0 + qrow) * rs + (long)head * D + 4 * hl;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[mb][4 * j4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * mb + 8 * j4) = o;
      }
    if (hl == 0)
      p.lse[lse_base + qrow] = l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, bool VARLEN>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  if (p.n_blocks == 0) return hipSuccess;
  void* args[] = {const_cast<FwdParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<D, VARLEN>), dim3(p.n_blocks),
                         dim3(256), args, 0, stream);
}

hipError_t launch_fwd(int D, bool varlen, const FwdParams& p, hipStream_t stream) {
  if (D == 64) return varlen ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return varlen ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
}

}  // namespace attn
