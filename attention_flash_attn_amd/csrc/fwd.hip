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
//  * K/V tiles of 64 keys are double-buffered in LDS and filled asynchronously
//    by buffer loads into LDS (tile j+1 is in flight while tile j is consumed; one
//    barrier per tile), one copy instruction after each of the first score MFMAs.  Tiles are unpadded and XOR-swizzled (tile.hpp) so the
//    row reads of K and the transposing reads of V are bank-conflict free.
//    K rows are stored permuted (kRowPerm) so that the exponentiated score
//    registers are directly the B operand of O^T += V^T P^T.
//  * Online softmax in base 2 with scale*log2(e) folded into one FMA.  The
//    running max is only moved (and O, l rescaled) when the new tile max
//    exceeds it by more than 8 (log2 units), so the rescale is rare; the
//    unnormalised weights stay below 2^8 and the final division uses the
//    same reference max, so the result is the same softmax.
//  * Tiles whose keys are all masked are skipped; in partially valid tiles (a
//    ragged tail or a mask edge) a branch taken only there sets the excluded
//    scores to -inf, so full tiles carry no per-element mask work.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace attn {

template <int D, bool VARLEN>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BM = 128, BN = 64;
  constexpr int RB = 2 * D;       // tile row bytes
  constexpr int NKS = D / 16;     // MFMA reduction steps over the head dim
  constexpr int NMB = D / 32;     // 32-row blocks of O^T
  __shared__ __attribute__((aligned(1024))) char sK0[BN * RB];
  __shared__ __attribute__((aligned(1024))) char sK1[BN * RB];
  __shared__ __attribute__((aligned(1024))) char sV0[BN * RB];
  __shared__ __attribute__((aligned(1024))) char sV1[BN * RB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  const int logical = xcd_remap(blockIdx.x, p.n_blocks);
  // Causal: the last query tiles see the most keys, so they are dealt out first.
  const int qt = p.causal ? p.n_qtiles - 1 - logical % p.n_qtiles : logical % p.n_qtiles;
  const int rest = logical / p.n_qtiles;
  // (outer, head) groups go head-major: each XCD's contiguous range of groups then holds
  // every batch|sequence of a few heads, so the ranges carry equal work even when the
  // sequences differ in length (varlen) or in valid keys (mask).
  const int head = rest / p.B, outer = rest % p.B;
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

  // Q/out rows hold H heads, K/V rows Hk; query head h reads key/value head h / G.
  const long rs = (long)p.H * D, rsk = (long)p.Hk * D;
  const int kvh = head / p.G;
  const bf16* kbase = p.k + (long)krow0 * rsk + (long)kvh * D;
  const bf16* vbase = p.v + (long)krow0 * rsk + (long)kvh * D;

  // Query rows of this wave, as B operand slices over the head dim.
  const int qrow = qb + wave * 32 + l32;
  bf16x8 qreg[NKS];
  {
    const bf16* qp = p.q + ((long)qrow0 + min(qrow, nq - 1)) * rs + (long)head * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = as_bf16x8(ld16(qp + 16 * ks));
  }

  // Per-lane swizzled LDS offsets: K rows (MFMA A operand, one row per lane) and the
  // transposing V reads (lane group g, source lane src; see lds_read_tr16).
  int koff[NKS], voff[NMB][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = tile_off<D>(l32, 2 * ks + hl);
  {
    const int g = lane >> 4, src = lane & 15;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        voff[mb][half] = tile_off_tr<D>(8 * (g >> 1) + 4 * half + (src >> 2),
                                        32 * mb + 16 * (g & 1) + 4 * (src & 3));
  }

  TileLoader<D, BN, 4> kld, vld;
  auto krow = [](int r) { return perm32_row(r); };
  auto vrow = [](int r) { return r; };
  kld.init(rsk, krow);
  vld.init(rsk, vrow);
  auto issue = [&](int k0, char* kt, char* vt) {
    kld.issue(kt, kbase, rsk, k0, nk, krow);
    vld.issue(vt, vbase, rsk, k0, nk, vrow);
  };

  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.c2;

  // Tiles that need per-element masking: not every key valid (mask, ragged tail), or, when
  // causal, some key of the tile after some query row of the workgroup.
  auto needs_mask = [&](int k0, uint64_t vw) { return vw != ~0ull || (p.causal && k0 + BN - 1 > qb); };
  // The copy of the next tile (n0 >= 0: its first key; a tile whose keys all exist) is
  // issued one instruction at a time between the score MFMAs: each copy instruction holds
  // the wave at issue for a while, and there the matrix unit still works on the MFMA
  // before it.
  auto compute = [&](auto spread, const char* kt, const char* vt, int k0, uint64_t vw, int n0,
                     char* kn, char* vn) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    constexpr int NI = decltype(kld)::NI;
    const auto krs = kld.rsrc(kbase, rsk, n0), vrs = vld.rsrc(vbase, rsk, n0);
    static_assert(2 * NI <= 2 * NKS, "one copy instruction per score MFMA at most");
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = mfma32(lds_row16(kt, kb * 32 * RB + koff[ks]), qreg[ks], sacc[kb]);
        const int n = 2 * ks + kb;
        if (decltype(spread)::value && n < 2 * NI) {
          if (n < NI)
            kld.issue_one_full(n, kn, krs);
          else
            vld.issue_one_full(n - NI, vn, vrs);
        }
      }
    if (decltype(spread)::value) {
      // K row reads two MFMAs ahead, one copy instruction after each of the first MFMAs.
      ATTN_SCHED(kSchedDSRead, 2);
#pragma unroll
      for (int n = 0; n < 2 * NKS; ++n) {
        ATTN_SCHED(kSchedMFMA, 1);
        if (n < 2 * NI) ATTN_SCHED(kSchedVMEMRead, 1);
        if (n + 2 < 2 * NKS) ATTN_SCHED(kSchedDSRead, 1);
      }
    }
    if (needs_mask(k0, vw)) {
      keep_branch();
      // Register r of half kb holds key k0 + 32kb + 16(r/8) + 8hl + r%8 (its bit in vw is
      // that minus k0) of this lane's query row qrow.
      const uint64_t vl = vw >> (8 * hl);
      const uint32_t w2[2] = {(uint32_t)vl, (uint32_t)(vl >> 32)};
      const int last = p.causal ? qrow - k0 - 8 * hl : BN;  // largest visible key - k0 - 8hl
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 16 * (r >> 3) + (r & 7);
          const bool on = ((w2[kb] >> (16 * (r >> 3) + (r & 7))) & 1u) && kr <= last;
          sacc[kb][r] = on ? sacc[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = wave_max_halves(mx);
    const float mt = mx * c2;
    if (__ballot(mt > m_run + 8.0f)) {
      keep_branch();
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
          const char* vb = vt + (32 * kb + 16 * t) * RB;
          oacc[mb] = mfma32(lds_tr8(vb, voff[mb][0], voff[mb][1]), pk[kb][t], oacc[mb]);
        }
  };

  // Causal: keys past the workgroup's last query row are never seen.
  const int kend = p.causal ? min(nk, min(qb + BM, nq)) : nk;
  const int ntiles = (kend + BN - 1) / BN;
  uint64_t vw = 0;
  const KeyValidity kv{mask, nk};
  uint32_t mbytes = 0;  // raw mask bytes of tile j + 1 during step j
  // Current and next tile buffers as distinct __restrict__ parameters: once inlined,
  // the compiler can tell reads of one from the asynchronous copy into the other
  // (without that it waits for the copy before the first LDS read).
  auto step = [&](int j, const char* __restrict__ kt, const char* __restrict__ vt,
                  char* __restrict__ kn, char* __restrict__ vn) {
    const bool more = j + 1 < ntiles;
    uint64_t vw_next = 0;
    if (more) {
      vw_next = kv.word((j + 1) * BN, mbytes);
      mbytes = kv.load((j + 2) * BN);  // clamped: unused past the last tile
    }
    // The next tile's copy: spread over the score MFMAs when there are any and the tile is
    // whole, else all at once here.
    const bool spread = more && vw != 0 && (j + 2) * BN <= nk;
    if (more && !spread) issue((j + 1) * BN, kn, vn);
    if (spread)
      compute(std::true_type{}, kt, vt, j * BN, vw, (j + 1) * BN, kn, vn);
    else if (vw != 0)
      compute(std::false_type{}, kt, vt, j * BN, vw, 0, kn, vn);
    wait_tile_loads();
    __syncthreads();
    vw = vw_next;
  };
  if (ntiles > 0) {
    vw = kv.word(0, kv.load(0));
    mbytes = kv.load(BN);
    issue(0, sK0, sV0);
    wait_tile_loads();
  }
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    step(j, sK0, sV0, sK1, sV1);
    if (j + 1 < ntiles) step(j + 1, sK1, sV1, sK0, sV0);
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
