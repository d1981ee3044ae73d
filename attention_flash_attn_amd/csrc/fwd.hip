// fwd.hip -- attention forward for gfx950: out = softmax(scale * Q K^T) V and LSE.
//
// The forward op of the op pairs in diffusers PR #14341 (body): BSHD in, out in
// BSHD, log-sum-exp per query row (kept because the backward needs it, same
// PR, follow-up 1).  Keys excluded by the head-broadcast bool mask act as a
// -inf bias (same PR, follow-up 2; diffusers PR #14834, "Unsupported cases").
//
// Design (one workgroup = 8 waves = 256 query rows of one (batch|sequence, head), one
// workgroup per CU):
//  * Each wave keeps its 32 query rows in registers as the B operand of
//    S^T = K Q^T, so the score tile arrives with one query per lane and all
//    row statistics (max, sum, LSE) are per-lane values; the only cross-lane
//    step is one exchange between the two 32-lane halves.
//  * K/V tiles of 64 keys are double- or triple-buffered in LDS and filled
//    asynchronously by buffer loads into LDS.  Tiles are unpadded and XOR-swizzled
//    (tile.hpp) so the row reads of K and the transposing reads of V are bank-conflict
//    free.  K rows are stored permuted (kRowPerm) so that the exponentiated score
//    registers are directly the B operand of O^T += V^T P^T.
//  * Ping-pong: the two 4-wave groups (one wave of each per SIMD) run half a tile
//    apart, so one group's MFMAs overlap the other group's softmax (see fwd_kernel).
//  * Online softmax in base 2 with scale*log2(e) folded into one FMA, against a lazily
//    moved reference: a tile's weights are formed against the row's current reference
//    max, and the reference (with O and l rescaled) only moves when some row's tile sum
//    exceeds 2^14, so every weight stays below 2^14 and the final division uses the same
//    reference, which gives the same softmax.
//  * Tiles whose keys are all masked are skipped; in partially valid tiles (a
//    ragged tail or a mask edge) a branch taken only there sets the excluded
//    scores to -inf, so full tiles carry no per-element mask work.
//  * Split tail workgroups: when the grid's last round would leave CUs idle, its query
//    tiles run as two or four workgroups each whose wave groups share out the keys and
//    combine their softmax states in LDS (see fwd_kernel).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace attn {

// Waves 0..3 (group A) and 4..7 (group B) sit one per SIMD each (wave w and w + 4 share a
// SIMD), so every SIMD holds one wave of each group.  The loop below is the one for
// masked and causal attention; dense attention runs a variant of it (dense_run) with a
// fused MFMA phase and the copies shared between the groups.
// The loop runs in phases separated by workgroup barriers, and the two groups are half a
// key tile apart: in each phase one group issues its MFMAs (O += P V for the previous
// tile, then S^T = K Q^T for the current one) while the other does the softmax VALU work,
// so the matrix units of a SIMD are fed by one wave while the other computes exponentials.
//   phase 2j  : A: PV(j-1), S(j)      B: softmax(j-1); B issues the copies of K(j+1), V(j)
//   phase 2j+1: A: softmax(j)         B: PV(j-1), S(j)
// B's copies have landed when phase 2j ends (__syncthreads() waits for the wave's
// outstanding loads before the barrier).  K(j) is read in phases 2j, 2j+1 and V(j) in
// phases 2j+2, 2j+3, so two buffers each suffice: a copy issued in phase 2j overwrites a
// tile last read in phase 2j-1.
template <int D, bool VARLEN>
__global__ __launch_bounds__(512, 1) void fwd_kernel(FwdParams p) {
  constexpr int BM = kFwdBlockM, BN = 64;
  constexpr int RB = 2 * D;
  constexpr int NKS = D / 16;
  constexpr int NMB = D / 32;
  constexpr int TILE = BN * RB;  // bytes of one K or V tile
  // Ping-pong workgroups use the first four tiles; a split workgroup (below) gives each
  // wave group four of its own.
  __shared__ __attribute__((aligned(1024))) char smem[8 * TILE];
  char* const sK0 = smem;
  char* const sK1 = smem + TILE;
  char* const sV0 = smem + 2 * TILE;
  char* const sV1 = smem + 3 * TILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_b = wave >= 4;
  const int hl = lane >> 5, l32 = lane & 31;

  // Blocks from p.n_full on are split workgroups: the p.split parts (256 / p.split rows) of
  // the query tiles n_full, n_full + 1, ..., each with its keys shared out between p.split
  // wave groups (see the split loop below).  They only exist for a non-causal dense launch
  // whose last round of full workgroups would leave most CUs idle.
  const bool split = (int)blockIdx.x >= p.n_full;
  int qt, rest, part = 0;
  if (split) {
    const int b = (int)blockIdx.x - p.n_full, t = p.n_full + b / p.split;
    part = b % p.split;
    qt = t % p.n_qtiles;
    rest = t / p.n_qtiles;
  } else if (p.causal) {
    // The last query tiles see the most keys: those of every (head, outer) first, over the
    // whole grid in plain block order (dealt round-robin to the XCDs).
    const int nbh = p.B * p.H;
    qt = p.n_qtiles - 1 - (int)blockIdx.x / nbh;
    rest = (int)blockIdx.x % nbh;
  } else {
    // Equal workgroups: consecutive query tiles of one head share an XCD range (and its
    // L2 holds that head's K and V); plain block order measured 2.6% slower.
    const int logical = xcd_remap(blockIdx.x, p.n_full);
    qt = logical % p.n_qtiles;
    rest = logical / p.n_qtiles;
  }
  // varlen: sequence ranks, longest first (see SeqOrder)
  const int head = rest / p.B, outer = VARLEN ? p.order(rest % p.B) : rest % p.B;
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
  const int qb = qt * BM + (split ? part * (BM / p.split) : 0);  // first row of this workgroup
  if (qb >= nq) return;  // block-uniform

  const long rs = (long)p.H * D, rsk = (long)p.Hk * D;
  const int kvh = head / p.G;
  const bf16* kbase = p.k + (long)krow0 * rsk + (long)kvh * D;
  const bf16* vbase = p.v + (long)krow0 * rsk + (long)kvh * D;

  // this wave's first query row (a split workgroup holds 8 / p.split row blocks of 32)
  const int qw = qb + (split ? wave % (8 / p.split) : wave) * 32;
  const int qrow = qw + l32;
  bf16x8 qreg[NKS];
  {
    const bf16* qp = p.q + ((long)qrow0 + min(qrow, nq - 1)) * rs + (long)head * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = as_bf16x8(ld16(qp + 16 * ks));
  }
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

  TileLoader<D, BN, 4> kld, vld;  // the masked / causal loop: used by group B only
  auto krow = [](int r) { return perm32_row(r); };
  auto vrow = [](int r) { return r; };
  kld.init(rsk, krow, 4);
  vld.init(rsk, vrow, 4);

  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};
  f32x16 sacc[2];
  bf16x8 pk[2][2];
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.c2;
  const std::integral_constant<int, 2> kTwoHalves{};

  const int kend = p.causal ? min(nk, min(qb + BM, nq)) : nk;
  const int ntiles = (kend + BN - 1) / BN;
  const KeyValidity kv{mask, nk};
  // Per wave: the key-validity word of the tile whose scores were formed last (0: nothing
  // in it for this wave; its softmax and P V are skipped).
  uint64_t vw_s = 0;
  uint32_t mbytes = 0;
  auto tile_word = [&](int j, uint32_t bytes) -> uint64_t __attribute__((always_inline)) {
    // causal: a tile whose first key comes after this wave's last row is skipped
    if (j >= ntiles || (p.causal && j * BN > qw + 31)) return 0;
    return kv.word(j * BN, bytes);
  };

  // Operand reads run several MFMAs ahead (explicit schedule): with one wave per SIMD in
  // its MFMA phase, nothing else hides an LDS read's latency from the matrix unit.
  // kbc: the tile's number of 32-key halves (2, or 1 in the 32-key tiles of 4-way split
  // workgroups), as a compile-time constant.
  auto gemm_s = [&](const char* kt, auto kbc) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        sacc[kb] = mfma32(lds_row16(kt, kb * 32 * RB + koff[ks]), qreg[ks], sacc[kb]);
    constexpr int AHEAD = 6, N = KB * NKS;
    ATTN_SCHED(kSchedDSRead, AHEAD);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      ATTN_SCHED(kSchedMFMA, 1);
      if (n + AHEAD < N) ATTN_SCHED(kSchedDSRead, 1);
    }
  };
  auto gemm_pv = [&](const char* vt, auto kbc) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const char* vb = vt + (32 * kb + 16 * t) * RB;
          oacc[mb] = mfma32(lds_tr8(vb, voff[mb][0], voff[mb][1]), pk[kb][t], oacc[mb]);
        }
    constexpr int AHEAD = 4, N = 2 * KB * NMB;  // MFMAs; two transposing reads each
    ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      ATTN_SCHED(kSchedMFMA, 1);
      if (n + AHEAD < N) ATTN_SCHED(kSchedDSRead, 2);
    }
  };
  // O += P V of the previous tile, then S^T = K Q^T of this one, as one read pipeline: the
  // first K reads issue under the last P V MFMAs, so the matrix unit does not wait for
  // them between the two products.
  auto gemm_pv_s = [&](const char* vt, const char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const char* vb = vt + (32 * kb + 16 * t) * RB;
          oacc[mb] = mfma32(lds_tr8(vb, voff[mb][0], voff[mb][1]), pk[kb][t], oacc[mb]);
        }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = mfma32(lds_row16(kt, kb * 32 * RB + koff[ks]), qreg[ks], sacc[kb]);
    // MFMA n < NPV reads two transposed V fragments, the others one K row fragment.
    constexpr int AHEAD = 4, NPV = 4 * NMB, N = NPV + 2 * NKS;
    ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      ATTN_SCHED(kSchedMFMA, 1);
      if (n + AHEAD < NPV) ATTN_SCHED(kSchedDSRead, 2);
      else if (n + AHEAD < N) ATTN_SCHED(kSchedDSRead, 1);
    }
  };
  auto softmax = [&](int k0, uint64_t vw, auto kbc) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value;
    constexpr uint64_t kFull = KB == 2 ? ~0ull : 0xFFFFFFFFull;  // bits of the tile's keys
    if ((vw & kFull) != kFull || (p.causal && k0 + 32 * KB - 1 > qw)) {
      keep_branch();
      // Register r of half kb holds key k0 + 32kb + 16(r/8) + 8hl + r%8 of row qrow.
      const uint64_t vl = vw >> (8 * hl);
      const uint32_t w2[2] = {(uint32_t)vl, (uint32_t)(vl >> 32)};
      const int last = p.causal ? qrow - k0 - 8 * hl : BN;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 16 * (r >> 3) + (r & 7);
          const bool on = ((w2[kb] >> (16 * (r >> 3) + (r & 7))) & 1u) && kr <= last;
          sacc[kb][r] = on ? sacc[kb][r] : -INFINITY;
        }
    }
    // Weights against the row's current reference m_run, with no max over the tile: the
    // exponent arguments y = c2 s - m_run stay in sacc, and the tile is accepted unless some
    // row's tile sum exceeds 2^14 (or overflows), which keeps every weight below 2^14.  The
    // first tile of a row (no reference yet) and the rare rejected tile form the tile max
    // from y, move the reference up by it, rescale O and l, and recompute the weights.
    const bool first = __ballot(m_run == -INFINITY) != 0;
    const float muse = m_run == -INFINITY ? 0.f : m_run;
    float la = 0.f, lb = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float y = fmaf(sacc[kb][8 * h + r], c2, -muse);
          sacc[kb][8 * h + r] = y;
          x[r] = __builtin_amdgcn_exp2f(y);
          if (r & 1) lb += x[r]; else la += x[r];
        }
        pk[kb][h] = pack8(x, 0);
      }
    float lt = la + lb;
    if (first || __ballot(!(lt <= 0x1p14f))) {
      keep_branch();
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = wave_max_halves(mx);
      const float mnew = fmaxf(m_run, muse + mx);
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mb][r] *= alpha;
      m_run = mnew;
      const float d = mnew == -INFINITY ? 0.f : mnew - muse;
      la = lb = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x16 x;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            x[r] = __builtin_amdgcn_exp2f(sacc[kb][8 * h + r] - d);
            if (r & 1) lb += x[r]; else la += x[r];
          }
          pk[kb][h] = pack8(x, 0);
        }
      lt = la + lb;
    }
    l_run += lt;
  };
  // MFMA phase of tile j: O += P(j-1) V(j-1), then S(j).  Group B then waits for the
  // copies it issued in its previous phase.
  auto gemm_phase = [&](int j, const char* __restrict__ kt, const char* __restrict__ vp)
      __attribute__((always_inline)) {
    if (vw_s != 0) gemm_pv(vp, kTwoHalves);  // vw_s: still the word of tile j-1
    vw_s = tile_word(j, mbytes);
    mbytes = kv.load((j + 1) * BN);  // clamped: unused past the last tile
    if (vw_s != 0) gemm_s(kt, kTwoHalves);
    if (grp_b) wait_tile_loads();
  };
  // VALU phase of tile j.  Group B first issues the copies of K(j+2) (into the buffer of
  // K(j), whose last reader was its own MFMA phase) and V(j+1) (into the buffer of V(j-1)).
  auto softmax_phase = [&](int j, char* __restrict__ kn, char* __restrict__ vn)
      __attribute__((always_inline)) {
    if (grp_b) {
      if (j + 2 < ntiles) kld.issue(kn, kbase, rsk, (j + 2) * BN, nk);
      if (j + 1 < ntiles) vld.issue(vn, vbase, rsk, (j + 1) * BN, nk);
    }
    if (vw_s != 0) softmax(j * BN, vw_s, kTwoHalves);
  };
  // Both groups run the same sequence, group B one phase later (it passes one barrier
  // before its first phase, group A one after its last), so register lifetimes at every
  // barrier are the same for both.
  // kc: the buffer of K(j) (and of K(j+2)), vp: the buffer of V(j-1) (and of V(j+1)).
  auto pair = [&](int j, char* __restrict__ kc, char* __restrict__ vp) __attribute__((always_inline)) {
    gemm_phase(j, kc, vp);
    __syncthreads();
    softmax_phase(j, kc, vp);
    __syncthreads();
  };

  // Dense ping-pong (no mask, non-causal): every tile before the end is valid for every
  // wave, so the MFMA phase of tile j is one read pipeline O += P(j-1) V(j-1), S(j)
  // (gemm_pv_s), with the first (S(0) only) and last (P V only) phases peeled.  K(j) and V(j)
  // sit in buffer j % 3 of each, and each group copies in its own VALU phase: group A
  // K(j+2) during softmax(j) (phase 2j+1), group B V(j+1) during its softmax(j) (phase
  // 2j+2), each waiting for its copies at the end of its next MFMA phase.  K(j+2) overwrites
  // K(j-1), last read in phase 2j-1; V(j+1) overwrites V(j-2), last read in phase 2j-1;
  // both are first read in phase 2j+4.  Splitting the copies halves the time a VALU phase
  // spends issuing them, and the phase barriers do not wait for copies in flight.
  // Dense ping-pong (no mask, non-causal): every tile before the end is valid for every
  // wave, so the MFMA phase of tile j is one read pipeline O += P(j-1) V(j-1), S(j)
  // (gemm_pv_s), with the first (S(0) only) and last (P V only) phases peeled.  K(j) and V(j)
  // sit in buffer j % 3 of each, and each group copies in its own VALU phase: group A
  // K(j+2) during softmax(j) (phase 2j+1), group B V(j+1) during its softmax(j) (phase
  // 2j+2), each waiting for its copies at the end of its next MFMA phase.  K(j+2) overwrites
  // K(j-1), last read in phase 2j-1; V(j+1) overwrites V(j-2), last read in phase 2j-1;
  // both are first read in phase 2j+4.  Splitting the copies halves the time a VALU phase
  // spends issuing them, and the phase barriers do not wait for copies in flight.
  auto dense_run = [&]() __attribute__((always_inline)) {
    char* const dK0 = smem;
    char* const dK1 = smem + TILE;
    char* const dK2 = smem + 2 * TILE;
    char* const dV0 = smem + 3 * TILE;
    char* const dV1 = smem + 4 * TILE;
    char* const dV2 = smem + 5 * TILE;
    // One loader per wave: group A copies K (rows permuted), group B copies V.  (Choosing
    // between two loader objects per group would put them in scratch memory.)
    TileLoader<D, BN, 4> cld;
    cld.init(rsk, [&](int r) { return grp_b ? r : perm32_row(r); }, 4 * grp_b);
    const bf16* const cbase = grp_b ? vbase : kbase;
    const int lead = grp_b ? 1 : 2;  // group A copies K(j+2), group B V(j+1)
    // A phase barrier that does not wait for copies in flight (__syncthreads() would).  Only
    // register operations can move across it: the compiler may issue the last MFMAs of a
    // phase after it, whose operands were read before it from buffers that the next phase
    // does not overwrite (measured 0.4% faster than keeping them in front).
    auto bar = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
    auto word = [&](int j) -> uint64_t __attribute__((always_inline)) { return kv.word(j * BN, 1u); };
    // VALU phase of tile j (kn: the buffer of K(j+2), vn: the buffer of V(j+1))
    auto vphase = [&](int j, char* __restrict__ kn, char* __restrict__ vn) __attribute__((always_inline)) {
      if (j + lead < ntiles) cld.issue(grp_b ? vn : kn, cbase, rsk, (j + lead) * BN, nk);
      softmax(j * BN, vw_s, kTwoHalves);
    };
    // pair of phases of tile j, 0 < j < ntiles (kt: K(j), vp: V(j-1))
    auto dpair = [&](int j, const char* __restrict__ kt, const char* __restrict__ vp,
                     char* __restrict__ kn, char* __restrict__ vn) __attribute__((always_inline)) {
      gemm_pv_s(vp, kt);
      vw_s = word(j);
      wait_tile_loads();
      bar();
      vphase(j, kn, vn);
      bar();
    };
    // K(0) and K(1) by group A, V(0) by group B, before the first phase
    if (grp_b) {
      cld.issue(dV0, vbase, rsk, 0, nk);
    } else {
      cld.issue(dK0, kbase, rsk, 0, nk);
      if (1 < ntiles) cld.issue(dK1, kbase, rsk, BN, nk);
    }
    wait_tile_loads();
    __syncthreads();
    if (grp_b) bar();  // phase 0: group A forms S(0)
    gemm_s(dK0, kTwoHalves);
    vw_s = word(0);
    wait_tile_loads();
    bar();
    vphase(0, dK2, dV1);
    bar();
    for (int j = 1; j < ntiles; j += 3) {  // j % 3 == 1, 2, 0
      dpair(j, dK1, dV0, dK0, dV2);
      if (j + 1 < ntiles) dpair(j + 1, dK2, dV1, dK1, dV0);
      if (j + 2 < ntiles) dpair(j + 2, dK0, dV2, dK2, dV1);
    }
    // phase pair ntiles: O += P V of the last tile only
    gemm_pv(smem + (3 + (ntiles - 1) % 3) * TILE, kTwoHalves);
    bar();
    bar();
    if (!grp_b) bar();
  };

  // Split workgroup: p.split groups of 8 / p.split waves take the same 256 / p.split rows
  // (wave w: row block w % (8 / p.split), group w / (8 / p.split)), group g the key tiles
  // [g hn, (g + 1) hn), each group with its own double-buffered K/V tiles and its own copies
  // (64-key tiles for two groups, 32-key tiles for four, so that every group's buffers fit);
  // all groups step in lockstep (one barrier per step).  The partial softmax states are
  // then combined through LDS.
  auto split_run = [&](auto sc) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    constexpr int RBK = 8 / S;               // row blocks, and waves per group
    constexpr int BNS = S == 2 ? 64 : 32;    // keys per tile
    constexpr int TS = BNS * RB;             // bytes of one K or V tile
    const std::integral_constant<int, BNS / 32> kb_c{};
    const int g = wave / RBK;
    const int nts = (kend + BNS - 1) / BNS;
    const int hn = (nts + S - 1) / S, t0 = g * hn, t1 = min(nts, t0 + hn);
    char* const gb = smem + 4 * TS * g;
    TileLoader<D, BNS, RBK> gk, gv;
    gk.init(rsk, krow, RBK * g);
    gv.init(rsk, vrow, RBK * g);
    auto word = [&](int j, uint32_t bytes) -> uint64_t __attribute__((always_inline)) {
      if (j >= nts || (p.causal && j * BNS > qw + 31)) return 0;
      return kv.word(j * BNS, bytes) & (BNS == 64 ? ~0ull : 0xFFFFFFFFull);
    };
    uint64_t vw = 0;
    auto sstep = [&](int j, const char* __restrict__ kt, const char* __restrict__ vt,
                     char* __restrict__ kn, char* __restrict__ vn) __attribute__((always_inline)) {
      const bool more = j + 1 < t1;
      uint64_t vw_next = 0;
      if (more) {
        vw_next = word(j + 1, mbytes);
        mbytes = kv.load((j + 2) * BNS);  // clamped: unused past the last tile
        gk.issue(kn, kbase, rsk, (j + 1) * BNS, nk);
        gv.issue(vn, vbase, rsk, (j + 1) * BNS, nk);
      }
      if (j < t1 && vw != 0) {
        gemm_s(kt, kb_c);
        softmax(j * BNS, vw, kb_c);
        gemm_pv(vt, kb_c);
      }
      wait_tile_loads();
      __syncthreads();
      vw = vw_next;
    };
    if (t0 < t1) {
      vw = word(t0, kv.load(t0 * BNS));
      mbytes = kv.load((t0 + 1) * BNS);
      gk.issue(gb, kbase, rsk, t0 * BNS, nk);
      gv.issue(gb + 2 * TS, vbase, rsk, t0 * BNS, nk);
    }
    wait_tile_loads();
    __syncthreads();
    for (int s = 0; s < hn; s += 2) {
      sstep(t0 + s, gb, gb + 2 * TS, gb + TS, gb + 3 * TS);
      if (s + 1 < hn) sstep(t0 + s + 1, gb + TS, gb + 3 * TS, gb, gb + 2 * TS);
    }
    // Combine: groups 1.. park (m, l, O) per lane in LDS (every tile read has completed at
    // the last step's barrier), group 0 merges them (m = max, each part scaled by 2^(m_g - m))
    // and stores.
    l_run = wave_sum_halves(l_run);
    constexpr int SLOT = 64 * (16 * NMB + 2);  // floats per parked wave
    static_assert((S - 1) * RBK * SLOT * 4 <= 8 * TILE, "combine space");
    const int rbk = wave % RBK;
    if (g > 0) {
      float* red = reinterpret_cast<float*>(smem) + ((g - 1) * RBK + rbk) * SLOT;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(mb * 16 + r) * 64 + lane] = oacc[mb][r];
      red[16 * NMB * 64 + lane] = m_run;
      red[(16 * NMB + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (g > 0) return false;
    float m = m_run;
#pragma unroll
    for (int gg = 1; gg < S; ++gg)
      m = fmaxf(m, reinterpret_cast<const float*>(smem)[((gg - 1) * RBK + rbk) * SLOT + 16 * NMB * 64 + lane]);
    const float a = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    l_run *= a;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mb][r] *= a;
#pragma unroll
    for (int gg = 1; gg < S; ++gg) {
      const float* red = reinterpret_cast<const float*>(smem) + ((gg - 1) * RBK + rbk) * SLOT;
      const float mg = red[16 * NMB * 64 + lane];
      const float b = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - m);
      l_run += b * red[(16 * NMB + 1) * 64 + lane];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mb][r] += b * red[(mb * 16 + r) * 64 + lane];
    }
    m_run = m;
    return true;
  };

  if (split) {
    const bool stores = p.split == 4 ? split_run(std::integral_constant<int, 4>{})
                                     : split_run(std::integral_constant<int, 2>{});
    if (!stores) return;
  } else if (!p.causal && !mask) {
    if (ntiles > 0) dense_run();
    l_run = wave_sum_halves(l_run);
  } else {
  if (ntiles > 0) {
    mbytes = kv.load(0);
    if (grp_b) {
      kld.issue(sK0, kbase, rsk, 0, nk);
      wait_tile_loads();
    }
    __syncthreads();
    if (grp_b) {  // phase 0 (group A: MFMAs of tile 0)
      if (1 < ntiles) kld.issue(sK1, kbase, rsk, BN, nk);
      vld.issue(sV0, vbase, rsk, 0, nk);
      __syncthreads();
    }
    // even j: K(j) in sK0, V(j) in sV0; odd j: sK1, sV1
    for (int j = 0; j <= ntiles; j += 2) {
      pair(j, sK0, sV1);
      if (j + 1 <= ntiles) pair(j + 1, sK1, sV0);
    }
    if (!grp_b) __syncthreads();
  }
  l_run = wave_sum_halves(l_run);
  }

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
                         dim3(512), args, 0, stream);
}

hipError_t launch_fwd(int D, bool varlen, const FwdParams& p, hipStream_t stream) {
  if (D == 64) return varlen ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return varlen ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
}

}  // namespace attn
