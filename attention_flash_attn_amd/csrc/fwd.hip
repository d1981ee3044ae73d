// fwd.hip -- attention forward for gfx950: out = softmax(scale * Q K^T) V and LSE.
//
// The forward op of the op pairs in diffusers PR #14341 (body): BSHD in, out in
// BSHD, log-sum-exp per query row (kept because the backward needs it, same
// PR, follow-up 1).  Keys excluded by the head-broadcast bool mask act as a
// -inf bias (same PR, follow-up 2; diffusers PR #14834, "Unsupported cases").
//
// Design (one workgroup = 8 waves = 256 query rows of one (batch|sequence, head), one
// workgroup per CU):
//  * Products on v_mfma_f32_16x16x32_bf16: under the package power limit this shape
//    delivers more FLOP/s than the 32x32x16 one on random operands (half the accumulator
//    traffic per multiply-add).  Each wave keeps its 32 query rows in registers as the B
//    operands (two 16-query blocks) of S^T = K Q^T, so every lane holds two queries, and
//    a query's scores are spread over four lanes (l, l^16, l^32, l^48); row statistics are
//    per-lane partials, combined across the four lanes only where needed.
//  * K/V tiles of 64 keys are double- or triple-buffered in LDS and filled
//    asynchronously by buffer loads into LDS.  Tiles are unpadded and XOR-swizzled
//    (tile.hpp) so the row reads of K and the transposing reads of V
//    are bank-conflict free.  The score registers of a lane (keys 4g..4g+3 and 16+4g..
//    16+4g+3 of each 32-key step, g = lane / 16) are directly the B operand of
//    O^T += V^T P^T; the transposing reads of V fetch the same key order.
//  * Ping-pong: the two 4-wave groups (one wave of each per SIMD) run half a tile
//    apart, so one group's MFMAs overlap the other group's softmax (see fwd_kernel).
//  * Online softmax in base 2 with scale*log2(e) folded into one FMA, against a lazily
//    moved reference: a tile's weights are formed against the row's current reference
//    max, and the reference (with O and l rescaled) only moves when some lane's partial
//    tile sum of a row exceeds 2^14, so every weight stays below 2^14 and the final
//    division uses the same reference, which gives the same softmax.
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
  constexpr int NKS = D / 32;  // 32-wide reduction steps of S^T = K Q^T
  constexpr int ND = D / 16;   // 16-row blocks of O^T
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
  // 16x16x32 operand roles: lane = 16 g + c holds column / row c of a block and reduction
  // slots 8g .. 8g+7; an output block gives it column c, rows 4g .. 4g+3.
  const int g = lane >> 4, c = lane & 15;

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
  const int q0w = qt * BM + (split ? part * (BM / p.split) : 0);  // first row of this workgroup
  if (q0w >= nq) return;  // block-uniform

  const long rs = (long)p.H * D, rsk = (long)p.Hk * D;
  const int kvh = head / p.G;
  const bf16* kbase = p.k + (long)krow0 * rsk + (long)kvh * D;
  const bf16* vbase = p.v + (long)krow0 * rsk + (long)kvh * D;

  // this wave's first query row (a split workgroup holds 8 / p.split row blocks of 32); the
  // lane's two queries are qw + c (block 0) and qw + 16 + c (block 1)
  const int qw = q0w + (split ? wave % (8 / p.split) : wave) * 32;
  bf16x8 qreg[2][NKS];  // [query block][step]: q[qw + 16 qb + c][32 ks + 8g .. +7]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bf16* qp = p.q + ((long)qrow0 + min(qw + 16 * qb + c, nq - 1)) * rs + (long)head * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[qb][ks] = as_bf16x8(ld16(qp + 32 * ks));
  }
  // K fragment of key block kb, step ks: tile row 16 kb + c, chunk 4 ks + g.  V^T fragment
  // of d block db in a 32-key step: keys 4g + e (low half) and 16 + 4g + e (high half),
  // e = 0..3, at d = 16 db + c (transposing reads; source lane 4e + t of a 16-lane group
  // addresses row 4g + e (+16), columns 16 db + 4t .. +3).
  int koff[NKS], voff[ND][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = tile_off<D>(c, 4 * ks + g);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      voff[db][h] = tile_off_tr<D>(16 * h + 4 * g + (c >> 2), 16 * db + 4 * (c & 3));

  TileLoader<D, BN, 4> kld, vld;  // the masked / causal loop: used by group B only
  auto same_row = [](int r) { return r; };
  kld.init(rsk, same_row, 4);
  vld.init(rsk, same_row, 4);

  f32x4 oacc[ND][2];  // O^T block (d 16 db + 4g + i, query 16 qb + c)
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db][0] = oacc[db][1] = f32x4{};
  f32x4 sacc[4][2];   // S^T block (key 16 kb + 4g + i, query 16 qb + c)
  bf16x8 pk[2][2];    // [32-key step][query block]: weights of keys 4g+i, 16+4g+i
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};  // per query; l: lane partial
  const float c2 = p.c2;
  const std::integral_constant<int, 2> kTwoHalves{};

  const int kend = p.causal ? min(nk, min(q0w + BM, nq)) : nk;
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
    constexpr int NKB = 2 * decltype(kbc)::value;  // 16-key blocks
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb][0] = sacc[kb][1] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 a = lds_row16(kt, kb * 16 * RB + koff[ks]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = mfma16(a, qreg[qb][ks], sacc[kb][qb]);
      }
    // one K fragment read per two MFMAs, issued AHEAD fragments early
    constexpr int AHEAD = 5, R = NKS * NKB;
    ATTN_SCHED(kSchedDSRead, AHEAD);
#pragma unroll
    for (int n = 0; n < R; ++n) {
      ATTN_SCHED(kSchedMFMA, 2);
      if (n + AHEAD < R) ATTN_SCHED(kSchedDSRead, 1);
    }
  };
  auto gemm_pv = [&](const char* vt, auto kbc) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value;  // 32-key steps
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 a = lds_tr8(vt + 32 * s * RB, voff[db][0], voff[db][1]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma16(a, pk[s][qb], oacc[db][qb]);
      }
    // two transposing reads per fragment, one fragment per two MFMAs
    constexpr int AHEAD = 3, F = KB * ND;
    ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
    for (int n = 0; n < F; ++n) {
      ATTN_SCHED(kSchedMFMA, 2);
      if (n + AHEAD < F) ATTN_SCHED(kSchedDSRead, 2);
    }
  };
  // O += P V of the previous tile, then S^T = K Q^T of this one, as one read pipeline: the
  // first K reads issue under the last P V MFMAs, so the matrix unit does not wait for
  // them between the two products.
  auto gemm_pv_s = [&](const char* vt, const char* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 a = lds_tr8(vt + 32 * s * RB, voff[db][0], voff[db][1]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma16(a, pk[s][qb], oacc[db][qb]);
      }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sacc[kb][0] = sacc[kb][1] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a = lds_row16(kt, kb * 16 * RB + koff[ks]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sacc[kb][qb] = mfma16(a, qreg[qb][ks], sacc[kb][qb]);
      }
    // fragments f < F read two transposed V halves, the others one K row fragment; each
    // feeds two MFMAs
    constexpr int AHEAD = 3, F = 2 * ND, N = F + 4 * NKS;
    ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      ATTN_SCHED(kSchedMFMA, 2);
      if (n + AHEAD < F) ATTN_SCHED(kSchedDSRead, 2);
      else if (n + AHEAD < N) ATTN_SCHED(kSchedDSRead, 1);
    }
  };
  // Sum / max of a query's four lanes (l, l^16, l^32, l^48).
  auto quad_sum = [](float x) __attribute__((always_inline)) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  };
  auto quad_max = [](float x) __attribute__((always_inline)) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
  };
  // later_c: a compile-time promise that the rows already have a reference (the dense loop
  // after its first tile), which drops the per-tile check for a first tile.
  const std::false_type kMayBeFirst{};
  auto softmax = [&](int k0, uint64_t vw, auto kbc, auto later_c) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value, NKB = 2 * KB;
    constexpr bool kLater = decltype(later_c)::value;
    constexpr uint64_t kFull = KB == 2 ? ~0ull : 0xFFFFFFFFull;  // bits of the tile's keys
    if ((vw & kFull) != kFull || (p.causal && k0 + 32 * KB - 1 > qw)) {
      keep_branch();
      // value i of block (kb, qb) is key k0 + 16 kb + 4g + i of query qw + 16 qb + c
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kr = 16 * kb + 4 * g + i;
            const bool on = ((vw >> kr) & 1u) && (!p.causal || k0 + kr <= qw + 16 * qb + c);
            sacc[kb][qb][i] = on ? sacc[kb][qb][i] : -INFINITY;
          }
    }
    // Weights against the rows' current references m_run, with no max over the tile: the
    // exponent arguments y = c2 s - m stay in sacc, and the tile is accepted unless some
    // lane's partial sum of a row exceeds 2^14 (or overflows), which keeps every weight
    // below 2^14.  The first tile of a row (no reference yet) and the rare rejected tile
    // form the tile max from y (over the row's four lanes), move the reference up by it,
    // rescale O and l, and recompute the weights.
    const bool first = kLater ? false : __ballot(m_run[0] == -INFINITY || m_run[1] == -INFINITY) != 0;
    float muse[2], lt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) muse[qb] = kLater ? m_run[qb] : (m_run[qb] == -INFINITY ? 0.f : m_run[qb]);
#pragma unroll
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 x;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float y = fmaf(sacc[2 * s + h][qb][i], c2, -muse[qb]);
            sacc[2 * s + h][qb][i] = y;
            x[4 * h + i] = __builtin_amdgcn_exp2f(y);
            // the weights are >= +0, so starting the sum from the first one is exact
            lt[qb] = (s == 0 && h == 0 && i == 0) ? x[0] : lt[qb] + x[4 * h + i];
          }
        pk[s][qb] = pack8(x, 0);
      }
    if (first || __ballot(!(lt[0] <= 0x1p14f) || !(lt[1] <= 0x1p14f))) {
      keep_branch();
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
        mx = quad_max(mx);
        const float mnew = fmaxf(m_run[qb], muse[qb] + mx);
        const float alpha = m_run[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - mnew);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db][qb] *= alpha;
        m_run[qb] = mnew;
        const float d = mnew == -INFINITY ? 0.f : mnew - muse[qb];
        lt[qb] = 0.f;
#pragma unroll
        for (int s = 0; s < KB; ++s) {
          f32x16 x;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[4 * h + i] = __builtin_amdgcn_exp2f(sacc[2 * s + h][qb][i] - d);
              lt[qb] += x[4 * h + i];
            }
          pk[s][qb] = pack8(x, 0);
        }
      }
    }
    l_run[0] += lt[0];
    l_run[1] += lt[1];
  };
  // MFMA phase of tile j: O += P(j-1) V(j-1), then S(j).  Group B then waits for the
  // copies it issued in its previous phase.
  auto gemm_phase = [&](int j, const char* __restrict__ kt, const char* __restrict__ vp)
      __attribute__((always_inline)) {
    // The group in its MFMA phase takes priority over the other wave of its SIMD (which runs
    // softmax): measured 0.5-1% faster than equal priorities on the masked and dense loops.
    __builtin_amdgcn_s_setprio(1);
    if (vw_s != 0) gemm_pv(vp, kTwoHalves);  // vw_s: still the word of tile j-1
    vw_s = tile_word(j, mbytes);
    mbytes = kv.load((j + 1) * BN);  // clamped: unused past the last tile
    if (vw_s != 0) gemm_s(kt, kTwoHalves);
    __builtin_amdgcn_s_setprio(0);
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
    if (vw_s != 0) softmax(j * BN, vw_s, kTwoHalves, kMayBeFirst);
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
  auto dense_run = [&]() __attribute__((always_inline)) {
    char* const dK0 = smem;
    char* const dK1 = smem + TILE;
    char* const dK2 = smem + 2 * TILE;
    char* const dV0 = smem + 3 * TILE;
    char* const dV1 = smem + 4 * TILE;
    char* const dV2 = smem + 5 * TILE;
    // One loader per wave: group A copies K, group B copies V.  (Choosing between two loader
    // objects per group would put them in scratch memory.)
    TileLoader<D, BN, 4> cld;
    cld.init(rsk, same_row, 4 * grp_b);
    const bf16* const cbase = grp_b ? vbase : kbase;
    const int lead = grp_b ? 1 : 2;  // group A copies K(j+2), group B V(j+1)
    // A phase barrier that does not wait for copies in flight (__syncthreads() would).  Only
    // register operations can move across it: the compiler may issue the last MFMAs of a
    // phase after it, whose operands were read before it from buffers that the next phase
    // does not overwrite (measured 0.4% faster than keeping them in front).
    auto bar = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };
    auto word = [&](int j) -> uint64_t __attribute__((always_inline)) { return kv.word(j * BN, 1u); };
    // VALU phase of tile j (kn: the buffer of K(j+2), vn: the buffer of V(j+1))
    // (after tile 0 every row has a finite reference: no mask, and tile 0 holds a valid key)
    auto vphase = [&](int j, char* __restrict__ kn, char* __restrict__ vn, auto later_c)
        __attribute__((always_inline)) {
      if (j + lead < ntiles) cld.issue(grp_b ? vn : kn, cbase, rsk, (j + lead) * BN, nk);
      softmax(j * BN, vw_s, kTwoHalves, later_c);
    };
    // pair of phases of tile j, 0 < j < ntiles (kt: K(j), vp: V(j-1))
    auto dpair = [&](int j, const char* __restrict__ kt, const char* __restrict__ vp,
                     char* __restrict__ kn, char* __restrict__ vn) __attribute__((always_inline)) {
      __builtin_amdgcn_s_setprio(1);  // MFMA phase first (as in gemm_phase)
      gemm_pv_s(vp, kt);
      __builtin_amdgcn_s_setprio(0);
      vw_s = word(j);
      wait_tile_loads();
      bar();
      vphase(j, kn, vn, std::true_type{});
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
    vphase(0, dK2, dV1, kMayBeFirst);
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
    const int grp = wave / RBK;
    const int nts = (kend + BNS - 1) / BNS;
    const int hn = (nts + S - 1) / S, t0 = grp * hn, t1 = min(nts, t0 + hn);
    char* const gb = smem + 4 * TS * grp;
    TileLoader<D, BNS, RBK> gk, gv;
    gk.init(rsk, same_row, RBK * grp);
    gv.init(rsk, same_row, RBK * grp);
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
        softmax(j * BNS, vw, kb_c, kMayBeFirst);
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
    // and stores.  l stays a per-lane partial here (the same lanes of every group hold the
    // same queries); it is summed over a query's four lanes afterwards.
    constexpr int NO = ND * 8;               // O values per lane
    constexpr int SLOT = 64 * (NO + 4);      // floats per parked wave
    static_assert((S - 1) * RBK * SLOT * 4 <= 8 * TILE, "combine space");
    const int rbk = wave % RBK;
    if (grp > 0) {
      float* red = reinterpret_cast<float*>(smem) + ((grp - 1) * RBK + rbk) * SLOT;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((db * 2 + qb) * 4 + i) * 64 + lane] = oacc[db][qb][i];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        red[(NO + qb) * 64 + lane] = m_run[qb];
        red[(NO + 2 + qb) * 64 + lane] = l_run[qb];
      }
    }
    __syncthreads();
    if (grp > 0) return false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = m_run[qb];
#pragma unroll
      for (int gg = 1; gg < S; ++gg)
        m = fmaxf(m, reinterpret_cast<const float*>(smem)[((gg - 1) * RBK + rbk) * SLOT + (NO + qb) * 64 + lane]);
      const float a = m_run[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - m);
      l_run[qb] *= a;
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db][qb] *= a;
#pragma unroll
      for (int gg = 1; gg < S; ++gg) {
        const float* red = reinterpret_cast<const float*>(smem) + ((gg - 1) * RBK + rbk) * SLOT;
        const float mg = red[(NO + qb) * 64 + lane];
        const float b = mg == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mg - m);
        l_run[qb] += b * red[(NO + 2 + qb) * 64 + lane];
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[db][qb][i] += b * red[((db * 2 + qb) * 4 + i) * 64 + lane];
      }
      m_run[qb] = m;
    }
    return true;
  };

  if (split) {
    const bool stores = p.split == 4 ? split_run(std::integral_constant<int, 4>{})
                                     : split_run(std::integral_constant<int, 2>{});
    if (!stores) return;
  } else if (!p.causal && !mask) {
    if (ntiles > 0) dense_run();
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
  }

  // l over each query's four lanes; lane (c, g) stores d = 16 db + 4g .. +3 of its two rows
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = quad_sum(l_run[qb]);
    const int qrow = qw + 16 * qb + c;
    if (qrow < nq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16* op = p.out + ((long)qrow0 + qrow) * rs + (long)head * D + 4 * g;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[db][qb][e] * inv);
        *reinterpret_cast<bf16x4*>(op + 16 * db) = o;
      }
      if (g == 0)
        p.lse[lse_base + qrow] = l > 0.f ? (m_run[qb] + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
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
