// bwd.hip -- attention backward for gfx950: delta preprocess, dK/dV kernel, dQ kernel.
//
// The backward op of the op pairs in diffusers PR #14341 (body): grad_out in
// BSHD, Q/K/V read in the layout the forward received them (the double
// transpose of K/V was the bug fixed there), dQ/dK/dV out in BSHD.  P is
// rebuilt from the forward's LSE (the reason the forward must always produce
// it: same PR, follow-up 1); LSE itself receives no gradient (diffusers PR
// #14834, summary).
//
//   delta_i = <dO_i, out_i>                    (preprocess, from the bf16 out)
//   P_ij = exp(scale s_ij - LSE_i), dP_ij = <dO_i, v_j>, dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
//
// dK/dV and dQ come from two kernels that each own their output rows, so
// there are no atomics and the result is bitwise reproducible.
//
// Both workgroup kinds run their products on v_mfma_f32_16x16x32_bf16, which delivers
// more FLOP/s than the 32x32x16 shape under the package power limit (half the accumulator
// traffic per multiply-add); every LDS fragment read feeds two or four MFMAs, so the LDS
// bytes per FLOP are those of the 32x32x16 layout.
//
// dK/dV workgroup: 8 waves, 256 keys.  The keys' K rows go to registers and their V rows
// sit in LDS for the whole loop; query tiles of 64 rows (Q, dO, LSE, delta) are
// double-buffered in LDS, filled asynchronously by buffer loads into XOR-swizzled LDS
// rows (tile.hpp; natural row order).  Wave w owns keys 32w .. 32w+31
// (two 16-key blocks: two keys per lane, the columns of the score blocks S = Q K^T) and
// both 32-row halves of every tile, with its dK^T, dV^T accumulators in registers across
// the loop.  Q^T and dO^T operands come from the LDS transposing read, in the row order of
// the lane's P and dS values.
//
// dQ workgroup: 8 waves, 256 query rows; each wave keeps its 32 rows of Q and dO (B
// operands of S^T = K Q^T and dP^T = V dO^T in two 16-query blocks: two queries per lane,
// so LSE and delta are per-lane scalars) and its dQ^T accumulator in registers; K/V tiles
// of 64 keys are double-buffered in LDS the same way; K^T comes from the transposing read,
// in the key order of the lane's dS values.
//
// Eight waves, two per SIMD, keep each wave within 256 registers, so that one wave's
// matrix instructions run while the other does its exponentials and conversions (a wave
// does not overlap the two itself).
//
// Both run in ONE launch: every workgroup of the longer kind first, in plain block order
// (dealt round-robin to the XCDs, so each XCD gets its share of both kinds), and in dense
// non-causal launches the last dQ tiles as split workgroups of half the rows, so that the
// launch's last round ends together (bwd_kernel).
//
// Partial tiles (a ragged tail, a mask edge) zero the excluded weights in a
// branch taken only there, so full tiles carry no per-element mask work.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace attn {

// ------------------------------------------------------------------ delta

template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const bf16* __restrict__ out,
                                                    const bf16* __restrict__ dout,
                                                    float* __restrict__ delta, long rows, int S,
                                                    int H) {
  constexpr int CPR = D / 8;      // lanes per row (16 bytes each)
  constexpr int RPB = 256 / CPR;  // rows per workgroup
  const long row = (long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int c = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = as_bf16x8(ld16(out + row * D + 8 * c));
    const bf16x8 b = as_bf16x8(ld16(dout + row * D + 8 * c));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) {
    const long h = row % H, bs = row / H;
    const long s = bs % S, b = bs / S;
    delta[(b * H + h) * S + s] = acc;
  }
}

hipError_t launch_delta(int D, long rows, int S, int H, const bf16* out, const bf16* dout,
                        float* delta, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (D / 8);
  const long nb = (rows + rpb - 1) / rpb;
  void* args[] = {&out, &dout, &delta, &rows, &S, &H};
  const void* fn = D == 64 ? reinterpret_cast<const void*>(&delta_kernel<64>)
                           : reinterpret_cast<const void*>(&delta_kernel<128>);
  return hipLaunchKernel(fn, dim3((unsigned)nb), dim3(256), args, 0, stream);
}

// Shared decode of one workgroup: its tile, (outer, key/value head) group, query head
// (query head i of the group: kvhead * G + i) and row ranges.  The LSE / delta rows of
// query head h + 1 follow those of head h at a distance of p.Sq in both layouts.
struct Slice {
  int tile, qhead, kvhead, qrow0, krow0, nq, nk;
  long lse_base;  // of qhead
  const uint8_t* mask;
};

template <bool VARLEN>
__device__ __forceinline__ Slice decode(const BwdParams& p, int group, int tile, int i) {
  Slice s;
  s.tile = tile;
  // group = key/value head * B + outer (batch entry), or for varlen sequence rank * Hk +
  // key/value head, the longest sequence's groups first (see SeqOrder)
  s.kvhead = VARLEN ? group % p.Hk : group / p.B;
  s.qhead = s.kvhead * p.G + i;
  const int outer = VARLEN ? p.order(group / p.Hk) : group % p.B;
  s.mask = nullptr;
  if (VARLEN) {
    const int s0 = p.cu[outer], s1 = p.cu[outer + 1];
    s.qrow0 = s.krow0 = s0;
    s.nq = s.nk = s1 - s0;
    s.lse_base = (long)s.qhead * p.Sq + s0;
  } else {
    s.qrow0 = outer * p.Sq;
    s.krow0 = outer * p.Sk;
    s.nq = p.Sq;
    s.nk = p.Sk;
    s.lse_base = ((long)outer * p.H + s.qhead) * p.Sq;
    if (p.mask) s.mask = p.mask + (long)outer * p.Sk;
  }
  return s;
}

// ------------------------------------------------------------------ dK / dV

template <int D>
struct DkdvSmem {
  static constexpr int BN = 256;  // keys per workgroup: 8 blocks of 32, one per wave
  static constexpr int BQ = 64;   // query rows per staged tile: 2 sub-tiles of 32
  // The Q/dO tiles come first: LDS reads address at most 64 KB past a register, so with
  // all four of them in the first 64 KB one set of per-lane offsets serves every buffer.
  // Before the loop the same 64 KB stage the workgroup's K rows on their way to registers.
  char q[2][BQ * 2 * D];          // double-buffered Q and dO tiles
  char o[2][BQ * 2 * D];
  char v[BN * 2 * D];             // V of the workgroup's keys, loaded once
  float l[2][BQ];                 // LSE * log2(e) and delta of the tile's rows
  float d[2][BQ];
};

template <int D>
struct DqSmem {
  static constexpr int BN = 64;  // keys per staged tile
  char k[2][BN * 2 * D];
  char v[2][BN * 2 * D];
};

// dK/dV: 8 waves, 256 keys.  Wave w owns keys 32w .. 32w+31 and both 32-row halves of
// every 64-row query tile, so each staged tile feeds 128 MFMAs per wave and no two waves
// share a key.  The wave's K fragments (the B operands of S = Q K^T, 32 registers) are read
// from LDS once and kept in registers for the whole loop; V stays in LDS, which keeps a
// wave within 256 registers: two waves per SIMD, so one wave's MFMAs run while the other
// does its softmax VALU work.
template <int D, bool VARLEN, bool ACC>
__device__ __forceinline__ void dkdv_block(const BwdParams& p, const Slice sl, DkdvSmem<D>& sm) {
  constexpr int BN = DkdvSmem<D>::BN, BQ = DkdvSmem<D>::BQ, NW = 8;
  constexpr int RB = 2 * D;
  constexpr int NKS = D / 32, ND = D / 16;
  static_assert(sizeof(sm.q) + sizeof(sm.o) == BN * RB && offsetof(DkdvSmem<D>, q) == 0,
                "the Q/dO buffers stage K");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  // 16x16x32 operand roles: lane = 16 g + c holds column / row c of a block and reduction
  // slots 8g .. 8g+7; an output block gives it column c, rows 4g .. 4g+3.
  const int g = lane >> 4, c = lane & 15;
  const int kb0 = sl.tile * BN;
  if (kb0 >= sl.nk) return;  // block-uniform
  // Q/dO rows hold H heads, K/V/dK/dV rows Hk.  The loop runs over the query tiles of all
  // G query heads that read this key/value head (query head qhead + i for i < G), so dK
  // and dV sum their contributions (grouped-query attention) without atomics.
  const long rs = (long)p.H * D, rsk = (long)p.Hk * D;
  const int nq = sl.nq, nk = sl.nk;

  // The wave's 32 keys in two 16-key blocks; the lane's keys are kw + c and kw + 16 + c.
  const int kw = kb0 + 32 * wave;
  bool kvalid[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + 16 * kb + c;
    kvalid[kb] = key < nk && (!sl.mask || sl.mask[key] != 0);
  }
  const uint64_t kball = __ballot(kvalid[0] || kvalid[1]);
  if (!__syncthreads_or(kvalid[0] || kvalid[1])) {
    // Every key of the workgroup is masked: dK = dV = 0 without the query loop (added to
    // nothing when accumulating).
    if (!(ACC && (p.acc_flags & 2))) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kw + 16 * kb + c;
        if (key >= nk) continue;
        const long off = ((long)sl.krow0 + key) * rsk + (long)sl.kvhead * D + 4 * g;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const long o = off + 16 * db;
          if (ACC) {
            *reinterpret_cast<f32x4*>(p.dk_acc + o) = f32x4{};
            *reinterpret_cast<f32x4*>(p.dv_acc + o) = f32x4{};
          } else {
            *reinterpret_cast<bf16x4*>(p.dk + o) = to_bf16x4(f32x4{});
            *reinterpret_cast<bf16x4*>(p.dv + o) = to_bf16x4(f32x4{});
          }
        }
      }
    }
    return;
  }

  // LDS offsets.  Q/dO/K/V fragment of 16-row block rb, step ks: row 16 rb + c, chunk
  // 4 ks + g; Q^T/dO^T fragment of d block db in a 32-row step: rows 4g + e and 16 + 4g + e
  // at d = 16 db + c (transposing reads).  Steps differ only in chunk bits, offset(ks) =
  // offset(0) ^ 64 ks and offset(db) = offset(0) ^ 32 db (tile.hpp swizzle); they are
  // rebuilt before every use from the step-0 offsets (3 registers held through the loop).
  int qoff0 = tile_off<D>(c, g), tr0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) tr0[h] = tile_off_tr<D>(16 * h + 4 * g + (c >> 2), 4 * (c & 3));
  int qoff[NKS], troff[ND][2];
  auto offsets = [&]() {
    // D = 128: not hoisted out of the loop (registers); D = 64 has room to keep them all
    if constexpr (D == 128) asm volatile("" : "+v"(qoff0), "+v"(tr0[0]), "+v"(tr0[1]));
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qoff[ks] = qoff0 ^ (64 * ks);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      troff[db][0] = tr0[0] ^ (32 * db);
      troff[db][1] = tr0[1] ^ (32 * db);
    }
  };

  auto same_row = [](int r) { return r; };
  const bf16* kbase = p.k + (long)sl.krow0 * rsk + (long)sl.kvhead * D;
  const bf16* vbase = p.v + (long)sl.krow0 * rsk + (long)sl.kvhead * D;
  const bf16* qbase = p.q + (long)sl.qrow0 * rs + (long)sl.qhead * D;
  const bf16* obase = p.dout + (long)sl.qrow0 * rs + (long)sl.qhead * D;
  char* kstage = reinterpret_cast<char*>(&sm);
  {
    TileLoader<D, BN, NW> kvld;
    kvld.init(rsk, same_row);
    kvld.issue(kstage, kbase, rsk, kb0, nk);
    kvld.issue(sm.v, vbase, rsk, kb0, nk);
  }
  TileLoader<D, BQ, 4> ld;  // used by waves 0..3
  ld.init(rs, same_row);
  // LSE and delta of the next tile are loaded raw (row clamped, no arithmetic) ahead of
  // its asynchronous copy and only used when published after the current tile's
  // compute: a use right after the load would make the wave wait for the whole copy.
  float lraw = 0.f, draw = 0.f;
  // Query tiles per query head: all of them, or (causal) those from the first one holding
  // a row that sees key kb0.
  const int ntq_all = (nq + BQ - 1) / BQ;
  const int qt0 = p.causal ? min(kb0 / BQ, ntq_all) : 0;
  const int ntq = ntq_all - qt0;
  // Tile t of the loop: query head qhead + t / ntq, rows (qt0 + t % ntq) * BQ ...
  auto tile_q0 = [&](int t) { return (qt0 + t - (t / ntq) * ntq) * BQ; };
  auto issue = [&](int t, char* qt, char* ot) {
    const int i = t / ntq, q0 = tile_q0(t);
    // Only wave 0 publishes the statistics, so only it loads them: any load issued behind
    // the copies waits in the same queue.
    if (wave == 0) {
      const long qi = sl.lse_base + (long)i * p.Sq + min(q0 + lane, nq - 1);
      lraw = p.lse[qi];
      draw = p.delta[qi];
    }
    // Only waves 0..3 copy: right after the barrier the copies queue up in the memory
    // pipeline and stall the waves that issue them (32 KB at ~64 B/clock), and meanwhile
    // the other wave of each SIMD has its matrix unit to itself.
    if (wave < 4) {
      ld.issue(qt, qbase + (long)i * D, rs, q0, nq);
      ld.issue(ot, obase + (long)i * D, rs, q0, nq);
    }
  };
  // Published per row: -LSE/scale and -delta, the starting values of the S and dP
  // accumulators (rows past the end, and rows with no key to attend to, get -inf, so
  // their P is 0).
  const float nis = -1.f / p.scale;
  auto publish_stats = [&](int t, float* lt, float* dt) {
    const int q0 = tile_q0(t);
    if (tid < BQ) {
      const bool in = q0 + tid < nq && lraw != -INFINITY;
      lt[tid] = in ? lraw * nis : -INFINITY;
      dt[tid] = in ? -draw : 0.f;
    }
  };

  f32x4 dkacc[ND][2], dvacc[ND][2];  // dK^T / dV^T block (d 16 db + 4g + i, key 16 kb + c)
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dkacc[db][kb] = dvacc[db][kb] = f32x4{};
  const float c2 = p.c2;
  const int kr = wave * 32 * RB;
  bf16x8 kreg[2][NKS];  // the wave's keys as the B operand of S = Q K^T: key 16 kb + c, d 32 ks + 8g ..

  // dP = dO V^T of the whole 64-row tile (query block qb = 0..3, key block kb), so that
  // each V fragment read feeds four MFMAs.  The accumulators start from their rows' -delta.
  auto scores_dp = [&](const char* vt, const char* ot, const float* dt, f32x4 (&dp)[4][2]) {
    offsets();
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) dp[qb][0] = dp[qb][1] = *reinterpret_cast<const f32x4*>(dt + 16 * qb + 4 * g);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {  // each V and dO fragment read once per step
      bf16x8 vf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) vf[kb] = lds_row16(vt, kr + 16 * kb * RB + qoff[ks]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const bf16x8 a = lds_row16(ot, 16 * qb * RB + qoff[ks]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dp[qb][kb] = mfma16(a, vf[kb], dp[qb][kb]);
      }
    }
  };
  // One 32x32 (query x key) step on half u of the tile (query blocks 2u, 2u + 1), given its
  // dP: scores S = Q K^T, weights P = exp(scale S - LSE) and dS = P (dP - delta), then
  // dV^T += dO^T P and dK^T += Q^T dS.  The S and dP accumulators start from their rows'
  // -LSE/scale and -delta, so P = exp2(c2 acc) and dS = P acc with no per-row operands in
  // registers.  No key-mask work here: P and dS of an excluded key only reach that key's
  // own accumulators (keys are output columns), which are stored as zeros.  Causal blocks
  // that hold a key after one of their rows zero P per element in a branch taken only there.
  auto compute = [&](const char* qt, const char* ot, const float* lt, int q0, int u, f32x4 (&dp)[4][2]) {
    const int qr = u * 32 * RB;
    offsets();
    // s[b][kb]: query 32u + 16b + 4g + i of the tile, key 16 kb + c of the wave
    f32x4 s[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) s[b][0] = s[b][1] = *reinterpret_cast<const f32x4*>(lt + 32 * u + 16 * b + 4 * g);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 a = lds_row16(qt, qr + 16 * b * RB + qoff[ks]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[b][kb] = mfma16(a, kreg[kb][ks], s[b][kb]);
      }
    {
      // one Q fragment read per two MFMAs, issued AHEAD fragments early (measured: 1.6% on
      // the backward together with the read-ahead below; more or less ahead was slower)
      constexpr int AHEAD = 4, R = 2 * NKS;
      ATTN_SCHED(kSchedDSRead, AHEAD);
#pragma unroll
      for (int n = 0; n < R; ++n) {
        ATTN_SCHED(kSchedMFMA, 2);
        if (n + AHEAD < R) ATTN_SCHED(kSchedDSRead, 1);
      }
    }
    if (p.causal && q0 + 32 * u < kw + 31) {
      keep_branch();
      // P = 0 where the lane's key comes after the value's row.
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[b][kb][i] = kw + 16 * kb + c <= q0 + 32 * u + 16 * b + 4 * g + i ? s[b][kb][i] : -INFINITY;
    }
    // pk[kb], ds[kb]: the B operands of the dV^T / dK^T steps (rows 4g + i of block 2u,
    // then of block 2u + 1)
    bf16x8 pk[2], ds[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 x, y;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = __builtin_amdgcn_exp2f(s[b][kb][i] * c2);
          x[4 * b + i] = pw;
          y[4 * b + i] = pw * dp[2 * u + b][kb][i];
        }
      pk[kb] = pack8(x, 0);
      ds[kb] = pack8(y, 0);
    }
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const bf16x8 ao = lds_tr8(ot + qr, troff[db][0], troff[db][1]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dvacc[db][kb] = mfma16(ao, pk[kb], dvacc[db][kb]);
      const bf16x8 aq = lds_tr8(qt + qr, troff[db][0], troff[db][1]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dkacc[db][kb] = mfma16(aq, ds[kb], dkacc[db][kb]);
    }
    {
      constexpr int AHEAD = 3, F = 2 * ND;  // fragments of two transposing reads, two MFMAs each
      ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
      for (int n = 0; n < F; ++n) {
        ATTN_SCHED(kSchedMFMA, 2);
        if (n + AHEAD < F) ATTN_SCHED(kSchedDSRead, 2);
      }
    }
  };

  const int ntiles = p.G * ntq;
  // All tile buffers are distinct __restrict__ parameters, so once inlined the compiler
  // can tell reads of the current tile from the asynchronous copy into the next one
  // (without that it waits for the copy before the first LDS read).
  auto step = [&](int j, const char* __restrict__ vt, const char* __restrict__ cq,
                  const char* __restrict__ co, const float* __restrict__ cl,
                  const float* __restrict__ cd, char* __restrict__ nq_, char* __restrict__ no_,
                  float* __restrict__ nl, float* __restrict__ nd) {
    const bool more = j + 1 < ntiles;
    if (more) issue(j + 1, nq_, no_);
    if (kball != 0) {
      const int q0 = tile_q0(j);
      f32x4 dp[4][2];
      scores_dp(vt, co, cd, dp);
      compute(cq, co, cl, q0, 0, dp);
      // The two waves of a SIMD do the same work, but waves 0..3 start late (copy issue)
      // and then win every tie (older waves issue first), so they finish early and wait at
      // the barrier while their partner runs alone.  Waves 4..7 take priority for their
      // second half, so both finish about together.
      if (wave >= 4) __builtin_amdgcn_s_setprio(1);
      compute(cq, co, cl, q0, 1, dp);
      if (wave >= 4) __builtin_amdgcn_s_setprio(0);
    }
    if (more) publish_stats(j + 1, nl, nd);
    wait_tile_loads();
    __syncthreads();
  };
  // K: staged, read into registers, then its staging space is handed to the Q/dO tiles
  // (the LDS reads must have returned before the barrier lets the copies in).
  wait_tile_loads();
  __syncthreads();
  offsets();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kreg[kb][ks] = lds_row16(kstage, kr + 16 * kb * RB + qoff[ks]);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();
  if (ntiles > 0) {
    issue(0, sm.q[0], sm.o[0]);
    publish_stats(0, sm.l[0], sm.d[0]);
  }
  wait_tile_loads();
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    step(j, sm.v, sm.q[0], sm.o[0], sm.l[0], sm.d[0], sm.q[1], sm.o[1], sm.l[1], sm.d[1]);
    if (j + 1 < ntiles)
      step(j + 1, sm.v, sm.q[1], sm.o[1], sm.l[1], sm.d[1], sm.q[0], sm.o[0], sm.l[0], sm.d[0]);
  }

  // lane (c, g) stores d = 16 db + 4g .. +3 of its two keys
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kw + 16 * kb + c;
    if (key >= nk) continue;
    const long off = ((long)sl.krow0 + key) * rsk + (long)sl.kvhead * D + 4 * g;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      f32x4 a = kvalid[kb] ? dkacc[db][kb] * p.scale : f32x4{};
      f32x4 b = kvalid[kb] ? dvacc[db][kb] : f32x4{};
      const long o = off + 16 * db;
      if (ACC) {
        f32x4* ka = reinterpret_cast<f32x4*>(p.dk_acc + o);
        f32x4* va = reinterpret_cast<f32x4*>(p.dv_acc + o);
        if (p.acc_flags & 2) {
          a += *ka;
          b += *va;
        }
        *ka = a;
        *va = b;
      } else {
        *reinterpret_cast<bf16x4*>(p.dk + o) = to_bf16x4(a);
        *reinterpret_cast<bf16x4*>(p.dv + o) = to_bf16x4(b);
      }
    }
  }
}

// ------------------------------------------------------------------ dQ

// half < 0: a whole workgroup, 256 query rows.  half = 0 or 1: a split workgroup, the
// 128-row half `half` of the tile, whose wave groups (waves 0..3 and 4..7, the same 128
// rows) each take one half of the key tiles with their own double-buffered K/V tiles in
// sm[group], and whose partial dQ sums are added through LDS at the end.  Split
// workgroups finish a launch's last round in half the time (dense non-causal grids only).
template <int D, bool VARLEN, bool ACC>
__device__ __forceinline__ void dq_block(const BwdParams& p, const Slice sl, DqSmem<D> (&sm)[2],
                                         int half) {
  constexpr int BM = 256, BN = DqSmem<D>::BN;
  constexpr int RB = 2 * D;
  constexpr int NKS = D / 32, ND = D / 16;
  constexpr int GB = sizeof(DqSmem<D>);  // LDS distance between the wave groups' tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  // 16x16x32 operand roles: lane = 16 g + c holds column / row c of a block and reduction
  // slots 8g .. 8g+7; an output block gives it column c, rows 4g .. 4g+3.
  const int g = lane >> 4, c = lane & 15;
  const bool split = half >= 0;
  const int grp = split ? wave >> 2 : 0;
  // Causal: the last query tiles see the most keys, so they are dealt out first.
  const int qb0 = (p.causal ? p.n_q_tiles - 1 - sl.tile : sl.tile) * BM + (split ? half * (BM / 2) : 0);
  if (qb0 >= sl.nq) return;  // block-uniform
  // Q/dO/dQ rows hold H heads, K/V rows Hk (this query head reads key/value head kvhead).
  const long rs = (long)p.H * D, rsk = (long)p.Hk * D;
  const int nq = sl.nq, nk = sl.nk;

  // The wave's 32 rows; the lane's two queries are qw + c (block 0) and qw + 16 + c (block 1).
  const int qw = qb0 + (split ? wave & 3 : wave) * 32;
  bf16x8 qreg[2][NKS], doreg[2][NKS];  // [query block][step]: row qw + 16 qb + c, d 32 ks + 8g ..
  float lse2[2], ndl[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw + 16 * qb + c;
    const long off = ((long)sl.qrow0 + min(qrow, nq - 1)) * rs + (long)sl.qhead * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qreg[qb][ks] = as_bf16x8(ld16(p.q + off + 32 * ks));
      doreg[qb][ks] = as_bf16x8(ld16(p.dout + off + 32 * ks));
    }
    // Rows past the end, and rows with no key to attend to (LSE = -inf: every visible key
    // masked), take +inf so that P = exp2(c2 S - lse2) is 0 even where S is -inf.
    const float lse_row = qrow < nq ? p.lse[sl.lse_base + qrow] : -INFINITY;
    lse2[qb] = lse_row == -INFINITY ? INFINITY : lse_row * kLog2e;
    ndl[qb] = qrow < nq ? -p.delta[sl.lse_base + qrow] : 0.f;
  }
  // The dP^T accumulators start from the row's -delta (their C operand).
  f32x4 ndl4[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) ndl4[qb] = f32x4{ndl[qb], ndl[qb], ndl[qb], ndl[qb]};

  // LDS offsets.  K/V fragment of key block kb, step ks: tile row 16 kb + c, chunk 4 ks + g;
  // K^T fragment of d block db in a 32-key step: keys 4g + e and 16 + 4g + e at d = 16 db + c
  // (transposing reads).  Steps differ only in chunk bits, offset(ks) = offset(0) ^ 64 ks and
  // offset(db) = offset(0) ^ 32 db (tile.hpp swizzle), so they are rebuilt at every step from
  // the step-0 offsets (3 registers held through the loop).  The offsets also carry the wave
  // group's distance to its own tiles (GB, a multiple of 256 bytes, which the XORs leave
  // alone), so the tile addresses stay constants.
  int koff0 = tile_off<D>(c, g) + grp * GB, tr0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) tr0[h] = tile_off_tr<D>(16 * h + 4 * g + (c >> 2), 4 * (c & 3)) + grp * GB;
  int koff[NKS], troff[ND][2];
  auto offsets = [&]() {
    // D = 128: not hoisted out of the loop (registers); D = 64 has room to keep them all
    if constexpr (D == 128) asm volatile("" : "+v"(koff0), "+v"(tr0[0]), "+v"(tr0[1]));
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) koff[ks] = koff0 ^ (64 * ks);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      troff[db][0] = tr0[0] ^ (32 * db);
      troff[db][1] = tr0[1] ^ (32 * db);
    }
  };

  const bf16* kbase = p.k + (long)sl.krow0 * rsk + (long)sl.kvhead * D;
  const bf16* vbase = p.v + (long)sl.krow0 * rsk + (long)sl.kvhead * D;
  auto same_row = [](int r) { return r; };
  TileLoader<D, BN, 4> ld;  // used by waves 0..3 (split: each group's four waves)
  ld.init(rsk, same_row, 4 * grp);
  // Only waves 0..3 copy (see dkdv_block): while they stall at issue, waves 4..7, one per
  // SIMD, keep the matrix units busy.  In a split workgroup each group copies its own tiles.
  auto issue = [&](int k0, char* kt, char* vt) {
    if (split || wave < 4) {
      ld.issue(kt + grp * GB, kbase, rsk, k0, nk);
      ld.issue(vt + grp * GB, vbase, rsk, k0, nk);
    }
  };

  f32x4 dqacc[ND][2];  // dQ^T block (d 16 db + 4g + i, query 16 qb + c)
#pragma unroll
  for (int db = 0; db < ND; ++db) dqacc[db][0] = dqacc[db][1] = f32x4{};
  const float c2 = p.c2;

  // Per 32-key half h of a tile: scores A (S^T, dP^T MFMAs over key blocks 2h, 2h+1),
  // weights B (VALU: P, dS), gradient C (dQ^T MFMAs), issued as A0 | A1 B0 | C0 B1 | C1 with
  // hard scheduling boundaries.  Partial tiles mask the scores (to -inf) between the groups.
  // st[b][qb], dpt[b][qb]: key block 2h + b, query block qb.
  auto scores = [&](const char* kt, const char* vt, int h, f32x4 (&st)[2][2], f32x4 (&dpt)[2][2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      st[b][0] = st[b][1] = f32x4{};
      dpt[b][0] = ndl4[0];
      dpt[b][1] = ndl4[1];
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 a = lds_row16(kt, (2 * h + b) * 16 * RB + koff[ks]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) st[b][qb] = mfma16(a, qreg[qb][ks], st[b][qb]);
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 a = lds_row16(vt, (2 * h + b) * 16 * RB + koff[ks]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) dpt[b][qb] = mfma16(a, doreg[qb][ks], dpt[b][qb]);
      }
    // one K or V fragment read per two MFMAs, issued AHEAD fragments early (measured on
    // the 27280-token shard: 2 ahead 0.6-2% faster than the compiler's own order, 1 ahead
    // 7% slower, 3 to 6 ahead 0.3% slower)
    constexpr int AHEAD = 2, R = 4 * NKS;
    ATTN_SCHED(kSchedDSRead, AHEAD);
#pragma unroll
    for (int n = 0; n < R; ++n) {
      ATTN_SCHED(kSchedMFMA, 2);
      if (n + AHEAD < R) ATTN_SCHED(kSchedDSRead, 1);
    }
  };
  auto mask_scores = [&](uint64_t vw, int k0, int h, f32x4 (&st)[2][2]) {
    // value i of block (b, qb) is key k0 + 32h + 16b + 4g + i of query qw + 16 qb + c;
    // causal: visible only up to the query's row
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = 32 * h + 16 * b + 4 * g + i;
          const bool on = ((vw >> kr) & 1u) && (!p.causal || k0 + kr <= qw + 16 * qb + c);
          st[b][qb][i] = on ? st[b][qb][i] : -INFINITY;
        }
  };
  // Tiles that need per-element masking: not every key valid, or (causal) some key of the
  // tile after some query row of the workgroup.
  auto needs_mask = [&](int k0, uint64_t vw) { return vw != ~0ull || (p.causal && k0 + BN - 1 > qb0); };
  // P = exp2(c2 S - lse2), dS = P (dP - delta); ds[qb]: the B operand of the dQ^T step (keys
  // 4g + i of block 2h, then of block 2h + 1)
  auto weights = [&](f32x4 (&st)[2][2], f32x4 (&dpt)[2][2], bf16x8 (&ds)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 x;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pw = __builtin_amdgcn_exp2f(fmaf(st[b][qb][i], c2, -lse2[qb]));
          x[4 * b + i] = pw * dpt[b][qb][i];
        }
      ds[qb] = pack8(x, 0);
    }
  };
  auto grad = [&](const char* kt, int h, const bf16x8 (&ds)[2]) {
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const bf16x8 a = lds_tr8(kt + 32 * h * RB, troff[db][0], troff[db][1]);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) dqacc[db][qb] = mfma16(a, ds[qb], dqacc[db][qb]);
    }
    // fragments of two transposing reads, two MFMAs each, issued AHEAD fragments early
    // (2 or 3 ahead: 0.7% faster than the compiler's own order; 4: 0.3%)
    constexpr int AHEAD = 3, F = ND;
    ATTN_SCHED(kSchedDSRead, 2 * AHEAD);
#pragma unroll
    for (int n = 0; n < F; ++n) {
      ATTN_SCHED(kSchedMFMA, 2);
      if (n + AHEAD < F) ATTN_SCHED(kSchedDSRead, 2);
    }
  };
  auto compute = [&](const char* kt, const char* vt, int k0, uint64_t vw) {
    offsets();
    f32x4 st0[2][2], dpt0[2][2], st1[2][2], dpt1[2][2];
    bf16x8 ds0[2], ds1[2];
    scores(kt, vt, 0, st0, dpt0);
    const bool masked = needs_mask(k0, vw);
    if (masked) {
      keep_branch();
      mask_scores(vw, k0, 0, st0);
    }
    __builtin_amdgcn_sched_barrier(0);
    scores(kt, vt, 1, st1, dpt1);
    weights(st0, dpt0, ds0);
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
      keep_branch();
      mask_scores(vw, k0, 1, st1);
    }
    // Waves 4..7 take priority from here to the step's end (see dkdv_block: waves 0..3
    // start late and win ties).  Split workgroups, where every wave copies, keep equal ones.
    if (!split && wave >= 4) __builtin_amdgcn_s_setprio(1);
    grad(kt, 0, ds0);
    weights(st1, dpt1, ds1);
    __builtin_amdgcn_sched_barrier(0);
    grad(kt, 1, ds1);
    if (!split && wave >= 4) __builtin_amdgcn_s_setprio(0);
  };

  // Causal: keys past the workgroup's last query row are never seen.
  const int kend = p.causal ? min(nk, min(qb0 + BM, nq)) : nk;
  const int ntiles = (kend + BN - 1) / BN;
  // This wave group's key tiles [t0, t1), hn steps (a split workgroup's groups step in
  // lockstep, one barrier per step; a group past its last tile only takes the barriers).
  const int hn = split ? (ntiles + 1) / 2 : ntiles;
  const int t0 = grp * hn, t1 = min(ntiles, t0 + hn);
  uint64_t vw = 0;
  const KeyValidity kv{sl.mask, nk};
  uint32_t mbytes = 0;  // raw mask bytes of tile j + 1 during step j
  // Current and next tile buffers as distinct __restrict__ parameters (see dkdv_block).
  auto step = [&](int j, const char* __restrict__ ck, const char* __restrict__ cv,
                  char* __restrict__ nk_, char* __restrict__ nv) {
    const bool more = j + 1 < t1;
    uint64_t vw_next = 0;
    if (more) {
      vw_next = kv.word((j + 1) * BN, mbytes);
      mbytes = kv.load((j + 2) * BN);  // clamped: unused past the last tile
      if (vw_next != 0) issue((j + 1) * BN, nk_, nv);  // a fully masked tile is not read
    }
    if (j < t1 && vw != 0) compute(ck, cv, j * BN, vw);
    wait_tile_loads();
    __syncthreads();
    vw = vw_next;
  };
  if (t0 < t1) {
    vw = kv.word(t0 * BN, kv.load(t0 * BN));
    mbytes = kv.load((t0 + 1) * BN);
    issue(t0 * BN, sm[0].k[0], sm[0].v[0]);
    wait_tile_loads();
  }
  __syncthreads();
  for (int s = 0; s < hn; s += 2) {
    step(t0 + s, sm[0].k[0], sm[0].v[0], sm[0].k[1], sm[0].v[1]);
    if (s + 1 < hn) step(t0 + s + 1, sm[0].k[1], sm[0].v[1], sm[0].k[0], sm[0].v[0]);
  }
  if (split) {
    // Group 1 parks its partial sums in LDS (every tile read has completed at the last
    // step's barrier), group 0 adds them and stores.
    static_assert(4 * ND * 8 * 64 * sizeof(float) <= 2 * sizeof(DqSmem<D>), "reduction space");
    float* red = reinterpret_cast<float*>(&sm[0]) + (wave & 3) * (ND * 8 * 64);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((db * 2 + qb) * 4 + i) * 64 + lane] = dqacc[db][qb][i];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dqacc[db][qb][i] += red[((db * 2 + qb) * 4 + i) * 64 + lane];
  }

  // lane (c, g) stores d = 16 db + 4g .. +3 of its two rows
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw + 16 * qb + c;
    if (qrow < nq) {
      const long off = ((long)sl.qrow0 + qrow) * rs + (long)sl.qhead * D + 4 * g;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const long o = off + 16 * db;
        const f32x4 x = dqacc[db][qb] * p.scale;
        if (ACC) {
          f32x4* a = reinterpret_cast<f32x4*>(p.dq_acc + o);
          *a = (p.acc_flags & 1) ? *a + x : x;
        } else {
          *reinterpret_cast<bf16x4*>(p.dq + o) = to_bf16x4(x);
        }
      }
    }
  }
}

// One launch for both workgroup kinds.  A group is one (outer, key/value head): the dQ
// workgroups of its G query heads and its dK/dV workgroups.  The grid holds every workgroup
// of the longer kind (host-chosen; with G > 1 the dK/dV ones, which loop over G query
// heads) before every one of the shorter kind, in plain block order, which the hardware
// deals round-robin to the XCDs: each XCD gets its share of both kinds, long ones first,
// so the last workgroups to start are short ones.  (Grouping the workgroups of one head
// into one XCD's range, for L2 reuse, measured 5% slower on the 27280-token shard and 15%
// slower with grouped-query heads.)
template <int D, bool VARLEN, bool ACC>
__global__ __launch_bounds__(512, 1) void bwd_kernel(BwdParams p) {
  union Smem {
    DkdvSmem<D> kv;
    DqSmem<D> q[2];  // [1]: the second wave group's tiles of a split dQ workgroup
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int nqw = p.G * p.n_q_tiles;
  const int per_group = p.n_kv_tiles + nqw;
  const int ngroups = (p.n_blocks - p.n_q_split) / per_group;
  const int n_kv_all = p.n_kv_tiles * ngroups, n_q_all = nqw * ngroups;
  const int n_q_blocks = n_q_all + p.n_q_split;  // split dQ tiles count twice
  const int L = blockIdx.x;
  const bool kv_first = p.G > 1 || p.dkdv_first;
  const bool kv = kv_first ? L < n_kv_all : L >= n_q_blocks;
  int r = kv ? (kv_first ? L : L - n_q_blocks) : (kv_first ? L - n_kv_all : L);
  // The last n_q_split dQ tiles of the grid (host-chosen: dense non-causal launches whose
  // dQ workgroups come last) run as two split workgroups each, one per 128-row half.
  int half = -1;
  if (!kv && r >= n_q_all - p.n_q_split) {
    const int b = r - (n_q_all - p.n_q_split);
    r = n_q_all - p.n_q_split + b / 2;
    half = b & 1;
  }
  int group, idx;
  if (p.causal) {
    // Causal workgroups differ in length by tile (dK/dV: the first key tiles, dQ: the last
    // query tiles see the most): within each kind, the longest tile of every group first.
    if (kv) {
      group = r % ngroups;
      idx = r / ngroups;
    } else {
      const int rank = r / (ngroups * p.G), rest = r % (ngroups * p.G);
      group = rest / p.G;
      idx = (rest % p.G) * p.n_q_tiles + rank;
    }
  } else if (kv) {
    group = r / p.n_kv_tiles;
    idx = r % p.n_kv_tiles;
  } else {
    group = r / nqw;
    idx = r % nqw;
  }
  if (kv)
    dkdv_block<D, VARLEN, ACC>(p, decode<VARLEN>(p, group, idx, 0), sm.kv);
  else
    dq_block<D, VARLEN, ACC>(p, decode<VARLEN>(p, group, idx % p.n_q_tiles, idx / p.n_q_tiles), sm.q,
                             half);
}

template <int D, bool VARLEN, bool ACC>
static hipError_t launch_t(const BwdParams& p, hipStream_t stream) {
  if (p.n_blocks == 0) return hipSuccess;
  void* args[] = {const_cast<BwdParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_kernel<D, VARLEN, ACC>),
                         dim3(p.n_blocks), dim3(512), args, 0, stream);
}

hipError_t launch_bwd(int D, bool varlen, bool accum, const BwdParams& p, hipStream_t stream) {
  if (accum) {
    if (varlen) return hipErrorInvalidValue;  // accumulating launches are dense only
    return D == 64 ? launch_t<64, false, true>(p, stream) : launch_t<128, false, true>(p, stream);
  }
  if (D == 64) return varlen ? launch_t<64, true, false>(p, stream) : launch_t<64, false, false>(p, stream);
  return varlen ? launch_t<128, true, false>(p, stream) : launch_t<128, false, false>(p, stream);
}

}  // namespace attn
