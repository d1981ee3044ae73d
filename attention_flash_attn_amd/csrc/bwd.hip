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
// dK/dV kernel: one workgroup = 4 waves = 128 keys; each wave keeps its 32
// keys' K and V rows in registers (B operands of S = Q K^T and dP = dO V^T,
// so the score tile has one key per lane) and its dK^T, dV^T accumulators in
// registers across the whole loop over query tiles.  Query tiles (Q, dO rows,
// LSE, delta) are double-buffered through LDS; Q^T and dO^T operands come from
// the LDS transposing read.
//
// Both run in ONE launch: the grid is grouped per (batch|sequence, head), each group
// holding that head's dK/dV workgroups followed by its dQ workgroups, and groups
// are dealt to XCDs in contiguous ranges.  Every XCD therefore gets the same mix
// of the two workgroup kinds, and the two kinds of one head share its Q/K/V/dO
// in that XCD's L2.
//
// dQ kernel: one workgroup = 4 waves = 128 query rows; each wave keeps Q and
// dO rows (B operands of S^T = K Q^T and dP^T = V dO^T: one query per lane, so
// LSE and delta are per-lane scalars) and its dQ^T accumulator in registers;
// K/V tiles of 64 keys are double-buffered through LDS; K^T comes from the
// transposing read.
#include "common.hpp"
#include "kernels.hpp"

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

// Shared decode of (tile, head, outer) and the row ranges of one workgroup.
struct Slice {
  int tile, head, qrow0, krow0, nq, nk;
  long lse_base;
  const uint8_t* mask;
};

template <bool VARLEN>
__device__ __forceinline__ Slice decode(const BwdParams& p, int group, int tile) {
  Slice s;
  s.tile = tile;
  s.head = group % p.H;
  const int outer = group / p.H;
  s.mask = nullptr;
  if (VARLEN) {
    const int s0 = p.cu[outer], s1 = p.cu[outer + 1];
    s.qrow0 = s.krow0 = s0;
    s.nq = s.nk = s1 - s0;
    s.lse_base = (long)s.head * p.Sq + s0;
  } else {
    s.qrow0 = outer * p.Sq;
    s.krow0 = outer * p.Sk;
    s.nq = p.Sq;
    s.nk = p.Sk;
    s.lse_base = ((long)outer * p.H + s.head) * p.Sq;
    if (p.mask) s.mask = p.mask + (long)outer * p.Sk;
  }
  return s;
}

__device__ __forceinline__ float pick16(const f32x4& a, const f32x4& b, const f32x4& c,
                                        const f32x4& d, int r) {
  return r < 4 ? a[r & 3] : r < 8 ? b[r & 3] : r < 12 ? c[r & 3] : d[r & 3];
}

// ------------------------------------------------------------------ dK / dV

template <int D>
struct DkdvSmem {
  static constexpr int BQ = 32, QS = D + 8;
  bf16 q[2][BQ * QS];
  bf16 o[2][BQ * QS];
  float l[2][BQ];
  float d[2][BQ];
};

template <int D>
struct DqSmem {
  static constexpr int BN = 64, KS = D + 8;
  bf16 k[2][BN * KS];
  bf16 v[2][BN * KS];
};

template <int D, bool VARLEN>
__device__ __forceinline__ void dkdv_block(const BwdParams& p, const Slice sl, DkdvSmem<D>& sm) {
  constexpr int BN = 128, BQ = DkdvSmem<D>::BQ;
  constexpr int QS = DkdvSmem<D>::QS;
  constexpr int NKS = D / 16, NMB = D / 32;
  constexpr int CPR = D / 8, RPP = 256 / CPR;
  constexpr int NPASS = (BQ + RPP - 1) / RPP;
  auto& sQ = sm.q;
  auto& sO = sm.o;
  auto& sL = sm.l;
  auto& sDl = sm.d;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int kb0 = sl.tile * BN;
  if (kb0 >= sl.nk) return;  // block-uniform
  const long rs = (long)p.H * D;
  const int nq = sl.nq, nk = sl.nk;

  const int key = kb0 + wave * 32 + l32;
  bool kvalid = key < nk;
  if (kvalid && sl.mask) kvalid = sl.mask[key] != 0;
  const bool wave_live = __ballot(kvalid) != 0;

  bf16x8 kreg[NKS], vreg[NKS];
  {
    const long off = ((long)sl.krow0 + key) * rs + (long)sl.head * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 z = {0, 0, 0, 0};
      kreg[ks] = as_bf16x8(key < nk ? ld16(p.k + off + 16 * ks) : z);
      vreg[ks] = as_bf16x8(key < nk ? ld16(p.v + off + 16 * ks) : z);
    }
  }

  const bf16* qbase = p.q + (long)sl.qrow0 * rs + (long)sl.head * D;
  const bf16* obase = p.dout + (long)sl.qrow0 * rs + (long)sl.head * D;
  const int sc = tid % CPR, sr0 = tid / CPR;
  u32x4 qr[NPASS], dr[NPASS];
  float lr = 0.f, dl = 0.f;
  auto load_tile = [&](int q0) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int r = sr0 + i * RPP;
      const int qi = q0 + r;
      const u32x4 z = {0, 0, 0, 0};
      const bool ok = r < BQ && qi < nq;
      qr[i] = ok ? ld16(qbase + (long)qi * rs + 8 * sc) : z;
      dr[i] = ok ? ld16(obase + (long)qi * rs + 8 * sc) : z;
    }
    if (tid < BQ) {
      const int qi = q0 + tid;
      lr = qi < nq ? p.lse[sl.lse_base + qi] * kLog2e : INFINITY;
      dl = qi < nq ? p.delta[sl.lse_base + qi] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int r = sr0 + i * RPP;
      if (r < BQ) {
        const int rq = (r & ~31) | kRowPerm(r & 31);
        *reinterpret_cast<u32x4*>(&sQ[buf][rq * QS + 8 * sc]) = qr[i];
        *reinterpret_cast<u32x4*>(&sO[buf][rq * QS + 8 * sc]) = dr[i];
      }
    }
    if (tid < BQ) {
      sL[buf][tid] = lr;
      sDl[buf][tid] = dl;
    }
  };

  const int g = lane >> 4, src = lane & 15;
  const int tr_off = (4 * (g >> 1) + (src >> 2)) * QS + 16 * (g & 1) + 4 * (src & 3);

  f32x16 dkacc[NMB], dvacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dkacc[mb] = dvacc[mb] = f32x16{};
  const float c2 = p.c2;

  const int ntiles = (nq + BQ - 1) / BQ;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < ntiles;
    if (more) load_tile((j + 1) * BQ);
    if (wave_live) {
      const bf16* sQb = sQ[buf];
      const bf16* sOb = sO[buf];
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sQb[l32 * QS + 16 * ks + 8 * hl]);
        s = mfma32(a, kreg[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sOb[l32 * QS + 16 * ks + 8 * hl]);
        dp = mfma32(a, vreg[ks], dp);
      }
      // Register r holds query 16*(r/8) + 8*hl + r%8 of the tile.
      const float* Lp = &sL[buf][8 * hl];
      const float* Dp = &sDl[buf][8 * hl];
      const f32x4 L0 = *reinterpret_cast<const f32x4*>(Lp), L1 = *reinterpret_cast<const f32x4*>(Lp + 4);
      const f32x4 L2 = *reinterpret_cast<const f32x4*>(Lp + 16), L3 = *reinterpret_cast<const f32x4*>(Lp + 20);
      const f32x4 D0 = *reinterpret_cast<const f32x4*>(Dp), D1 = *reinterpret_cast<const f32x4*>(Dp + 4);
      const f32x4 D2 = *reinterpret_cast<const f32x4*>(Dp + 16), D3 = *reinterpret_cast<const f32x4*>(Dp + 20);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = kvalid ? __builtin_amdgcn_exp2f(fmaf(s[r], c2, -pick16(L0, L1, L2, L3, r))) : 0.f;
        s[r] = pr;
        dp[r] = pr * (dp[r] - pick16(D0, D1, D2, D3, r));
      }
      bf16x8 pk[2], dsk[2];
      pk[0] = pack8(s, 0);
      pk[1] = pack8(s, 8);
      dsk[0] = pack8(dp, 0);
      dsk[1] = pack8(dp, 8);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16* op = sOb + 16 * t * QS + 32 * mb + tr_off;
          const bf16x8 ao = cat_tr(lds_read_tr16(op), lds_read_tr16(op + 8 * QS));
          dvacc[mb] = mfma32(ao, pk[t], dvacc[mb]);
          const bf16* qp = sQb + 16 * t * QS + 32 * mb + tr_off;
          const bf16x8 aq = cat_tr(lds_read_tr16(qp), lds_read_tr16(qp + 8 * QS));
          dkacc[mb] = mfma32(aq, dsk[t], dkacc[mb]);
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (key < nk) {
    const long off = ((long)sl.krow0 + key) * rs + (long)sl.head * D + 4 * hl;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (bf16)(dkacc[mb][4 * j4 + e] * p.scale);
          b[e] = (bf16)dvacc[mb][4 * j4 + e];
        }
        *reinterpret_cast<bf16x4*>(p.dk + off + 32 * mb + 8 * j4) = a;
        *reinterpret_cast<bf16x4*>(p.dv + off + 32 * mb + 8 * j4) = b;
      }
  }
}

// ------------------------------------------------------------------ dQ

template <int D, bool VARLEN>
__device__ __forceinline__ void dq_block(const BwdParams& p, const Slice sl, DqSmem<D>& sm) {
  constexpr int BM = 128, BN = DqSmem<D>::BN;
  constexpr int KS = DqSmem<D>::KS;
  constexpr int NKS = D / 16, NMB = D / 32;
  constexpr int CPR = D / 8, RPP = 256 / CPR, NPASS = BN / RPP;
  auto& sK = sm.k;
  auto& sV = sm.v;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int qb = sl.tile * BM;
  if (qb >= sl.nq) return;  // block-uniform
  const long rs = (long)p.H * D;
  const int nq = sl.nq, nk = sl.nk;

  const int qrow = qb + wave * 32 + l32;
  bf16x8 qreg[NKS], doreg[NKS];
  {
    const long off = ((long)sl.qrow0 + qrow) * rs + (long)sl.head * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 z = {0, 0, 0, 0};
      qreg[ks] = as_bf16x8(qrow < nq ? ld16(p.q + off + 16 * ks) : z);
      doreg[ks] = as_bf16x8(qrow < nq ? ld16(p.dout + off + 16 * ks) : z);
    }
  }
  const float lse2 = qrow < nq ? p.lse[sl.lse_base + qrow] * kLog2e : INFINITY;
  const float dl = qrow < nq ? p.delta[sl.lse_base + qrow] : 0.f;

  const bf16* kbase = p.k + (long)sl.krow0 * rs + (long)sl.head * D;
  const bf16* vbase = p.v + (long)sl.krow0 * rs + (long)sl.head * D;
  const int sc = tid % CPR, sr0 = tid / CPR;
  u32x4 kr[NPASS], vr[NPASS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int kk = k0 + sr0 + i * RPP;
      const u32x4 z = {0, 0, 0, 0};
      kr[i] = kk < nk ? ld16(kbase + (long)kk * rs + 8 * sc) : z;
      vr[i] = kk < nk ? ld16(vbase + (long)kk * rs + 8 * sc) : z;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      const int r = sr0 + i * RPP;
      const int rk = (r & ~31) | kRowPerm(r & 31);
      *reinterpret_cast<u32x4*>(&sK[buf][rk * KS + 8 * sc]) = kr[i];
      *reinterpret_cast<u32x4*>(&sV[buf][rk * KS + 8 * sc]) = vr[i];
    }
  };
  auto tile_valid = [&](int k0) -> uint64_t {
    const int kk = k0 + lane;
    bool ok = kk < nk;
    if (ok && sl.mask) ok = sl.mask[kk] != 0;
    return __ballot(ok);
  };

  const int g = lane >> 4, src = lane & 15;
  const int tr_off = (4 * (g >> 1) + (src >> 2)) * KS + 16 * (g & 1) + 4 * (src & 3);

  f32x16 dqacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) dqacc[mb] = f32x16{};
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
      f32x16 st[2], dpt[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        st[kb] = f32x16{};
        dpt[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sKb[(32 * kb + l32) * KS + 16 * ks + 8 * hl]);
          st[kb] = mfma32(a, qreg[ks], st[kb]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sVb[(32 * kb + l32) * KS + 16 * ks + 8 * hl]);
          dpt[kb] = mfma32(a, doreg[ks], dpt[kb]);
        }
      }
      const bool full = vw == ~0ull;
      bf16x8 dsk[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(fmaf(st[kb][r], c2, -lse2));
          if (!full && !((vw >> (32 * kb + c_row_permuted(r, hl))) & 1ull)) pr = 0.f;
          dpt[kb][r] = pr * (dpt[kb][r] - dl);
        }
        dsk[kb][0] = pack8(dpt[kb], 0);
        dsk[kb][1] = pack8(dpt[kb], 8);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16* kp = sKb + (32 * kb + 16 * t) * KS + 32 * mb + tr_off;
            const bf16x8 a = cat_tr(lds_read_tr16(kp), lds_read_tr16(kp + 8 * KS));
            dqacc[mb] = mfma32(a, dsk[kb][t], dqacc[mb]);
          }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    vw = vw_next;
  }

  if (qrow < nq) {
    bf16* dqp = p.dq + ((long)sl.qrow0 + qrow) * rs + (long)sl.head * D + 4 * hl;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(dqacc[mb][4 * j4 + e] * p.scale);
        *reinterpret_cast<bf16x4*>(dqp + 32 * mb + 8 * j4) = o;
      }
  }
}

// One launch for the whole backward.  Logical workgroup ids are grouped per
// (outer, head): [dK/dV tiles of that head][dQ tiles of that head].
template <int D, bool VARLEN>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  union Smem {
    DkdvSmem<D> kv;
    DqSmem<D> q;
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int logical = xcd_remap(blockIdx.x, p.n_blocks);
  const int per_group = p.n_kv_tiles + p.n_q_tiles;
  const int group = logical / per_group, within = logical % per_group;
  if (within < p.n_kv_tiles)
    dkdv_block<D, VARLEN>(p, decode<VARLEN>(p, group, within), sm.kv);
  else
    dq_block<D, VARLEN>(p, decode<VARLEN>(p, group, within - p.n_kv_tiles), sm.q);
}

template <int D, bool VARLEN>
static hipError_t launch_t(const BwdParams& p, hipStream_t stream) {
  if (p.n_blocks == 0) return hipSuccess;
  void* args[] = {const_cast<BwdParams*>(&p)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_kernel<D, VARLEN>), dim3(p.n_blocks),
                         dim3(256), args, 0, stream);
}

hipError_t launch_bwd(int D, bool varlen, const BwdParams& p, hipStream_t stream) {
  if (D == 64) return varlen ? launch_t<64, true>(p, stream) : launch_t<64, false>(p, stream);
  return varlen ? launch_t<128, true>(p, stream) : launch_t<128, false>(p, stream);
}

}  // namespace attn
