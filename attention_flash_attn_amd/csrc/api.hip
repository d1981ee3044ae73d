// api.hip -- the C ABI of libattn: argument validation on the host, then launches.
//
// Every check runs before anything is enqueued, so a call that returns an
// error has launched nothing and written nothing.  No allocation, no
// synchronisation (the caller's stream orders the work), and no state beyond a
// per-device cache of the compute-unit count that sizes the grids.
#include <math.h>
#include <limits.h>

#include <algorithm>
#include <atomic>

#include "libattn.h"
#include "common.hpp"
#include "kernels.hpp"

using attn::BwdParams;
using attn::FwdParams;

namespace {

constexpr int kAbiVersion = 5;

bool head_dim_ok(int D) { return D == 64 || D == 128; }
// The backward starts its score accumulators from -LSE/scale; the lower bound keeps that
// finite for any LSE the forward can produce.
bool scale_ok(float s) { return isfinite(s) && s >= 0x1p-64f; }
// Tile copies address up to 256 rows of one tensor (row stride H * D elements) with 32-bit
// signed byte offsets.
bool row_width_ok(int H, int D) { return 256L * 2 * H * D <= INT_MAX; }
long cdiv(long a, long b) { return (a + b - 1) / b; }
int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }
// A tensor pointer may be NULL only when the tensor has no elements.
bool missing(const void* ptr, bool has_elements) { return ptr == nullptr && has_elements; }

// Sizes for dense calls; returns ATTN_OK or an error code.
int check_dense(int B, int Sq, int Sk, int H, int D, float scale) {
  if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (!scale_ok(scale)) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(D) || !row_width_ok(H, D)) return ATTN_ERR_UNSUPPORTED;
  // Row indices (b*S + s) and workgroup counts are kept in 32-bit integers.
  if ((long)B * Sq > INT_MAX || (long)B * Sk > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  if ((cdiv(Sq, 32) + cdiv(Sk, 32)) * H * (long)B > INT_MAX)
    return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// Key/value head count of grouped-query attention: it divides H (H = G * Hk, G >= 1).
int check_kv_heads(int H, int Hk) {
  if (Hk < 0) return ATTN_ERR_SHAPE;
  if (H == 0) return Hk == 0 ? ATTN_OK : ATTN_ERR_SHAPE;
  if (Hk == 0 || H % Hk != 0) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Validates the host copy of cu_seqlens; on success sets T and the longest length.
int check_varlen(int nseq, const int32_t* cu, int H, int D, float scale, int* T, int* maxlen) {
  if (nseq < 0 || H < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (!scale_ok(scale)) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(D) || !row_width_ok(H, D)) return ATTN_ERR_UNSUPPORTED;
  if (cu[0] != 0) return ATTN_ERR_SEQLENS;
  int mx = 0;
  for (int n = 0; n < nseq; ++n) {
    if (cu[n + 1] < cu[n]) return ATTN_ERR_SEQLENS;
    const int len = cu[n + 1] - cu[n];
    if (len > mx) mx = len;
  }
  if (2 * cdiv(mx, 32) * H * (long)nseq > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  *T = cu[nseq];
  *maxlen = mx;
  return ATTN_OK;
}

// Sequences by length, longest first (stable), when there are few enough to list.
attn::SeqOrder seq_order(int nseq, const int32_t* cu) {
  attn::SeqOrder o{};
  if (nseq <= 1 || nseq > attn::kMaxOrderedSeqs) return o;
  o.n_order = nseq;
  for (int n = 0; n < nseq; ++n) o.seq[n] = (int16_t)n;
  for (int i = 1; i < nseq; ++i) {  // insertion sort, at most 64 entries
    const int16_t x = o.seq[i];
    const int len = cu[x + 1] - cu[x];
    int j = i - 1;
    while (j >= 0 && cu[o.seq[j] + 1] - cu[o.seq[j]] < len) {
      o.seq[j + 1] = o.seq[j];
      --j;
    }
    o.seq[j + 1] = x;
  }
  return o;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid size or scale";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim or size";
    case ATTN_ERR_SEQLENS: return "invalid cu_seqlens";
    case ATTN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return kAbiVersion; }

// Compute units of the device that runs `stream`.  The count is a fixed property of the
// device, so it is cached per device: the library's only state.  Concurrent first calls
// may both query it and store the same value; the atomics make that race well defined.
static int cu_count(hipStream_t stream) {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) dev = 0;
  if (dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Grid of the forward launch: one block per whole query tile, except that the last
// partial round of `rem` tiles of a grid of at least one full round may run as S split
// blocks per tile (S = 2 or 4: 256 / S rows each, the keys shared out between S wave
// groups), which take about 1 / S as long.  S is chosen to minimise the rounds of split
// blocks, ceil(S rem / ncu) / S, in units of a whole tile's time (ties: fewer parts).  Only
// where the tiles are of equal length (`may_split`: dense, non-causal).  A grid of fewer
// tiles than CUs is not split: its key loops are short enough that the split blocks'
// lockstep steps cost more than the idle CUs (1024-token shape: 27 -> 36 us).
static void fwd_grid(FwdParams& p, int tiles, bool may_split, hipStream_t stream) {
  p.n_full = tiles;
  p.n_blocks = tiles;
  p.split = 2;
  if (!may_split || tiles == 0) return;
  const int ncu = cu_count(stream);
  const int rem = tiles % ncu;
  if (tiles < ncu || rem == 0) return;
  int best = 1;
  double best_t = 1.0;
  for (int S : {2, 4}) {
    const double t = (double)cdiv((long)S * rem, ncu) / S;
    if (t < best_t) {
      best = S;
      best_t = t;
    }
  }
  if (best > 1) {
    p.split = best;
    p.n_full = tiles - rem;
    p.n_blocks = p.n_full + best * rem;
  }
}

int attn_fwd(int B, int Sq, int Sk, int H, int D, float scale, const void* q, const void* k,
             const void* v, const uint8_t* key_mask, void* out, float* lse, void* stream) {
  return attn_fwd_ex(B, Sq, Sk, H, H, D, scale, 0, q, k, v, key_mask, out, lse, stream);
}

int attn_fwd_gqa(int B, int Sq, int Sk, int H, int Hk, int D, float scale, const void* q,
                 const void* k, const void* v, const uint8_t* key_mask, void* out, float* lse,
                 void* stream) {
  return attn_fwd_ex(B, Sq, Sk, H, Hk, D, scale, 0, q, k, v, key_mask, out, lse, stream);
}

int attn_fwd_ex(int B, int Sq, int Sk, int H, int Hk, int D, float scale, int flags,
                const void* q, const void* k, const void* v, const uint8_t* key_mask, void* out,
                float* lse, void* stream) {
  int st = check_dense(B, Sq, Sk, H, D, scale);
  if (st == ATTN_OK) st = check_kv_heads(H, Hk);
  if (st == ATTN_OK && (flags & ~ATTN_CAUSAL)) st = ATTN_ERR_SHAPE;
  if (st != ATTN_OK) return st;
  const bool has_q = (long)B * Sq * H > 0, has_k = (long)B * Sk * Hk > 0;
  if (missing(q, has_q) || missing(out, has_q) || missing(lse, has_q) || missing(k, has_k) ||
      missing(v, has_k))
    return ATTN_ERR_NULL;
  if ((long)B * H * Sq == 0) return ATTN_OK;
  FwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.mask = Sk > 0 ? key_mask : nullptr;  // with no keys there is no mask byte to read
  p.out = static_cast<__bf16*>(out);
  p.lse = lse;
  p.cu = nullptr;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.H = H;
  p.Hk = Hk;
  p.G = H / Hk;
  p.causal = flags & ATTN_CAUSAL;
  p.n_qtiles = (int)cdiv(Sq, attn::kFwdBlockM);
  fwd_grid(p, p.n_qtiles * H * B, !p.causal, static_cast<hipStream_t>(stream));
  p.c2 = scale * attn::kLog2e;
  return status_of(attn::launch_fwd(D, false, p, static_cast<hipStream_t>(stream)));
}

int attn_bwd_preprocess(int B, int S, int H, int D, const void* out, const void* dout,
                        float* delta, void* stream) {
  if (B < 0 || S < 0 || H < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(D)) return ATTN_ERR_UNSUPPORTED;
  const long rows = (long)B * S * H;
  if (missing(out, rows > 0) || missing(dout, rows > 0) || missing(delta, rows > 0))
    return ATTN_ERR_NULL;
  if (rows == 0) return ATTN_OK;
  if (cdiv(rows, 256 / (D / 8)) > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  return status_of(attn::launch_delta(D, rows, S, H, static_cast<const __bf16*>(out),
                                      static_cast<const __bf16*>(dout), delta,
                                      static_cast<hipStream_t>(stream)));
}

static BwdParams bwd_params(int B, int Sq, int Sk, int H, int Hk, float scale, const void* q,
                            const void* k, const void* v, const uint8_t* key_mask,
                            const float* lse, const float* delta, const void* dout, void* dq,
                            void* dk, void* dv, const int32_t* cu) {
  BwdParams p{};
  p.Hk = Hk;
  p.G = Hk > 0 ? H / Hk : 1;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.mask = Sk > 0 ? key_mask : nullptr;  // with no keys there is no mask byte to read
  p.lse = lse;
  p.delta = delta;
  p.dout = static_cast<const __bf16*>(dout);
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.cu = cu;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.H = H;
  p.c2 = scale * attn::kLog2e;
  p.scale = scale;
  return p;
}

// Grid of the backward launch: per (outer, key/value head) the dQ workgroups of its G query
// heads and its dK/dV workgroups; the kernel starts every workgroup of the longer kind
// before the shorter ones.  Work per workgroup: dK/dV 256 keys x G * nq query rows x 4
// products, dQ 256 query rows x nk keys x 3 products.  When the dQ workgroups come last
// and all take equally long (dense, non-causal), the last half-CU-count of them run as
// split workgroups (two per tile, 128 rows each, half the time), so that the launch's last
// round finishes together instead of leaving most CUs idle behind a few whole tiles.
static void bwd_grid(BwdParams& p, int nq, int nk, int outer, bool may_split, hipStream_t stream) {
  p.n_kv_tiles = (int)cdiv(nk, attn::kDkvBlockN);
  p.n_q_tiles = (int)cdiv(nq, attn::kDqBlockM);
  p.dkdv_first = (long)attn::kDkvBlockN * 4 * p.G * nq > (long)attn::kDqBlockM * 3 * nk;
  const int n_q_all = p.G * p.n_q_tiles * p.Hk * outer;
  p.n_q_split = 0;
  if (may_split && (p.G > 1 || p.dkdv_first)) p.n_q_split = std::min(n_q_all, cu_count(stream) / 2);
  p.n_blocks = (p.n_kv_tiles + p.G * p.n_q_tiles) * p.Hk * outer + p.n_q_split;
}

int attn_bwd(int B, int Sq, int Sk, int H, int D, float scale, const void* q, const void* k,
             const void* v, const uint8_t* key_mask, const float* lse, const float* delta,
             const void* dout, void* dq, void* dk, void* dv, void* stream) {
  return attn_bwd_ex(B, Sq, Sk, H, H, D, scale, 0, q, k, v, key_mask, lse, delta, dout, dq, dk,
                     dv, stream);
}

int attn_bwd_gqa(int B, int Sq, int Sk, int H, int Hk, int D, float scale, const void* q,
                 const void* k, const void* v, const uint8_t* key_mask, const float* lse,
                 const float* delta, const void* dout, void* dq, void* dk, void* dv,
                 void* stream) {
  return attn_bwd_ex(B, Sq, Sk, H, Hk, D, scale, 0, q, k, v, key_mask, lse, delta, dout, dq, dk,
                     dv, stream);
}

int attn_bwd_ex(int B, int Sq, int Sk, int H, int Hk, int D, float scale, int flags,
                const void* q, const void* k, const void* v, const uint8_t* key_mask,
                const float* lse, const float* delta, const void* dout, void* dq, void* dk,
                void* dv, void* stream) {
  int st = check_dense(B, Sq, Sk, H, D, scale);
  if (st == ATTN_OK) st = check_kv_heads(H, Hk);
  if (st == ATTN_OK && (flags & ~ATTN_CAUSAL)) st = ATTN_ERR_SHAPE;
  if (st != ATTN_OK) return st;
  const bool hq = (long)B * Sq * H > 0, hk = (long)B * Sk * Hk > 0;
  if (missing(q, hq) || missing(lse, hq) || missing(delta, hq) || missing(dout, hq) ||
      missing(dq, hq) || missing(k, hk) || missing(v, hk) || missing(dk, hk) || missing(dv, hk))
    return ATTN_ERR_NULL;
  if ((long)B * H == 0) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  BwdParams p = bwd_params(B, Sq, Sk, H, Hk, scale, q, k, v, key_mask, lse, delta, dout, dq, dk,
                           dv, nullptr);
  p.causal = flags & ATTN_CAUSAL;
  bwd_grid(p, Sq, Sk, B, !p.causal, s);
  return status_of(attn::launch_bwd(D, false, false, p, s));
}

int attn_bwd_accum(int B, int Sq, int Sk, int H, int D, float scale, const void* q,
                   const void* k, const void* v, const uint8_t* key_mask, const float* lse,
                   const float* delta, const void* dout, float* dq_acc, float* dk_acc,
                   float* dv_acc, int flags, void* stream) {
  const int st = check_dense(B, Sq, Sk, H, D, scale);
  if (st != ATTN_OK) return st;
  if (flags & ~(ATTN_ACC_DQ | ATTN_ACC_DKDV)) return ATTN_ERR_SHAPE;
  const bool hq = (long)B * Sq * H > 0, hk = (long)B * Sk * H > 0;
  if (missing(q, hq) || missing(lse, hq) || missing(delta, hq) || missing(dout, hq) ||
      missing(dq_acc, hq) || missing(k, hk) || missing(v, hk) || missing(dk_acc, hk) ||
      missing(dv_acc, hk))
    return ATTN_ERR_NULL;
  if ((long)B * H == 0) return ATTN_OK;
  BwdParams p = bwd_params(B, Sq, Sk, H, H, scale, q, k, v, key_mask, lse, delta, dout, nullptr,
                           nullptr, nullptr, nullptr);
  p.dq_acc = dq_acc;
  p.dk_acc = dk_acc;
  p.dv_acc = dv_acc;
  p.acc_flags = flags;
  bwd_grid(p, Sq, Sk, B, true, static_cast<hipStream_t>(stream));
  return status_of(attn::launch_bwd(D, false, true, p, static_cast<hipStream_t>(stream)));
}

int attn_lse_merge(int n, int B, int S, int H, int D, const void* const* outs,
                   const float* const* lses, void* out, float* lse, void* stream) {
  if (n < 1 || B < 0 || S < 0 || H < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (!head_dim_ok(D) || n > attn::kMaxMergeChunks) return ATTN_ERR_UNSUPPORTED;
  if (!outs || !lses) return ATTN_ERR_NULL;
  const long rows = (long)B * S * H;
  for (int i = 0; i < n; ++i)
    if (missing(outs[i], rows > 0) || missing(lses[i], rows > 0)) return ATTN_ERR_NULL;
  if (missing(out, rows > 0) || missing(lse, rows > 0)) return ATTN_ERR_NULL;
  if (rows == 0) return ATTN_OK;
  if (cdiv(rows, 256 / (D / 8)) > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  attn::MergeParams p{};
  for (int i = 0; i < n; ++i) {
    p.out[i] = static_cast<const __bf16*>(outs[i]);
    p.lse[i] = lses[i];
  }
  p.dst = static_cast<__bf16*>(out);
  p.dst_lse = lse;
  p.rows = rows;
  p.S = S;
  p.H = H;
  p.n = n;
  return status_of(attn::launch_merge(D, p, static_cast<hipStream_t>(stream)));
}

int attn_cast_bf16(int64_t n, const float* src, void* dst, void* stream) {
  if (n < 0) return ATTN_ERR_SHAPE;
  if (missing(src, n > 0) || missing(dst, n > 0)) return ATTN_ERR_NULL;
  if (n == 0) return ATTN_OK;
  if (cdiv(n, 2048) > INT_MAX) return ATTN_ERR_UNSUPPORTED;
  return status_of(attn::launch_cast_bf16(n, src, static_cast<__bf16*>(dst),
                                          static_cast<hipStream_t>(stream)));
}

int attn_varlen_fwd(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                    int H, int D, float scale, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* stream) {
  return attn_varlen_fwd_ex(nseq, cu_seqlens_host, cu_seqlens_dev, H, D, scale, 0, q, k, v, out,
                            lse, stream);
}

int attn_varlen_fwd_ex(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       int H, int D, float scale, int flags, const void* q, const void* k,
                       const void* v, void* out, float* lse, void* stream) {
  return attn_varlen_fwd_gqa(nseq, cu_seqlens_host, cu_seqlens_dev, H, H, D, scale, flags, q, k,
                             v, out, lse, stream);
}

int attn_varlen_fwd_gqa(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int H, int Hk, int D, float scale, int flags, const void* q,
                        const void* k, const void* v, void* out, float* lse, void* stream) {
  if (!cu_seqlens_host || !cu_seqlens_dev) return ATTN_ERR_NULL;
  if (flags & ~ATTN_CAUSAL) return ATTN_ERR_SHAPE;
  int T = 0, maxlen = 0;
  int st = check_varlen(nseq, cu_seqlens_host, H, D, scale, &T, &maxlen);
  if (st == ATTN_OK) st = check_kv_heads(H, Hk);
  if (st != ATTN_OK) return st;
  const bool ht = (long)T * H > 0, hk = (long)T * Hk > 0;
  if (missing(q, ht) || missing(k, hk) || missing(v, hk) || missing(out, ht) || missing(lse, ht))
    return ATTN_ERR_NULL;
  if ((long)T * H == 0) return ATTN_OK;
  FwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.mask = nullptr;
  p.out = static_cast<__bf16*>(out);
  p.lse = lse;
  p.cu = cu_seqlens_dev;
  p.B = nseq;
  p.Sq = p.Sk = T;
  p.H = H;
  p.Hk = Hk;
  p.G = H / Hk;
  p.causal = flags & ATTN_CAUSAL;
  p.n_qtiles = (int)cdiv(maxlen, attn::kFwdBlockM);
  p.order = seq_order(nseq, cu_seqlens_host);
  fwd_grid(p, p.n_qtiles * H * nseq, false, static_cast<hipStream_t>(stream));
  p.c2 = scale * attn::kLog2e;
  return status_of(attn::launch_fwd(D, true, p, static_cast<hipStream_t>(stream)));
}

int attn_varlen_bwd(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                    int H, int D, float scale, const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dout, void* dq, void* dk,
                    void* dv, void* stream) {
  return attn_varlen_bwd_ex(nseq, cu_seqlens_host, cu_seqlens_dev, H, D, scale, 0, q, k, v, lse,
                            delta, dout, dq, dk, dv, stream);
}

int attn_varlen_bwd_ex(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       int H, int D, float scale, int flags, const void* q, const void* k,
                       const void* v, const float* lse, const float* delta, const void* dout,
                       void* dq, void* dk, void* dv, void* stream) {
  return attn_varlen_bwd_gqa(nseq, cu_seqlens_host, cu_seqlens_dev, H, H, D, scale, flags, q, k,
                             v, lse, delta, dout, dq, dk, dv, stream);
}

int attn_varlen_bwd_gqa(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int H, int Hk, int D, float scale, int flags, const void* q,
                        const void* k, const void* v, const float* lse, const float* delta,
                        const void* dout, void* dq, void* dk, void* dv, void* stream) {
  if (!cu_seqlens_host || !cu_seqlens_dev) return ATTN_ERR_NULL;
  if (flags & ~ATTN_CAUSAL) return ATTN_ERR_SHAPE;
  int T = 0, maxlen = 0;
  int st = check_varlen(nseq, cu_seqlens_host, H, D, scale, &T, &maxlen);
  if (st == ATTN_OK) st = check_kv_heads(H, Hk);
  if (st != ATTN_OK) return st;
  const bool ht = (long)T * H > 0, hk = (long)T * Hk > 0;
  if (missing(q, ht) || missing(k, hk) || missing(v, hk) || missing(lse, ht) ||
      missing(delta, ht) || missing(dout, ht) || missing(dq, ht) || missing(dk, hk) ||
      missing(dv, hk))
    return ATTN_ERR_NULL;
  if ((long)T * H == 0) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  BwdParams p = bwd_params(nseq, T, T, H, Hk, scale, q, k, v, nullptr, lse, delta, dout, dq, dk,
                           dv, cu_seqlens_dev);
  p.causal = flags & ATTN_CAUSAL;
  p.order = seq_order(nseq, cu_seqlens_host);
  bwd_grid(p, maxlen, maxlen, nseq, false, s);
  return status_of(attn::launch_bwd(D, true, false, p, s));
}

}  // extern "C"
