/*
 * attn_oracle.c -- plain fp64 CPU reference for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes is the textbook definition of non-causal attention that the
 * pages refer to by op name only (diffusers PR #14341, body: the cuDNN / native
 * flash forward and backward op pairs; "Not verified": bf16, no dropout,
 * non-causal).  For one (batch, head) with query rows i and key rows j:
 *
 *   s_ij   = scale * <q_i, k_j>                      (only keys j the mask keeps)
 *   LSE_i  = log sum_j exp(s_ij)                     (natural log, scale included)
 *   P_ij   = exp(s_ij - LSE_i)
 *   out_i  = sum_j P_ij v_j
 *   delta_i= <dO_i, out_i>
 *   dP_ij  = <dO_i, v_j>,   dS_ij = P_ij (dP_ij - delta_i)
 *   dQ_i   = scale sum_j dS_ij k_j
 *   dK_j   = scale sum_i dS_ij q_i
 *   dV_j   = sum_i P_ij dO_i
 *
 * LSE is an auxiliary, non-differentiable output (diffusers PR #14834 summary).
 * Causal (the _ex entry points, causal = 1; named as not extended in diffusers PR
 * #14834, description, and defined on no page): query row i attends to keys j <= i only,
 * top-left aligned when Sq != Sk (the convention of torch's scaled_dot_product_attention
 * with is_causal); in varlen mode within each sequence.  It combines with the key mask.
 * A boolean key mask becomes a 0 / -inf bias (diffusers PR #14341, follow-up 2);
 * here excluded keys are simply skipped.  The mask is head-broadcast, shape
 * (B, 1, 1, Sk) passed as (B, Sk) bytes, nonzero = attend (diffusers PR #14834,
 * "Unsupported cases", per-head masks).  A query row whose keys are all masked
 * gets out = 0, LSE = -inf, dQ = 0 and contributes nothing to dK, dV.
 *
 * Layouts: q, k, v, out, dO, dQ, dK, dV are BSHD (element (b,s,h,d) at
 * ((b*S+s)*H+h)*D+d), matching the op contract that out is returned in BSHD.
 * LSE and delta are (B, H, Sq) row-major.  Varlen tensors are packed (T, H, D)
 * with int32 cu_seqlens[nseq+1]; their LSE / delta are (H, T).
 *
 * Loop form: forward by query rows, dQ by query rows (recomputing P and dP),
 * dK/dV by key columns (using the stored LSE and delta).  No tiling, no online
 * softmax: every score of a row is formed, then normalised.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static double dot(const double* a, const double* b, int D) {
  double acc = 0.0;
  for (int d = 0; d < D; ++d) acc += a[d] * b[d];
  return acc;
}

/* One (batch|sequence, head) slice.  Row r of q lives at q + r*rs (likewise k,
 * v, out, dout, dq, dk, dv); lse/delta are contiguous over query rows. */
typedef struct {
  const double *q, *k, *v;
  long rs;
  int nq, nk, D;
  const uint8_t* mask; /* nk bytes or NULL */
  double scale;
  int causal; /* query i sees keys j <= i only */
} slice_t;

static int key_on(const slice_t* s, int j) { return s->mask == NULL || s->mask[j] != 0; }
/* Whether query row i attends to key j: the key mask and, when causal, j <= i. */
static int pair_on(const slice_t* s, int i, int j) {
  return key_on(s, j) && (!s->causal || j <= i);
}

/* Forward for query row i of the slice.  sbuf holds nk doubles. */
static void fwd_row(const slice_t* s, int i, double* sbuf, double* out_i, double* lse_i) {
  const double* qi = s->q + (long)i * s->rs;
  double m = -INFINITY;
  for (int j = 0; j < s->nk; ++j) {
    if (!pair_on(s, i, j)) continue;
    sbuf[j] = s->scale * dot(qi, s->k + (long)j * s->rs, s->D);
    if (sbuf[j] > m) m = sbuf[j];
  }
  for (int d = 0; d < s->D; ++d) out_i[d] = 0.0;
  if (m == -INFINITY) { /* no key to attend to */
    *lse_i = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int j = 0; j < s->nk; ++j)
    if (pair_on(s, i, j)) l += exp(sbuf[j] - m);
  const double lse = m + log(l);
  for (int j = 0; j < s->nk; ++j) {
    if (!pair_on(s, i, j)) continue;
    const double p = exp(sbuf[j] - lse);
    const double* vj = s->v + (long)j * s->rs;
    for (int d = 0; d < s->D; ++d) out_i[d] += p * vj[d];
  }
  *lse_i = lse;
}

/* dQ for query row i, given its LSE and delta. */
static void dq_row(const slice_t* s, const double* dout, int i, double lse_i, double delta_i,
                   double* dq_i) {
  for (int d = 0; d < s->D; ++d) dq_i[d] = 0.0;
  if (lse_i == -INFINITY) return;
  const double* qi = s->q + (long)i * s->rs;
  const double* doi = dout + (long)i * s->rs;
  for (int j = 0; j < s->nk; ++j) {
    if (!pair_on(s, i, j)) continue;
    const double* kj = s->k + (long)j * s->rs;
    const double p = exp(s->scale * dot(qi, kj, s->D) - lse_i);
    const double dp = dot(doi, s->v + (long)j * s->rs, s->D);
    const double ds = p * (dp - delta_i);
    for (int d = 0; d < s->D; ++d) dq_i[d] += s->scale * ds * kj[d];
  }
}

/* dK and dV for key column j, given every row's LSE and delta. */
static void dkdv_col(const slice_t* s, const double* dout, int j, const double* lse,
                     const double* delta, double* dk_j, double* dv_j) {
  for (int d = 0; d < s->D; ++d) dk_j[d] = dv_j[d] = 0.0;
  if (!key_on(s, j)) return;
  const double* kj = s->k + (long)j * s->rs;
  const double* vj = s->v + (long)j * s->rs;
  for (int i = 0; i < s->nq; ++i) {
    if (lse[i] == -INFINITY || !pair_on(s, i, j)) continue;
    const double* qi = s->q + (long)i * s->rs;
    const double* doi = dout + (long)i * s->rs;
    const double p = exp(s->scale * dot(qi, kj, s->D) - lse[i]);
    const double dp = dot(doi, vj, s->D);
    const double ds = p * (dp - delta[i]);
    for (int d = 0; d < s->D; ++d) {
      dv_j[d] += p * doi[d];
      dk_j[d] += s->scale * ds * qi[d];
    }
  }
}

static int check_dims(int B, int Sq, int Sk, int H, int D) {
  return B >= 0 && Sq >= 0 && Sk >= 0 && H >= 0 && D > 0;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads used by the parallel loops from now on (n >= 1); returns the new count. */
int oracle_set_num_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
}

/* ---------------------------------------------------------------- dense BSHD */

int oracle_attn_fwd_ex(int B, int Sq, int Sk, int H, int D, double scale, const double* q,
                    const double* k, const double* v, const uint8_t* key_mask, double* out,
                    double* lse, int causal) {
  if (!check_dims(B, Sq, Sk, H, D)) return 2;
  const long rs = (long)H * D;
#pragma omp parallel
  {
    double* sbuf = (double*)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
#pragma omp for collapse(3) schedule(dynamic, 16)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int i = 0; i < Sq; ++i) {
          slice_t s = {q + (long)b * Sq * rs + (long)h * D, k + (long)b * Sk * rs + (long)h * D,
                       v + (long)b * Sk * rs + (long)h * D, rs, Sq, Sk, D,
                       key_mask ? key_mask + (long)b * Sk : NULL, scale, causal};
          fwd_row(&s, i, sbuf, out + ((long)b * Sq + i) * rs + (long)h * D,
                  lse + ((long)b * H + h) * Sq + i);
        }
    free(sbuf);
  }
  return 0;
}

int oracle_attn_fwd(int B, int Sq, int Sk, int H, int D, double scale, const double* q,
                    const double* k, const double* v, const uint8_t* key_mask, double* out,
                    double* lse) {
  return oracle_attn_fwd_ex(B, Sq, Sk, H, D, scale, q, k, v, key_mask, out, lse, 0);
}

int oracle_attn_delta(int B, int S, int H, int D, const double* out, const double* dout,
                      double* delta) {
  if (!check_dims(B, S, S, H, D)) return 2;
  const long rs = (long)H * D;
#pragma omp parallel for collapse(3)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < S; ++i) {
        const long o = ((long)b * S + i) * rs + (long)h * D;
        delta[((long)b * H + h) * S + i] = dot(dout + o, out + o, D);
      }
  return 0;
}

/* Backward.  out and lse are the forward's results; delta is formed from out
 * and written to delta_out when that is non-NULL.  Any of dq, dk, dv may be
 * NULL to skip that pass (dk and dv go together). */
int oracle_attn_bwd_ex(int B, int Sq, int Sk, int H, int D, double scale, const double* q,
                    const double* k, const double* v, const uint8_t* key_mask, const double* out,
                    const double* lse, const double* dout, double* delta_out, double* dq,
                    double* dk, double* dv, int causal) {
  if (!check_dims(B, Sq, Sk, H, D)) return 2;
  if ((dk == NULL) != (dv == NULL)) return 1;
  const long rs = (long)H * D;
  double* delta = delta_out ? delta_out : (double*)malloc(sizeof(double) * ((long)B * H * Sq + 1));
  oracle_attn_delta(B, Sq, H, D, out, dout, delta);
  if (dq) {
#pragma omp parallel for collapse(3) schedule(dynamic, 16)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int i = 0; i < Sq; ++i) {
          slice_t s = {q + (long)b * Sq * rs + (long)h * D, k + (long)b * Sk * rs + (long)h * D,
                       v + (long)b * Sk * rs + (long)h * D, rs, Sq, Sk, D,
                       key_mask ? key_mask + (long)b * Sk : NULL, scale, causal};
          const long r = ((long)b * H + h) * Sq + i;
          dq_row(&s, dout + (long)b * Sq * rs + (long)h * D, i, lse[r], delta[r],
                 dq + ((long)b * Sq + i) * rs + (long)h * D);
        }
  }
  if (dk) {
#pragma omp parallel for collapse(3) schedule(dynamic, 16)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int j = 0; j < Sk; ++j) {
          slice_t s = {q + (long)b * Sq * rs + (long)h * D, k + (long)b * Sk * rs + (long)h * D,
                       v + (long)b * Sk * rs + (long)h * D, rs, Sq, Sk, D,
                       key_mask ? key_mask + (long)b * Sk : NULL, scale, causal};
          const long r0 = ((long)b * H + h) * Sq;
          const long o = ((long)b * Sk + j) * rs + (long)h * D;
          dkdv_col(&s, dout + (long)b * Sq * rs + (long)h * D, j, lse + r0, delta + r0, dk + o,
                   dv + o);
        }
  }
  if (!delta_out) free(delta);
  return 0;
}

int oracle_attn_bwd(int B, int Sq, int Sk, int H, int D, double scale, const double* q,
                    const double* k, const double* v, const uint8_t* key_mask, const double* out,
                    const double* lse, const double* dout, double* delta_out, double* dq,
                    double* dk, double* dv) {
  return oracle_attn_bwd_ex(B, Sq, Sk, H, D, scale, q, k, v, key_mask, out, lse, dout, delta_out, dq, dk, dv, 0);
}

/* ------------------------------------------------------------ packed varlen */

static int check_cu(int nseq, const int32_t* cu) {
  if (nseq < 0 || cu == NULL || cu[0] != 0) return 0;
  for (int n = 0; n < nseq; ++n)
    if (cu[n + 1] < cu[n]) return 0;
  return 1;
}

/* Sequence n covers packed rows [cu[n], cu[n+1]); queries attend only to keys
 * of their own sequence (block-diagonal).  LSE is (H, T). */
int oracle_attn_varlen_fwd_ex(int nseq, const int32_t* cu, int H, int D, double scale,
                           const double* q, const double* k, const double* v, double* out,
                           double* lse, int causal) {
  if (!check_cu(nseq, cu) || H < 0 || D <= 0) return 4;
  const long rs = (long)H * D;
  const int T = cu[nseq];
  int maxlen = 1;
  for (int n = 0; n < nseq; ++n)
    if (cu[n + 1] - cu[n] > maxlen) maxlen = cu[n + 1] - cu[n];
#pragma omp parallel
  {
    double* sbuf = (double*)malloc(sizeof(double) * maxlen);
#pragma omp for collapse(2) schedule(dynamic, 16)
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < T; ++t) {
        int n = 0;
        while (cu[n + 1] <= t) ++n;
        const int s0 = cu[n], L = cu[n + 1] - cu[n];
        slice_t s = {q + (long)s0 * rs + (long)h * D, k + (long)s0 * rs + (long)h * D,
                     v + (long)s0 * rs + (long)h * D, rs, L, L, D, NULL, scale, causal};
        fwd_row(&s, t - s0, sbuf, out + (long)t * rs + (long)h * D, lse + (long)h * T + t);
      }
    free(sbuf);
  }
  return 0;
}

int oracle_attn_varlen_fwd(int nseq, const int32_t* cu, int H, int D, double scale,
                           const double* q, const double* k, const double* v, double* out,
                           double* lse) {
  return oracle_attn_varlen_fwd_ex(nseq, cu, H, D, scale, q, k, v, out, lse, 0);
}

int oracle_attn_varlen_bwd_ex(int nseq, const int32_t* cu, int H, int D, double scale,
                           const double* q, const double* k, const double* v, const double* out,
                           const double* lse, const double* dout, double* delta_out, double* dq,
                           double* dk, double* dv, int causal) {
  if (!check_cu(nseq, cu) || H < 0 || D <= 0) return 4;
  if ((dk == NULL) != (dv == NULL)) return 1;
  const long rs = (long)H * D;
  const int T = cu[nseq];
  double* delta = delta_out ? delta_out : (double*)malloc(sizeof(double) * ((long)H * T + 1));
  /* delta is a per-row quantity: the dense (B=1, S=T) form applies as is. */
  oracle_attn_delta(1, T, H, D, out, dout, delta);
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int h = 0; h < H; ++h)
    for (int t = 0; t < T; ++t) {
      int n = 0;
      while (cu[n + 1] <= t) ++n;
      const int s0 = cu[n], L = cu[n + 1] - cu[n];
      slice_t s = {q + (long)s0 * rs + (long)h * D, k + (long)s0 * rs + (long)h * D,
                   v + (long)s0 * rs + (long)h * D, rs, L, L, D, NULL, scale, causal};
      const long r0 = (long)h * T + s0;
      if (dq)
        dq_row(&s, dout + (long)s0 * rs + (long)h * D, t - s0, lse[r0 + t - s0],
               delta[r0 + t - s0], dq + (long)t * rs + (long)h * D);
      if (dk)
        dkdv_col(&s, dout + (long)s0 * rs + (long)h * D, t - s0, lse + r0, delta + r0,
                 dk + (long)t * rs + (long)h * D, dv + (long)t * rs + (long)h * D);
    }
  if (!delta_out) free(delta);
  return 0;
}

int oracle_attn_varlen_bwd(int nseq, const int32_t* cu, int H, int D, double scale,
                           const double* q, const double* k, const double* v, const double* out,
                           const double* lse, const double* dout, double* delta_out, double* dq,
                           double* dk, double* dv) {
  return oracle_attn_varlen_bwd_ex(nseq, cu, H, D, scale, q, k, v, out, lse, dout, delta_out, dq, dk, dv, 0);
}

/* ---------------------------------------------------------------- chunk merge */

/*
 * Merge of partial results over disjoint key chunks (ring / context-parallel
 * attention, whose backward diffusers PR #14834 names as missing in its
 * description).  It follows from the definition at the top of this file: with the
 * keys split into chunks c and lse_c, out_c each chunk's own forward,
 *   LSE_i = log sum_c sum_{j in c} exp(s_ij) = log sum_c exp(lse_c,i)
 *   out_i = sum_c sum_{j in c} exp(s_ij - LSE_i) v_j = sum_c exp(lse_c,i - LSE_i) out_c,i.
 * Computed as written; the largest lse_c,i is factored out of the first sum only to keep
 * exp() in range.  A row with lse_c,i = -inf in every chunk gets out = 0, LSE = -inf.
 * outs[c] are (B, S, H, D), lses[c] (B, H, S).
 */
int oracle_attn_lse_merge(int n, int B, int S, int H, int D, const double* const* outs,
                          const double* const* lses, double* out, double* lse) {
  if (n < 1 || !check_dims(B, S, S, H, D)) return 1;
  const long rows = (long)B * S * H;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const long h = r % H, bs = r / H, i = bs % S, b = bs / S;
    const long li = (b * H + h) * S + i;
    double m = -INFINITY;
    for (int c = 0; c < n; ++c)
      if (lses[c][li] > m) m = lses[c][li];
    double* o = out + r * D;
    if (m == -INFINITY) {
      lse[li] = -INFINITY;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      continue;
    }
    double sum = 0.0;
    for (int c = 0; c < n; ++c) sum += exp(lses[c][li] - m);
    const double L = m + log(sum);
    lse[li] = L;
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int c = 0; c < n; ++c) acc += exp(lses[c][li] - L) * outs[c][r * D + d];
      o[d] = acc;
    }
  }
  return 0;
}
