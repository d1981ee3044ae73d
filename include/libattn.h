/*
 * libattn.h -- scaled-dot-product attention forward/backward for AMD MI355X (gfx950).
 *
 * The operation is the per-GPU attention a Ulysses sequence-parallel rank runs
 * once the all-to-all has handed it the full sequence and its share of the
 * heads (LightX2V PR #1234, "Performance": the Ulysses attention layer;
 * diffusers PR #14834, summary).  It is non-causal, dropout-free attention
 * (diffusers PR #14341, "Not verified") over BSHD tensors: the forward op
 * returns out in BSHD and the backward op consumes grad_out in BSHD, with K/V
 * read in the very layout they were handed in (diffusers PR #14341, body: the
 * K/V double-transpose fix).  For one (batch, head), query row i, key row j:
 *
 *   s_ij = scale * <q_i, k_j>, masked keys excluded (a bool key mask acts as a
 *          0 / -inf additive bias: diffusers PR #14341, follow-up 2)
 *   LSE_i = log sum_j exp(s_ij)        natural log, fp32, always produced
 *   out_i = sum_j exp(s_ij - LSE_i) v_j
 *   delta_i = <dO_i, out_i>
 *   dS_ij = P_ij (<dO_i, v_j> - delta_i),  P_ij = exp(s_ij - LSE_i)
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
 *
 * LSE is an auxiliary output with no gradient (diffusers PR #14834, summary),
 * and the backward needs it: a forward that skipped it broke training
 * (diffusers PR #14341, follow-up 1), so every forward here writes it.
 *
 * Conventions shared by every entry point
 *  - Tensors are bf16 (raw 16-bit patterns), contiguous.  Dense BSHD element
 *    (b,s,h,d) is at ((b*S + s)*H + h)*D + d.  Varlen tensors are packed
 *    (T, H, D), i.e. BSHD with B = 1 and S = T.
 *  - lse and delta are fp32, (B, H, Sq) row-major; varlen: (H, T).
 *  - key_mask: NULL (attend to every key) or (B, Sk) bytes, nonzero = attend.
 *    It is broadcast over heads and queries, i.e. a (B,1,1,Sk) mask.  A
 *    per-head (B,H,1,Sk) mask is not expressible and must be rejected by the
 *    caller before any work (diffusers PR #14834, "Unsupported cases").
 *  - Supported: head dim D in {64, 128}; Sq may differ from Sk.  The plain calls
 *    take Hk == H key/value heads; the _gqa and _ex calls take any Hk that
 *    divides H (grouped-query attention, below).
 *  - key_mask is read only for keys that exist: with Sk = 0 it is never read.
 *  - A query row whose keys are all masked gets out = 0, LSE = -inf, dQ = 0.
 *  - A tensor pointer may be NULL only when that tensor has no elements (e.g. k
 *    and v when Sk = 0); otherwise NULL is ATTN_ERR_NULL.
 *  - Every tensor pointer is device memory the caller allocated and owns; the
 *    library allocates nothing and is reentrant.  Its only state is a per-device
 *    cache of the compute-unit count (read once per device, with atomics, to size
 *    the grids); results therefore depend on the device a call runs on (see
 *    attn_fwd / attn_bwd on reproducibility).  Calls only
 *    enqueue work on `stream` (a hipStream_t; NULL = the default stream) and
 *    never synchronise.  Inputs must not alias outputs.
 *  - Every argument is checked on the host before any launch.  A call that
 *    returns an error has enqueued nothing and written nothing.  Nothing aborts.
 *  - Zero-sized problems (B, H, Sq or T = 0) return ATTN_OK and launch nothing.
 */
#ifndef LIBATTN_H
#define LIBATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is negative, or scale is not finite and >= 2^-64 */
  ATTN_ERR_UNSUPPORTED = 3, /* head dim not 64/128, H * D > 2^22, or a size beyond the
                               index range */
  ATTN_ERR_SEQLENS = 4,     /* cu_seqlens is not 0 = c0 <= c1 <= ... <= c_nseq = T */
  ATTN_ERR_HIP = 5          /* the HIP runtime refused a launch */
} attn_status;

/* Human-readable name of a status code (static storage). */
const char* attn_status_str(int status);

/* ABI revision of this header; bumped on any signature change. */
int attn_abi_version(void);

/*
 * Forward: q (B,Sq,H,D), k and v (B,Sk,H,D) bf16 -> out (B,Sq,H,D) bf16 and
 * lse (B,H,Sq) fp32.  scale multiplies q.k: finite and at least 2^-64 (callers
 * normally pass 1/sqrt(D)).
 * key_mask may be NULL.  Results are bitwise reproducible for a given shape on a
 * given device: when the grid's last round of workgroups would leave most compute
 * units idle, its query tiles run as split workgroups (chosen from the device's
 * compute-unit count) whose two key halves are combined at the end, which rounds
 * out and lse slightly differently from a whole tile.
 */
int attn_fwd(int B, int Sq, int Sk, int H, int D, float scale, const void* q, const void* k,
             const void* v, const uint8_t* key_mask, void* out, float* lse, void* stream);

/*
 * Backward preprocess: delta[b,h,i] = sum_d dO[b,i,h,d] * out[b,i,h,d] in fp32,
 * from the bf16 out the forward wrote.  out, dout (B,S,H,D) -> delta (B,H,S).
 * For varlen data call it with B = 1, S = T (delta is a per-row quantity).
 */
int attn_bwd_preprocess(int B, int S, int H, int D, const void* out, const void* dout,
                        float* delta, void* stream);

/*
 * Backward: from q, k, v, the forward's lse, the preprocess's delta and dout,
 * write dq (B,Sq,H,D), dk and dv (B,Sk,H,D), all bf16.  Keys excluded by
 * key_mask get dk = dv = 0 exactly.  dK/dV and dQ are produced by separate
 * workgroups (of one launch), each owning its output rows, so no atomics are
 * used and results are bitwise reproducible for a given shape on a given device
 * (the last dQ tiles of a dense call may run as split workgroups, chosen from the
 * device's compute-unit count, which sum their two key halves separately; another
 * device can therefore round dQ differently).  key_mask may be NULL.
 */
int attn_bwd(int B, int Sq, int Sk, int H, int D, float scale, const void* q, const void* k,
             const void* v, const uint8_t* key_mask, const float* lse, const float* delta,
             const void* dout, void* dq, void* dk, void* dv, void* stream);

/*
 * Grouped-query attention (named as not yet extended in diffusers PR #14834, description;
 * the key/value head count must divide the query head count, as the flash / cuDNN errors
 * quoted in diffusers PR #14341, reporter's tables, state): as attn_fwd / attn_bwd, but k
 * and v (and dk, dv) are (B,Sk,Hk,D) with H = G * Hk, and query head h attends with key /
 * value head h / G.  dk, dv of a key/value head sum the contributions of its G query heads
 * (computed in one workgroup per key tile, no atomics, bitwise reproducible for a given
 * shape and device).  Hk that does not divide H: ATTN_ERR_SHAPE.  attn_fwd / attn_bwd are
 * these calls with Hk = H.
 */
int attn_fwd_gqa(int B, int Sq, int Sk, int H, int Hk, int D, float scale, const void* q,
                 const void* k, const void* v, const uint8_t* key_mask, void* out, float* lse,
                 void* stream);
int attn_bwd_gqa(int B, int Sq, int Sk, int H, int Hk, int D, float scale, const void* q,
                 const void* k, const void* v, const uint8_t* key_mask, const float* lse,
                 const float* delta, const void* dout, void* dq, void* dk, void* dv,
                 void* stream);

/*
 * The general forms: Hk key/value heads as in attn_fwd_gqa / attn_bwd_gqa, and flags.
 * ATTN_CAUSAL: query row i attends to keys j <= i only (top-left aligned when Sq != Sk,
 * as torch's scaled_dot_product_attention with is_causal), combined with key_mask.  Causal
 * attention is named as not yet extended in diffusers PR #14834 (description); the pages
 * define no convention of their own.  Key tiles past a workgroup's last query row are
 * skipped, so a causal call does about half the work.  Unknown flag bits: ATTN_ERR_SHAPE.
 */
enum { ATTN_CAUSAL = 1 };
int attn_fwd_ex(int B, int Sq, int Sk, int H, int Hk, int D, float scale, int flags,
                const void* q, const void* k, const void* v, const uint8_t* key_mask, void* out,
                float* lse, void* stream);
int attn_bwd_ex(int B, int Sq, int Sk, int H, int Hk, int D, float scale, int flags,
                const void* q, const void* k, const void* v, const uint8_t* key_mask,
                const float* lse, const float* delta, const void* dout, void* dq, void* dk,
                void* dv, void* stream);

/*
 * Packed variable-length forward (the FA3-varlen path of diffusers PR #14834,
 * "Model test coverage"): nseq sequences packed back to back in q, k, v
 * (T, H, D); sequence n owns rows [cu[n], cu[n+1]) and attends only to its own
 * keys (block-diagonal, non-causal).  cu_seqlens_host and cu_seqlens_dev are
 * the same int32[nseq+1] array in host and device memory: the host copy is
 * validated (cu[0] = 0, non-decreasing) and sizes the launch; the kernels read
 * the device copy.  T = cu[nseq].  lse is (H, T).  No key mask in varlen mode.
 */
int attn_varlen_fwd(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                    int H, int D, float scale, const void* q, const void* k, const void* v,
                    void* out, float* lse, void* stream);

/* Packed variable-length backward; arguments as in attn_varlen_fwd and attn_bwd.
 * delta comes from attn_bwd_preprocess(1, T, H, D, out, dout, delta). */
int attn_varlen_bwd(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                    int H, int D, float scale, const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dout, void* dq, void* dk,
                    void* dv, void* stream);

/*
 * Merge of partial results over disjoint key chunks (ring / context-parallel attention:
 * the Ring-Anything backward that diffusers PR #14834 names as missing (description),
 * ring CP left unverified in diffusers PR #14341, "Not verified").  Chunk c's forward
 * over its own keys gave outs[c] (B,S,H,D) bf16 and lses[c] (B,H,S) fp32; writes
 *   lse = log sum_c exp(lses[c]),   out = sum_c exp(lses[c] - lse) outs[c]
 * (fp32 inside, out rounded once to bf16).  A chunk whose lse is -inf for a row adds
 * nothing to it; a row with -inf in every chunk gets out = 0, lse = -inf.
 * outs and lses are HOST arrays of n DEVICE pointers, 1 <= n <= 16 (else
 * ATTN_ERR_SHAPE / ATTN_ERR_UNSUPPORTED).  out and lse may alias one chunk's buffers
 * (in-place accumulation); they must not partially overlap them.
 */
int attn_lse_merge(int n, int B, int S, int H, int D, const void* const* outs,
                   const float* const* lses, void* out, float* lse, void* stream);

/*
 * Backward of one key chunk with the statistics of the whole key set (the merge-aware
 * backward of ring attention, same passages as attn_lse_merge).  Arguments as attn_bwd,
 * except that k, v, key_mask are the chunk's (Sk = chunk length), lse is the merged
 * (whole key set) LSE and delta = rowsum(dout * merged out), and the gradients go to
 * fp32 buffers: dq_acc (B,Sq,H,D) gets this chunk's dQ, dk_acc and dv_acc (B,Sk,H,D) the
 * chunk's dK, dV -- added to what the buffer holds if flags has ATTN_ACC_DQ (dq_acc) /
 * ATTN_ACC_DKDV (dk_acc, dv_acc), else written over it.  Summed over the chunks these
 * equal the full backward (first chunk: flags 0, later chunks: ATTN_ACC_DQ); round them
 * with attn_cast_bf16.  Other flag bits: ATTN_ERR_SHAPE.  Calls that share a buffer must
 * be ordered (same stream); the read-add-write is not atomic across concurrent calls.
 */
enum { ATTN_ACC_DQ = 1, ATTN_ACC_DKDV = 2 };
int attn_bwd_accum(int B, int Sq, int Sk, int H, int D, float scale, const void* q,
                   const void* k, const void* v, const uint8_t* key_mask, const float* lse,
                   const float* delta, const void* dout, float* dq_acc, float* dk_acc,
                   float* dv_acc, int flags, void* stream);

/* dst[i] = bf16(src[i]), round to nearest even, for n fp32 values (device pointers). */
int attn_cast_bf16(int64_t n, const float* src, void* dst, void* stream);

/* Varlen with flags (ATTN_CAUSAL applies inside each sequence). */
int attn_varlen_fwd_ex(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       int H, int D, float scale, int flags, const void* q, const void* k,
                       const void* v, void* out, float* lse, void* stream);
int attn_varlen_bwd_ex(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       int H, int D, float scale, int flags, const void* q, const void* k,
                       const void* v, const float* lse, const float* delta, const void* dout,
                       void* dq, void* dk, void* dv, void* stream);

/* Varlen with grouped-query heads (as attn_fwd_gqa / attn_bwd_gqa, inside each sequence):
 * q, out, dout, dq are (T, H, D), k, v, dk, dv (T, Hk, D), lse and delta (H, T); query head
 * h reads key/value head h / (H / Hk), and dk, dv of a key/value head sum its H / Hk query
 * heads.  Hk must divide H (else ATTN_ERR_SHAPE); flags as attn_varlen_fwd_ex.  The
 * attn_varlen_*_ex calls are these with Hk = H. */
int attn_varlen_fwd_gqa(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int H, int Hk, int D, float scale, int flags, const void* q,
                        const void* k, const void* v, void* out, float* lse, void* stream);
int attn_varlen_bwd_gqa(int nseq, const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int H, int Hk, int D, float scale, int flags, const void* q,
                        const void* k, const void* v, const float* lse, const float* delta,
                        const void* dout, void* dq, void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_H */
