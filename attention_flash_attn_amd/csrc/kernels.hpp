// kernels.hpp -- launch parameters shared between the host entry points and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Dense problems: outer index = batch, rows of batch b start at b*Sq (q) / b*Sk (k).
// Varlen problems: outer index = sequence n, rows [cu[n], cu[n+1]); Sq = Sk = T.
// Varlen launches order their sequences longest first (the workgroups of a sequence all
// take about its length), for up to this many sequences; seq_order[r] is the sequence of
// rank r.  With more sequences (n_order = 0) they run in their given order.
constexpr int kMaxOrderedSeqs = 64;
struct SeqOrder {
  int n_order;  // 0: given order
  int16_t seq[kMaxOrderedSeqs];
  __device__ __forceinline__ int operator()(int r) const { return n_order ? seq[r] : r; }
};

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const uint8_t* mask;  // dense only: (B, Sk) bytes or null
  __bf16* out;
  float* lse;
  const int32_t* cu;  // varlen only (device)
  int B, Sq, Sk, H;
  int Hk, G;     // key/value heads and query heads per key/value head (H = G * Hk)
  int causal;    // query row i sees keys j <= i only (within its sequence)
  int n_qtiles;  // query tiles per (outer, head)
  int n_full;    // blocks [0, n_full): whole query tiles; the rest: parts of tiles n_full...
  int split;     // parts (2 or 4) per query tile of the split blocks
  int n_blocks;
  float c2;  // scale * log2(e)
  SeqOrder order;  // varlen only
};

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const uint8_t* mask;
  const float* lse;
  const float* delta;
  const __bf16* dout;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* dq_acc;  // fp32-output launches: written instead of dq/dk/dv
  float* dk_acc;
  float* dv_acc;
  int acc_flags;  // bit 0: add into dq_acc, bit 1: add into dk_acc/dv_acc (else overwrite)
  const int32_t* cu;
  int B, Sq, Sk, H;
  int Hk, G;       // key/value heads and query heads per key/value head (H = G * Hk)
  int causal;      // query row i sees keys j <= i only (within its sequence)
  int n_kv_tiles;  // dK/dV workgroups per (outer, key/value head)
  int n_q_tiles;   // dQ workgroups per (outer, query head)
  int dkdv_first;  // grid order: the dK/dV workgroups first (they are the longer kind)
  int n_q_split;   // the last dQ tiles of the grid that run as two half-row workgroups each
  int n_blocks;
  float c2;     // scale * log2(e)
  float scale;
  SeqOrder order;  // varlen only
};

constexpr int kFwdBlockM = 256;   // query rows per forward workgroup (8 waves x 32)
constexpr int kDqBlockM = 256;    // query rows per dQ workgroup
constexpr int kDkvBlockN = 256;   // key rows per dK/dV workgroup

hipError_t launch_fwd(int D, bool varlen, const FwdParams& p, hipStream_t stream);
// accum: fp32 dQ/dK/dV into p.dq_acc/dk_acc/dv_acc (added or overwritten per p.acc_flags)
// instead of bf16 dq/dk/dv (dense only)
hipError_t launch_bwd(int D, bool varlen, bool accum, const BwdParams& p, hipStream_t stream);
hipError_t launch_delta(int D, long rows, int S, int H, const __bf16* out, const __bf16* dout,
                        float* delta, hipStream_t stream);

// Merge of partial attention results over disjoint key chunks (see merge.hip).
constexpr int kMaxMergeChunks = 16;
struct MergeParams {
  const __bf16* out[kMaxMergeChunks];  // (B, S, H, D) each
  const float* lse[kMaxMergeChunks];   // (B, H, S) each
  __bf16* dst;
  float* dst_lse;
  long rows;  // B * S * H
  int S, H, n;
};
hipError_t launch_merge(int D, const MergeParams& p, hipStream_t stream);
hipError_t launch_cast_bf16(long n, const float* src, __bf16* dst, hipStream_t stream);

}  // namespace attn
