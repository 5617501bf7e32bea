// Internal declarations shared by the C-ABI layer (api.hip) and the kernel translation units.
// Not installed; the public interface is include/ebattn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ebattn {

// Arguments of one attention-forward launch over B*H independent (batch, head) slices.
// Layout: q [BH, Nq, d], k/v [BH / kv_group, Nk, d], o [BH, Nq, d], lse [BH, Nq], all contiguous, d fastest;
// query slice bh reads key/value slice bh / kv_group (grouped-query heads: consecutive query heads share one
// key/value head; kv_group = 1 is plain multi-head attention).
// Causal masking by global position, with an optional sliding window, reduces to "key j visible to query i iff
// i + lo <= j <= i + diag" (host computes diag = floor((q_off - k_off) / pos_stride) and, for a window of w
// positions, lo = floor((q_off - k_off - w) / pos_stride) + 1, both clamped; without a window lo = kNoWindow).
// Non-causal launches ignore diag and lo.
constexpr int kNoWindow = -(1 << 30);
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH;
  int Nq;
  int Nk;
  float scale_log2;   // softmax scale times log2(e): the kernels work in the exp2 domain
  int causal;
  int diag;
  int lo;
  int kv_group;
  // Optional running result to merge with (bf16 MFMA path only; null otherwise): fp32 o [BH, Nq, d] and lse
  // [BH, Nq] of the same query rows over other keys. The kernel then writes the log-sum-exp merge of that running
  // result and its own in place of its own; o may alias merge_o (fp32 output) and lse may alias merge_lse.
  const float* merge_o;
  const float* merge_lse;
};

// bf16 operands on MFMA; d in {24, 64, 128}; o is bf16 (o_f32 = 0) or fp32 (o_f32 = 1); merges with
// (merge_o, merge_lse) when they are set.
hipError_t launch_attn_fwd_bf16(const FwdArgs& a, int d, int o_f32, hipStream_t stream);
// fp32 operands and output on the vector ALU (the fp32 correctness path); d in {24, 64, 128}.
hipError_t launch_attn_fwd_f32(const FwdArgs& a, int d, hipStream_t stream);
// Short sequences (Nq, Nk <= kShortMax), bf16 in, bf16/fp32 out, d in {24, 64, 128}: one lane per query row,
// many (batch, head) slices per workgroup.
constexpr int kShortMax = 16;
hipError_t launch_attn_fwd_short(const FwdArgs& a, int d, int o_f32, hipStream_t stream);

// Arguments of one attention-backward call (both kernels). q, dout, dq: [BH, Nq, d]; k, v, dk, dv:
// [BH / kv_group, Nk, d]; o: [BH, Nq, d] (bf16, or fp32 when o_f32); lse, delta: [BH, Nq]. lse and o are the
// forward's results over the full key set; delta receives rowsum(dout * o). Masks as in FwdArgs.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int64_t BH;
  int Nq;
  int Nk;
  float scale;        // the softmax scale: the factor of dq and dk
  float scale_log2;   // scale * log2(e)
  int causal;
  int diag;
  int lo;
  int kv_group;
  int o_f32;          // o is fp32 (else bf16)
  int accumulate;     // add into dq, dk, dv instead of overwriting (fp32 gradients only)
};
// bf16 q, k, v, dout on MFMA; d in {24, 64, 128} (24 padded to 32); gradients fp32 (grad_f32 = 1) or bf16.
// The dq kernel (which also writes delta) runs first, then the dk/dv kernel, both on `stream`.
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int d, int grad_f32, hipStream_t stream);
// fp32 q, k, v, dout and o on the vector ALU (the fp32 correctness path); d in {24, 64, 128}; same order of
// kernels and same outputs as the bf16 path.
hipError_t launch_attn_bwd_f32(const BwdArgs& a, int d, int grad_f32, hipStream_t stream);

struct MergeArgs {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* o;
  float* lse;
  int64_t rows;
  int d;
};
// part_f32 / o_f32: 1 for fp32 tensors, 0 for bf16. d multiple of 4 (fp32 parts) or 8 (bf16 parts).
hipError_t launch_lse_merge(const MergeArgs& a, int part_f32, int o_f32, hipStream_t stream);
// Writes o = 0 (rows x d, bf16 or fp32) and lse = -inf (rows): the result for rows with no visible key.
hipError_t launch_fill_empty(void* o, float* lse, int64_t rows, int d, int o_f32, hipStream_t stream);

}  // namespace ebattn
