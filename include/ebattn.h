/* ebattn.h -- C ABI of the exact blockwise attention library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * Exact softmax attention, o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the keys j visible to query i, and
 * its per-row natural-log normaliser lse_i = log sum_j exp(scale * q_i . k_j):
 *   - the three-step definition of "深度学习注意力机制优化与FlashAttention实践" §2.1 (scores, softmax over keys,
 *     weighted sum of V), with the scale an explicit argument;
 *   - computed blockwise with an online softmax as in §4.2 of the same page (running maximum and running sum
 *     per query row, output rescaled whenever the maximum grows), which reaches the same result up to
 *     rounding ("架构层解决方案 - Sparse Attention与Ring Attention", Ring Attention / 核心创新);
 *   - partial results over disjoint key sets combine exactly with the log-sum-exp merge of
 *     "分布式注意力机制突破：长序列处理的全景技术架构与实践指南" §3.4 (and §2.2 stage 3, pairwise form with the
 *     sign of its exponent corrected);
 *   - ring_local is one device's share of Ring Attention ("Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈"
 *     §3.2): a resident query shard attended against a sequence of key/value blocks, merged as they come,
 *     ending with the complete output of that shard.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   Layout    q, k, v, o are contiguous [B, H, N, d] (row-major, d fastest; "BHSD"); lse is fp32 [B, H, Nq].
 *             lse is the natural log of the sum of exp(scale * q.k) over the visible keys (no bias).
 *   Pointers  q, k, v, o, lse, the merge operands and the workspace are DEVICE pointers owned by the caller;
 *             the library never frees or keeps them. Tensor pointers must be 16-byte aligned, lse pointers
 *             4-byte aligned. `stream` is a hipStream_t (NULL = the default stream).
 *   Masks     causal = 0: every key is visible. causal = 1: the mask is by GLOBAL POSITION. Local query row i
 *             sits at position q_off + i*pos_stride, local key j at k_off + j*pos_stride, and key j is visible
 *             to query i iff its position is <= the query's (inclusive diagonal, "深度学习注意力机制优化与
 *             FlashAttention实践" §5.1). pos_stride = 1 for contiguous shards; striping a sequence over W
 *             devices (token t on device t mod W, "注意力机制演进" timeline, Striped Attention) uses
 *             pos_stride = W, q_off = the query stripe, k_off = the key stripe.
 *   Empty rows A query row with no visible key gets o = 0 and lse = -inf (no epsilon anywhere); the merge
 *             gives such a part zero weight.
 *   Dtypes    ATTN_BF16 inputs run on bf16 MFMA with fp32 accumulation and fp32 softmax statistics
 *             ("深度学习注意力机制优化与FlashAttention实践" §5.1 advises fp32 for the statistics); the softmax
 *             weights P are rounded to bf16 before the P.V product, and o and lse are both normalised by the sum
 *             of the fp32 weights, so o carries the bf16 rounding of P: |o - exact| <= 2^-8 sum_j P_j |v_j|
 *             before the output's own rounding (each weight rounded to nearest with 8 significant bits).
 *             On the MFMA path the weights of a query block's later key tiles are taken against the largest score
 *             its first two tiles showed; a block whose later scores rise far enough above that to overflow
 *             fp32 (about 2^127 in weight) is computed a second time with the running maximum at every tile,
 *             so the bound above holds either way and only the time differs.
 *             ATTN_F32 inputs run in fp32 throughout.
 *   Asynchrony Every call only enqueues work on `stream`; nothing synchronises the device.
 *   Errors    Return ATTN_OK (0) or a negative code. Argument errors are detected before anything is
 *             launched; attn_last_error() then holds a message (thread-local). Launch failures return
 *             ATTN_EHIP with the HIP error string. Nothing throws across this boundary. On error the contents
 *             of the outputs are unspecified.
 */
#ifndef EBATTN_H
#define EBATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_EINVAL (-1)        /* bad argument: null pointer, negative size, bad flag, misalignment, overlap */
#define ATTN_EUNSUPPORTED (-2)  /* well-formed but not implemented: head dim, dtype combination */
#define ATTN_EHIP (-3)          /* the HIP runtime reported an error while launching */
#define ATTN_EWORKSPACE (-4)    /* ring_local: workspace missing or smaller than ring_local_workspace_bytes() */

#define ATTN_F32 0
#define ATTN_BF16 1

/* Largest sequence length (Nq, Nk) accepted by every entry point. */
#define ATTN_MAX_SEQ (1 << 28)

/* Most live incoming blocks ring_local_pipelined accepts in one call. */
#define ATTN_MAX_RING_BLOCKS 4096

/* attn_fwd -- exact attention of q [B,H,Nq,d] against k, v [B,H,Nk,d]; writes o [B,H,Nq,d] and lse [B,H,Nq].
 *   scale       softmax scale applied to q.k (workloads use 1/sqrt(d)); must be finite and > 0.
 *   causal      0 or 1, see "Masks"; q_off, k_off, pos_stride (>= 1) give the global positions.
 *   in_dtype    ATTN_BF16 (d in {24, 64, 128}) or ATTN_F32 (d in {24, 64, 128}).
 *   o_dtype     ATTN_BF16 or ATTN_F32 for bf16 inputs; ATTN_F32 for fp32 inputs.
 *   Sizes       B, H, Nq, Nk >= 0 (zero-sized calls are no-ops, except Nk = 0, which writes (0, -inf) rows);
 *               Nq, Nk <= ATTN_MAX_SEQ. k and v may be NULL when Nk = 0.
 *   Overlap     o and lse must not overlap q, k, v or each other.
 *   Sequences of at most 16 queries and 16 keys take a one-lane-per-row path (fp32 weights, no bf16 P). */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Nq, int Nk, int d, float scale, int causal,
             int64_t q_off, int64_t k_off, int pos_stride, int in_dtype, int o_dtype, void* stream);

/* attn_fwd_ex -- attn_fwd with two mask/indexing variants of "架构层解决方案 - Sparse Attention与Ring Attention":
 *   Hkv         key/value heads (section "MQA与GQA"): k and v are [B,Hkv,Nk,d], Hkv divides H, and query head h
 *               reads key/value head h / (H/Hkv), so consecutive query heads share one (Hkv = H: attn_fwd;
 *               Hkv = 1: multi-query attention).
 *   window      sliding window in positions (section "Sliding Window Attention": each token attends only to the
 *               w most recent tokens): 0 = none; w > 0 keeps key j for query i iff
 *               q_pos - w < k_pos <= q_pos (the query's own position included) and requires causal = 1.
 *   Everything else, errors included, as attn_fwd; attn_fwd(...) equals attn_fwd_ex(..., Hkv = H, window = 0).
 *   Additional errors: ATTN_EINVAL if Hkv does not divide H, window < 0, or window > 0 without causal. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                int64_t q_off, int64_t k_off, int pos_stride, int64_t window, int in_dtype, int o_dtype,
                void* stream);

/* attn_fwd_merge -- attention of one key/value block merged into a running result in the same kernel: the
 * "accumulate each received block" step of "Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈" §3.2, with the
 * log-sum-exp merge of "分布式注意力机制突破：长序列处理的全景技术架构与实践指南" §3.4 done in the attention
 * kernel's epilogue (no partial result in memory, no separate merge pass).
 *   (o, lse) = merge((run_o, run_lse), attn_fwd_ex(q, k, v, ...)), i.e. lse = log(exp(run_lse) + exp(lse_blk)),
 *   o = exp(run_lse - lse) * run_o + exp(lse_blk - lse) * o_blk; a part with lse = -inf weighs zero.
 *   run_o       fp32 [B,H,Nq,d] and run_lse fp32 [B,H,Nq]: the running result over other keys (device pointers).
 *   In place    o may be exactly run_o (o_dtype ATTN_F32) and lse exactly run_lse; any other overlap of o, lse,
 *               run_o, run_lse, q, k, v is ATTN_EINVAL.
 *   in_dtype    ATTN_BF16 only (ATTN_EUNSUPPORTED otherwise); d in {24, 64, 128}.
 *   A block that hides every key (or Nk = 0) leaves the running result unchanged (copied to o, lse).
 *   Everything else, errors included, as attn_fwd_ex. */
int attn_fwd_merge(const void* q, const void* k, const void* v, const float* run_o, const float* run_lse,
                   void* o, float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int64_t q_off, int64_t k_off, int pos_stride, int64_t window, int in_dtype, int o_dtype,
                   void* stream);

/* attn_bwd -- gradients of exact attention (the backward pass of attn_fwd_ex), with the attention weights
 * recomputed tile by tile from the saved lse instead of stored ("深度学习注意力机制优化与FlashAttention实践"
 * §4.1 item 3 and §3.3). For an output gradient dout = dL/do:
 *   P_ij = exp(scale q_i.k_j - lse_i) on visible pairs (0 elsewhere), delta_i = dout_i . o_i,
 *   dv_j = sum_i P_ij dout_i,  ds_ij = P_ij (dout_i . v_j - delta_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 * summed over the query heads of a group for a shared key/value head. These are the exact gradients of the
 * forward when lse and o are the forward's results over the same keys. When k, v are one block of a larger key
 * set (a ring share), pass the lse and o of the FULL key set: the returned dq is then that block's contribution
 * (dq over the full set is the sum over the blocks; see `accumulate`), and dk, dv are exact for the block's keys.
 *   q, dout      [B,H,Nq,d]; k, v [B,Hkv,Nk,d] (Hkv divides H, as attn_fwd_ex), all in in_dtype.
 *   o            [B,H,Nq,d] in o_dtype (ATTN_BF16 or ATTN_F32); lse fp32 [B,H,Nq] (-inf rows contribute nothing).
 *   dq           [B,H,Nq,d], dk, dv [B,Hkv,Nk,d], in grad_dtype (ATTN_F32 or ATTN_BF16); written.
 *   delta        fp32 [B,H,Nq], written with rowsum(dout * o) (a per-row value the caller may reuse).
 *   accumulate   0: overwrite dq, dk, dv; 1: add into them (ATTN_F32 gradients only).
 *   in_dtype     ATTN_BF16 (MFMA) or ATTN_F32 (vector ALU, the fp32 correctness path; o must then be ATTN_F32 and
 *                q, k, v, dout fp32); d in {24, 64, 128} (ATTN_EUNSUPPORTED otherwise).
 *   Masks, offsets, window, scale, stream: as attn_fwd_ex.
 *   Sizes        B, H, Hkv, Nq, Nk >= 0; Nq = 0 writes zero dk, dv (or leaves them, with accumulate); Nk = 0 or
 *                a mask that hides every key writes zero dq; pointers of zero-sized tensors may be NULL.
 *   Overlap      dq, dk, dv and delta must not overlap each other or any input (ATTN_EINVAL).
 *   Numerics     bf16 inputs: bf16 MFMA products with fp32 accumulation, P rounded to bf16 for dv and ds to
 *                bf16 for dq and dk; fp32 inputs: fp32 throughout. lse, delta and the exponentials are fp32.
 *   Two kernels run in order on `stream`: dq (which also writes delta), then dk and dv. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* delta,
             int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
             int64_t q_off, int64_t k_off, int pos_stride, int64_t window,
             int in_dtype, int o_dtype, int grad_dtype, int accumulate, void* stream);

/* attn_lse_merge -- merges two partial results over disjoint key sets of the same query rows:
 *   lse = log(exp(lse_a) + exp(lse_b)),  o = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b.
 *   Operands are `rows` rows of d values (any [.., rows, d] contiguous layout; for attention rows = B*H*Nq).
 *   part_dtype  dtype of o_a and o_b (ATTN_F32: d a multiple of 4, <= 256; ATTN_BF16: multiple of 8, <= 512).
 *   o_dtype     dtype of o. lse_* and lse are fp32.
 *   In place    o may be exactly o_a or o_b when o_dtype == part_dtype, and lse may be exactly lse_a or lse_b;
 *               any other overlap is ATTN_EINVAL.
 *   Empty       a part with lse = -inf weighs zero; two empty parts give (0, -inf). rows = 0 is a no-op. */
int attn_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                   void* o, float* lse, int64_t rows, int d, int part_dtype, int o_dtype, void* stream);

/* One key/value block of a ring: k, v [B,H,Nk,d] (same B, H, d and dtype as the query shard), and the global
 * position of its first key (positions advance by pos_stride per key, as for attn_fwd). */
typedef struct {
  const void* k;
  const void* v;
  int Nk;
  int64_t k_off;
} attn_kv_block;

/* ring_local -- one device's share of Ring Attention: q_shard [B,H,Nq,d] against kv_blocks[0..n_blocks-1],
 * processed in the given order (the order the blocks would arrive around the ring). Blocks that hide every
 * key from every query row (causal) are skipped without a launch. The first live block's attention goes to
 * the fp32 accumulator in the workspace. With bf16 inputs every later block is merged into that accumulator
 * inside its attention kernel (as attn_fwd_merge), the last one writing o (o_dtype) and lse; with fp32 inputs
 * every later block goes to a second fp32 partial in the workspace that attn_lse_merge folds into the
 * accumulator, the last merge writing o and lse. A single live block writes o and lse directly; no live block
 * writes (0, -inf) rows. The result equals attention over the union of the blocks.
 *   workspace   device buffer of at least ring_local_workspace_bytes(B, H, Nq, d) bytes, 256-byte aligned,
 *               not overlapping anything else; may be NULL only if at most one block is live.
 *   Other arguments as attn_fwd. */
int ring_local(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse,
               int B, int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride,
               int in_dtype, int o_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace ring_local needs: two fp32 (o, lse) buffers of B*H*Nq rows, each 256-byte aligned (the
 * second is used with fp32 inputs only). Returns 0 for negative sizes. */
size_t ring_local_workspace_bytes(int B, int H, int Nq, int d);

/* Size of the per-GPU scratch array behind ring_local_noalloc: 256 MiB, enough for the fp32 accumulator of a
 * share of up to about 500 thousand query rows (B*H*Nq) at d = 128 with bf16 inputs, half that with fp32 inputs. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* ring_local_noalloc -- ring_local for callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same computation, kernels and results as ring_local, with
 * the workspace taken from a scratch array that the library holds in each GPU's memory (ATTN_NOALLOC_SCRATCH_BYTES,
 * reserved on a GPU while its code object is loaded, until the process ends) instead of a caller's buffer. The
 * call allocates nothing: no hipMalloc, no hipFree, no library routine that allocates. Its first call on a device
 * looks the array's device address up on the current device, which must be the device of q_shard, o, lse, the
 * blocks and `stream`.
 *   Scratch     a share needs B*H*Nq*(d + 1)*4 bytes (each part rounded up to 256 bytes), twice that with fp32
 *               inputs; more than ATTN_NOALLOC_SCRATCH_BYTES returns ATTN_EWORKSPACE before anything is launched.
 *               Nothing in the array needs to start at any value: every call writes its accumulator before reading
 *               it, and the array keeps the last call's contents.
 *   Concurrency every call on one GPU uses that GPU's single array: calls whose work overlaps on the device (on
 *               different streams, or from different threads without ordering) race and give wrong results. Calls
 *               enqueued on one stream are ordered and safe.
 *   Arguments, masks, dtypes and errors otherwise as ring_local. */
int ring_local_noalloc(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse,
                       int B, int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride,
                       int in_dtype, int o_dtype, void* stream);

/* ring_local_pipelined -- ring_local with the exchange step of the ring on the same device: compute on the block
 * in hand while the next one arrives ("架构层解决方案 - Sparse Attention与Ring Attention", Ring Attention /
 * 计算-通信重叠; "Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈" §3.2). kv_blocks[0] is this device's own
 * block and is read in place; every later block is an incoming one: it is copied (hipMemcpyAsync on
 * copy_stream) into one of two receive slots in the workspace while compute_stream attends the block before it,
 * and merged into the running result in the attention kernel's epilogue (as attn_fwd_merge). Events order the
 * two streams: a block is attended only once it has landed, and a slot is refilled only once the block in it
 * has been attended. Incoming blocks may live in any memory hipMemcpyAsync reads (pinned host memory stands in
 * for the link to the neighbouring device, device memory for a block already received).
 *   Inputs      bf16 only (in_dtype is ATTN_BF16); blocks that hide every key are neither copied nor attended.
 *   Streams     compute_stream receives the attention launches and, at the end, holds the result. The first
 *               copy waits for everything enqueued on compute_stream before the call (an incoming block produced
 *               there, an earlier call still reading the same workspace); every copy is waited for by a launch on
 *               compute_stream, so synchronising compute_stream is enough.
 *               Both are hipStream_t (NULL = the default stream), both of default priority, both on the
 *               current device (the call creates its ordering events there).
 *   workspace   at least ring_local_pipelined_workspace_bytes(B, H, Nq, d, Nk_max) bytes (Nk_max = the largest
 *               incoming block), 256-byte aligned, overlapping nothing else; it must stay untouched until
 *               compute_stream has passed this call's work. May be NULL only when block 0 is the only live one.
 *   Host blocks incoming blocks in host memory are read by the copy engines after the call returns: they must
 *               stay allocated and unchanged until compute_stream has passed this call's work.
 *   Errors      as ring_local; ATTN_EINVAL for more than ATTN_MAX_RING_BLOCKS live incoming blocks.
 *   The result equals ring_local over the same blocks. */
int ring_local_pipelined(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse,
                         int B, int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride,
                         int o_dtype, void* workspace, size_t workspace_bytes, void* compute_stream,
                         void* copy_stream);

/* Bytes of workspace ring_local_pipelined needs: the fp32 (o, lse) accumulator of B*H*Nq rows and two receive
 * slots of bf16 K and V blocks of B*H*Nk_max rows, each buffer 256-byte aligned. Returns 0 for negative sizes. */
size_t ring_local_pipelined_workspace_bytes(int B, int H, int Nq, int d, int Nk_max);

/* ring_local_plan -- host-only classification of each block, exactly as ring_local decides it (no device
 * work). kinds[i] = 0: every key hidden from every row (skipped); 1: every key visible to every row;
 * 2: partly visible. Returns the number of live (kind != 0) blocks, or a negative error code. */
int ring_local_plan(const attn_kv_block* kv_blocks, int n_blocks, int Nq, int causal, int64_t q_off,
                    int pos_stride, int* kinds);

/* Message describing the last error returned on the calling thread ("" if none). Owned by the library. */
const char* attn_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EBATTN_H */
