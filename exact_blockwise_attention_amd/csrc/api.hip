// C ABI of the library: argument validation, mask-to-diagonal reduction, kernel dispatch and the ring_local
// driver. Every check runs on the host before the first HIP call, so argument errors never touch the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/ebattn.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

int64_t elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool dtype_ok(int t) { return t == ATTN_F32 || t == ATTN_BF16; }
bool head_dim_ok(int d) { return d == 24 || d == 64 || d == 128; }

// floor(num / s), clamped to [-2^29, 2^29] so that every int32 expression in the kernels stays in range; with
// Nq, Nk <= 2^28 the clamp never changes which keys are visible. num is formed in 128 bits: offsets and windows
// of up to 2^62 in magnitude would overflow 64.
int floor_div_clamped(__int128 num, int s) {
  __int128 dq = num / s;
  if ((num % s != 0) && (num < 0)) dq -= 1;
  const __int128 lim = (__int128)1 << 29;
  if (dq > lim) dq = lim;
  if (dq < -lim) dq = -lim;
  return (int)dq;
}

// "key j visible to query i" <=> k_off + j*s <= q_off + i*s <=> j <= i + floor((q_off - k_off) / s).
int diag_offset(int64_t q_off, int64_t k_off, int s) { return floor_div_clamped((__int128)q_off - k_off, s); }

// With a sliding window of w positions, key j is also required to satisfy k_off + j*s > q_off + i*s - w, i.e.
// j >= i + floor((q_off - k_off - w) / s) + 1.
int window_lo(int64_t q_off, int64_t k_off, int s, int64_t window) {
  if (window <= 0) return ebattn::kNoWindow;
  return floor_div_clamped((__int128)q_off - k_off - window, s) + 1;
}

const int64_t kOffLimit = (int64_t)1 << 62;

// Common validation of a query-side call. Returns ATTN_OK or an error code (message set).
int check_query_side(const void* q, const void* o, const float* lse, int B, int H, int Nq, int d, float scale,
                     int causal, int64_t q_off, int pos_stride, int in_dtype, int o_dtype) {
  if (B < 0 || H < 0 || Nq < 0) return fail(ATTN_EINVAL, "negative size (B=%d H=%d Nq=%d)", B, H, Nq);
  if (Nq > ATTN_MAX_SEQ) return fail(ATTN_EINVAL, "Nq=%d exceeds ATTN_MAX_SEQ", Nq);
  if (!(causal == 0 || causal == 1)) return fail(ATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (pos_stride < 1) return fail(ATTN_EINVAL, "pos_stride must be >= 1 (got %d)", pos_stride);
  if (!(scale > 0.0f) || !isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite and > 0");
  if (q_off > kOffLimit || q_off < -kOffLimit) return fail(ATTN_EINVAL, "q_off out of range");
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype)) return fail(ATTN_EINVAL, "unknown dtype code");
  if (in_dtype == ATTN_F32 && o_dtype != ATTN_F32)
    return fail(ATTN_EUNSUPPORTED, "fp32 inputs require an fp32 output");
  if (!head_dim_ok(d)) return fail(ATTN_EUNSUPPORTED, "head dim d=%d not supported (24, 64, 128)", d);
  const int64_t rows = (int64_t)B * H * Nq;
  if (rows == 0) return ATTN_OK;
  if (!q || !o || !lse) return fail(ATTN_EINVAL, "null q, o or lse pointer");
  if (!aligned(q, 16) || !aligned(o, 16)) return fail(ATTN_EINVAL, "q and o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_EINVAL, "lse must be 4-byte aligned");
  return ATTN_OK;
}

// BH: key/value slices (B * Hkv); BHq: query slices (B * H), which size o and lse.
int check_kv(const void* k, const void* v, int64_t BH, int Nk, int d, int in_dtype, int64_t k_off,
             const void* q, const void* o, const float* lse, int64_t Nq, int o_dtype, int64_t BHq) {
  if (Nk < 0) return fail(ATTN_EINVAL, "negative Nk=%d", Nk);
  if (Nk > ATTN_MAX_SEQ) return fail(ATTN_EINVAL, "Nk=%d exceeds ATTN_MAX_SEQ", Nk);
  if (k_off > kOffLimit || k_off < -kOffLimit) return fail(ATTN_EINVAL, "k_off out of range");
  if (Nk == 0 || BH == 0) return ATTN_OK;
  if (!k || !v) return fail(ATTN_EINVAL, "null k or v pointer");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(ATTN_EINVAL, "k and v must be 16-byte aligned");
  const int64_t kvb = BH * Nk * d * elem_bytes(in_dtype);
  const Span so = span(o, BHq * Nq * d * elem_bytes(o_dtype)), sl = span(lse, BHq * Nq * 4);
  if (overlap(so, span(k, kvb)) || overlap(so, span(v, kvb)) || overlap(sl, span(k, kvb)) ||
      overlap(sl, span(v, kvb)))
    return fail(ATTN_EINVAL, "o/lse overlap k or v");
  (void)q;
  return ATTN_OK;
}

int check_outputs_disjoint(const void* q, const void* o, const float* lse, int64_t rows, int d, int in_dtype,
                           int o_dtype) {
  const Span sq = span(q, rows * d * elem_bytes(in_dtype));
  const Span so = span(o, rows * d * elem_bytes(o_dtype));
  const Span sl = span(lse, rows * 4);
  if (overlap(so, sq) || overlap(sl, sq) || overlap(so, sl)) return fail(ATTN_EINVAL, "o/lse overlap q or each other");
  return ATTN_OK;
}

// Enqueue one attention forward whose arguments have been validated.
// With merge_o / merge_lse set (bf16 inputs only), the result is merged in the kernel's epilogue with that
// running fp32 result; o / lse may be exactly merge_o / merge_lse. Such a launch always runs the MFMA kernel (it
// also covers blocks that hide every key: their rows keep the running result).
int enqueue_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int Nq, int Nk,
                int d, float scale, int causal, int diag, int in_dtype, int o_dtype, hipStream_t stream,
                int lo = ebattn::kNoWindow, int kv_group = 1, const float* merge_o = nullptr,
                const float* merge_lse = nullptr) {
  const int64_t rows = BH * Nq;
  if (rows == 0) return ATTN_OK;
  const bool merging = merge_o != nullptr;
  const bool all_hidden = !merging && ((Nk == 0) || (causal && (int64_t)Nq - 1 + diag < 0));
  hipError_t e;
  if (all_hidden) {
    e = ebattn::launch_fill_empty(o, lse, rows, d, o_dtype == ATTN_F32, stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill launch");
  }
  ebattn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  // a causal mask under which even the first query row sees every key (and the last row's window reaches back
  // to key 0) hides nothing: run the unmasked kernel
  const bool masks = causal && ((int64_t)diag < (int64_t)Nk - 1 || (int64_t)Nq - 1 + lo > 0);
  a.causal = masks ? 1 : 0;
  a.diag = masks ? diag : 0;
  a.lo = masks ? lo : ebattn::kNoWindow;
  a.kv_group = kv_group;
  a.merge_o = merge_o;
  a.merge_lse = merge_lse;
  if (merging)
    e = ebattn::launch_attn_fwd_bf16(a, d, o_dtype == ATTN_F32, stream);
  else if (in_dtype == ATTN_F32)
    e = ebattn::launch_attn_fwd_f32(a, d, stream);
  else if (Nq <= ebattn::kShortMax && Nk <= ebattn::kShortMax)
    e = ebattn::launch_attn_fwd_short(a, d, o_dtype == ATTN_F32, stream);
  else
    e = ebattn::launch_attn_fwd_bf16(a, d, o_dtype == ATTN_F32, stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attention launch");
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int classify(int Nq, int Nk, int causal, int64_t q_off, int64_t k_off, int s) {
  if (Nk <= 0 || Nq <= 0) return 0;
  if (!causal) return 1;
  const int diag = diag_offset(q_off, k_off, s);
  if ((int64_t)Nq - 1 + diag < 0) return 0;   // even the last query row sees no key
  if ((int64_t)diag >= (int64_t)Nk - 1) return 1;  // even the first query row sees every key
  return 2;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

int attn_version(void) { return 100; }

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int Nq,
                int Nk, int d, float scale, int causal, int64_t q_off, int64_t k_off, int pos_stride, int64_t window,
                int in_dtype, int o_dtype, void* stream) {
  g_err[0] = '\0';
  int rc = check_query_side(q, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_EINVAL, "Hkv=%d must divide H=%d", Hkv, H);
  if (window < 0) return fail(ATTN_EINVAL, "window must be >= 0 (got %lld)", (long long)window);
  if (window > 0 && !causal) return fail(ATTN_EINVAL, "a sliding window requires causal = 1");
  if (window > kOffLimit) return fail(ATTN_EINVAL, "window out of range");
  const int64_t BH = (int64_t)B * H;
  const int group = H > 0 ? H / Hkv : 1;
  rc = check_kv(k, v, (int64_t)B * (H > 0 ? Hkv : 0), Nk, d, in_dtype, k_off, q, o, lse, Nq, o_dtype, BH);
  if (rc != ATTN_OK) return rc;
  if (BH * Nq == 0) return ATTN_OK;
  rc = check_outputs_disjoint(q, o, lse, BH * Nq, d, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;
  (void)hipGetLastError();  // drop a stale error so a failure below is attributed to this call
  return enqueue_fwd(q, k, v, o, lse, BH, Nq, Nk, d, scale, causal, diag_offset(q_off, k_off, pos_stride),
                     in_dtype, o_dtype, reinterpret_cast<hipStream_t>(stream),
                     window_lo(q_off, k_off, pos_stride, window), group);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
             float scale, int causal, int64_t q_off, int64_t k_off, int pos_stride, int in_dtype, int o_dtype,
             void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, H, Nq, Nk, d, scale, causal, q_off, k_off, pos_stride, 0, in_dtype,
                     o_dtype, stream);
}

int attn_fwd_merge(const void* q, const void* k, const void* v, const float* run_o, const float* run_lse, void* o,
                   float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int64_t q_off,
                   int64_t k_off, int pos_stride, int64_t window, int in_dtype, int o_dtype, void* stream) {
  g_err[0] = '\0';
  int rc = check_query_side(q, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;
  if (in_dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "attn_fwd_merge takes bf16 q, k, v");
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0))
    return fail(ATTN_EINVAL, "Hkv=%d must divide H=%d", Hkv, H);
  if (window < 0) return fail(ATTN_EINVAL, "window must be >= 0 (got %lld)", (long long)window);
  if (window > 0 && !causal) return fail(ATTN_EINVAL, "a sliding window requires causal = 1");
  if (window > kOffLimit) return fail(ATTN_EINVAL, "window out of range");
  const int64_t BH = (int64_t)B * H;
  const int64_t rows = BH * Nq;
  rc = check_kv(k, v, (int64_t)B * (H > 0 ? Hkv : 0), Nk, d, in_dtype, k_off, q, o, lse, Nq, o_dtype, BH);
  if (rc != ATTN_OK) return rc;
  if (rows == 0) return ATTN_OK;
  if (!run_o || !run_lse) return fail(ATTN_EINVAL, "null run_o or run_lse");
  if (!aligned(run_o, 16) || !aligned(run_lse, 4)) return fail(ATTN_EINVAL, "run_o / run_lse misaligned");
  rc = check_outputs_disjoint(q, o, lse, rows, d, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;
  // o may be exactly run_o (fp32 output), lse exactly run_lse; any other overlap is an error
  const Span sro = span(run_o, rows * d * 4), srl = span(run_lse, rows * 4);
  const Span so = span(o, rows * d * elem_bytes(o_dtype)), sl = span(lse, rows * 4);
  const bool o_in_place = (o == (const void*)run_o) && o_dtype == ATTN_F32;
  const bool l_in_place = (lse == run_lse);
  if ((!o_in_place && overlap(so, sro)) || (!l_in_place && overlap(sl, srl)) || overlap(so, srl) ||
      overlap(sl, sro) || overlap(sro, srl))
    return fail(ATTN_EINVAL, "o / lse overlap run_o / run_lse other than exactly in place");
  const int64_t qb = rows * d * 2, kvb = (int64_t)B * (H > 0 ? Hkv : 0) * Nk * d * 2;
  if (overlap(sro, span(q, qb)) || overlap(srl, span(q, qb)) ||
      (Nk > 0 && (overlap(sro, span(k, kvb)) || overlap(sro, span(v, kvb)) || overlap(srl, span(k, kvb)) ||
                  overlap(srl, span(v, kvb)))))
    return fail(ATTN_EINVAL, "run_o / run_lse overlap q, k or v");
  (void)hipGetLastError();
  return enqueue_fwd(q, k, v, o, lse, BH, Nq, Nk, d, scale, causal, diag_offset(q_off, k_off, pos_stride), in_dtype,
                     o_dtype, reinterpret_cast<hipStream_t>(stream), window_lo(q_off, k_off, pos_stride, window),
                     H > 0 ? H / Hkv : 1, run_o, run_lse);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, float* delta, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
             int64_t q_off, int64_t k_off, int pos_stride, int64_t window, int in_dtype, int o_dtype, int grad_dtype,
             int accumulate, void* stream) {
  g_err[0] = '\0';
  if (B < 0 || H < 0 || Hkv < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_EINVAL, "negative size (B=%d H=%d Hkv=%d Nq=%d Nk=%d)", B, H, Hkv, Nq, Nk);
  if (Nq > ATTN_MAX_SEQ || Nk > ATTN_MAX_SEQ) return fail(ATTN_EINVAL, "Nq or Nk exceeds ATTN_MAX_SEQ");
  if (H > 0 && (Hkv < 1 || Hkv > H || H % Hkv != 0)) return fail(ATTN_EINVAL, "Hkv=%d must divide H=%d", Hkv, H);
  if (!(causal == 0 || causal == 1)) return fail(ATTN_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (!(accumulate == 0 || accumulate == 1)) return fail(ATTN_EINVAL, "accumulate must be 0 or 1");
  if (pos_stride < 1) return fail(ATTN_EINVAL, "pos_stride must be >= 1 (got %d)", pos_stride);
  if (!(scale > 0.0f) || !isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite and > 0");
  if (q_off > kOffLimit || q_off < -kOffLimit || k_off > kOffLimit || k_off < -kOffLimit)
    return fail(ATTN_EINVAL, "q_off or k_off out of range");
  if (window < 0 || window > kOffLimit) return fail(ATTN_EINVAL, "window out of range (got %lld)", (long long)window);
  if (window > 0 && !causal) return fail(ATTN_EINVAL, "a sliding window requires causal = 1");
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype) || !dtype_ok(grad_dtype)) return fail(ATTN_EINVAL, "unknown dtype code");
  if (in_dtype == ATTN_F32 && o_dtype != ATTN_F32) return fail(ATTN_EINVAL, "fp32 inputs come with an fp32 o");
  if (accumulate && grad_dtype != ATTN_F32) return fail(ATTN_EINVAL, "accumulate requires fp32 gradients");
  if (!head_dim_ok(d)) return fail(ATTN_EUNSUPPORTED, "head dim d=%d not supported by the backward (24, 64, 128)", d);
  const int64_t BH = (int64_t)B * H, BHkv = (int64_t)B * (H > 0 ? Hkv : 0);
  const int64_t qrows = BH * Nq, krows = BHkv * Nk;
  if (qrows == 0 && krows == 0) return ATTN_OK;
  if (qrows > 0) {
    if (!q || !o || !lse || !dout || !dq || !delta) return fail(ATTN_EINVAL, "null q, o, lse, dout, dq or delta");
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16))
      return fail(ATTN_EINVAL, "q, o, dout and dq must be 16-byte aligned");
    if (!aligned(lse, 4) || !aligned(delta, 4)) return fail(ATTN_EINVAL, "lse and delta must be 4-byte aligned");
  }
  if (krows > 0) {
    if (!k || !v || !dk || !dv) return fail(ATTN_EINVAL, "null k, v, dk or dv");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))
      return fail(ATTN_EINVAL, "k, v, dk and dv must be 16-byte aligned");
  }
  // the four outputs must not overlap each other or any input
  const int64_t gb = elem_bytes(grad_dtype), ib = elem_bytes(in_dtype);
  const Span outs[4] = {span(dq, qrows * d * gb), span(dk, krows * d * gb), span(dv, krows * d * gb),
                        span(delta, qrows * 4)};
  const Span ins[6] = {span(q, qrows * d * ib), span(k, krows * d * ib), span(v, krows * d * ib),
                       span(o, qrows * d * elem_bytes(o_dtype)), span(lse, qrows * 4), span(dout, qrows * d * ib)};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(ATTN_EINVAL, "dq, dk, dv and delta must not overlap");
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], ins[j])) return fail(ATTN_EINVAL, "an output (dq, dk, dv, delta) overlaps an input");
  }
  const int diag = diag_offset(q_off, k_off, pos_stride);
  const int lo = window_lo(q_off, k_off, pos_stride, window);
  const bool masks = causal && ((int64_t)diag < (int64_t)Nk - 1 || (int64_t)Nq - 1 + lo > 0);
  ebattn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.causal = masks ? 1 : 0;
  a.diag = masks ? diag : 0;
  a.lo = masks ? lo : ebattn::kNoWindow;
  a.kv_group = H > 0 ? H / Hkv : 1;
  a.o_f32 = o_dtype == ATTN_F32;
  a.accumulate = accumulate;
  (void)hipGetLastError();  // drop a stale error so a failure below is attributed to this call
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = in_dtype == ATTN_F32 ? ebattn::launch_attn_bwd_f32(a, d, grad_dtype == ATTN_F32, st)
                                            : ebattn::launch_attn_bwd_bf16(a, d, grad_dtype == ATTN_F32, st);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "backward launch");
}

int attn_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                   int64_t rows, int d, int part_dtype, int o_dtype, void* stream) {
  g_err[0] = '\0';
  if (rows < 0) return fail(ATTN_EINVAL, "negative rows");
  if (d <= 0) return fail(ATTN_EINVAL, "d must be > 0");
  if (!dtype_ok(part_dtype) || !dtype_ok(o_dtype)) return fail(ATTN_EINVAL, "unknown dtype code");
  const int vec = part_dtype == ATTN_F32 ? 4 : 8;
  if (d % vec != 0 || d > 64 * vec)
    return fail(ATTN_EUNSUPPORTED, "d=%d must be a multiple of %d and at most %d", d, vec, 64 * vec);
  if (rows == 0) return ATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return fail(ATTN_EINVAL, "null pointer");
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16)) return fail(ATTN_EINVAL, "o_a, o_b, o not 16-byte aligned");
  if (!aligned(lse_a, 4) || !aligned(lse_b, 4) || !aligned(lse, 4)) return fail(ATTN_EINVAL, "lse not 4-byte aligned");
  const int64_t pb = rows * d * elem_bytes(part_dtype), ob = rows * d * elem_bytes(o_dtype), lb = rows * 4;
  const Span sa = span(o_a, pb), sb = span(o_b, pb), so = span(o, ob);
  const Span sla = span(lse_a, lb), slb = span(lse_b, lb), sl = span(lse, lb);
  const bool o_in_place = (o == o_a || o == o_b) && o_dtype == part_dtype;
  if (!o_in_place && (overlap(so, sa) || overlap(so, sb)))
    return fail(ATTN_EINVAL, "o overlaps o_a/o_b without being exactly one of them (same dtype)");
  if (o == o_a && o == o_b) return fail(ATTN_EINVAL, "o_a and o_b are the same buffer as o");
  const bool l_in_place = (lse == lse_a || lse == lse_b);
  if (!l_in_place && (overlap(sl, sla) || overlap(sl, slb)))
    return fail(ATTN_EINVAL, "lse overlaps lse_a/lse_b without being exactly one of them");
  if (overlap(so, sl) || overlap(so, sla) || overlap(so, slb) || overlap(sl, sa) || overlap(sl, sb))
    return fail(ATTN_EINVAL, "an output overlaps a buffer of the other kind");
  ebattn::MergeArgs a;
  a.o_a = o_a;
  a.lse_a = lse_a;
  a.o_b = o_b;
  a.lse_b = lse_b;
  a.o = o;
  a.lse = lse;
  a.rows = rows;
  a.d = d;
  (void)hipGetLastError();
  const hipError_t e = ebattn::launch_lse_merge(a, part_dtype == ATTN_F32, o_dtype == ATTN_F32,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "merge launch");
}

size_t ring_local_workspace_bytes(int B, int H, int Nq, int d) {
  if (B < 0 || H < 0 || Nq < 0 || d < 0) return 0;
  const size_t rows = (size_t)B * H * Nq;
  return 2 * (align256(rows * d * 4) + align256(rows * 4));
}

int ring_local_plan(const attn_kv_block* kv_blocks, int n_blocks, int Nq, int causal, int64_t q_off, int pos_stride,
                    int* kinds) {
  g_err[0] = '\0';
  if (n_blocks < 0) return fail(ATTN_EINVAL, "negative n_blocks");
  if (n_blocks > 0 && (!kv_blocks || !kinds)) return fail(ATTN_EINVAL, "null kv_blocks or kinds");
  if (Nq < 0) return fail(ATTN_EINVAL, "negative Nq");
  if (!(causal == 0 || causal == 1)) return fail(ATTN_EINVAL, "causal must be 0 or 1");
  if (pos_stride < 1) return fail(ATTN_EINVAL, "pos_stride must be >= 1");
  if (q_off > kOffLimit || q_off < -kOffLimit) return fail(ATTN_EINVAL, "q_off out of range");
  int live = 0;
  for (int i = 0; i < n_blocks; ++i) {
    const attn_kv_block& b = kv_blocks[i];
    if (b.Nk < 0 || b.Nk > ATTN_MAX_SEQ) return fail(ATTN_EINVAL, "block %d: bad Nk=%d", i, b.Nk);
    if (b.k_off > kOffLimit || b.k_off < -kOffLimit) return fail(ATTN_EINVAL, "block %d: k_off out of range", i);
    kinds[i] = classify(Nq, b.Nk, causal, q_off, b.k_off, pos_stride);
    live += kinds[i] != 0;
  }
  return live;
}

}  // extern "C"

namespace {

// Workspace ring_local actually touches: the fp32 accumulator (o, lse), plus the fp32 partial for fp32 inputs
// (bf16 inputs merge in the attention epilogue and need no partial).
size_t ring_local_bytes_used(int B, int H, int Nq, int d, int in_dtype) {
  const size_t rows = (size_t)B * H * Nq;
  const size_t one = align256(rows * d * 4) + align256(rows * 4);
  return in_dtype == ATTN_F32 ? 2 * one : one;
}

// ring_local with the workspace requirement given by the caller (`need` bytes when two or more blocks are live).
int ring_local_run(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse, int B,
                   int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride, int in_dtype,
                   int o_dtype, void* workspace, size_t workspace_bytes, size_t need, void* stream) {
  int rc = check_query_side(q_shard, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;
  if (n_blocks < 0) return fail(ATTN_EINVAL, "negative n_blocks");
  if (n_blocks > 0 && !kv_blocks) return fail(ATTN_EINVAL, "null kv_blocks");
  const int64_t BH = (int64_t)B * H;
  const int64_t rows = BH * Nq;
  for (int i = 0; i < n_blocks; ++i) {
    rc = check_kv(kv_blocks[i].k, kv_blocks[i].v, BH, kv_blocks[i].Nk, d, in_dtype, kv_blocks[i].k_off, q_shard, o,
                  lse, Nq, o_dtype, BH);
    if (rc != ATTN_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "block %d: %s", i, g_err);
      return fail(rc, "%s", msg);
    }
  }
  if (rows == 0) return ATTN_OK;
  rc = check_outputs_disjoint(q_shard, o, lse, rows, d, in_dtype, o_dtype);
  if (rc != ATTN_OK) return rc;

  // Host plan: which blocks can contribute at all.
  int live = 0;
  for (int i = 0; i < n_blocks; ++i)
    live += classify(Nq, kv_blocks[i].Nk, causal, q_off, kv_blocks[i].k_off, pos_stride) != 0;

  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (live >= 2) {
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
    const Span sw = span(workspace, (int64_t)need);
    if (overlap(sw, span(o, rows * d * elem_bytes(o_dtype))) || overlap(sw, span(lse, rows * 4)) ||
        overlap(sw, span(q_shard, rows * d * elem_bytes(in_dtype))))
      return fail(ATTN_EINVAL, "workspace overlaps q, o or lse");
    for (int i = 0; i < n_blocks; ++i) {
      const int64_t kvb = BH * kv_blocks[i].Nk * d * elem_bytes(in_dtype);
      if (kv_blocks[i].Nk > 0 && (overlap(sw, span(kv_blocks[i].k, kvb)) || overlap(sw, span(kv_blocks[i].v, kvb))))
        return fail(ATTN_EINVAL, "workspace overlaps block %d", i);
    }
  }
  (void)hipGetLastError();  // drop a stale error so a failure below is attributed to this call
  if (live == 0) {
    const hipError_t e = ebattn::launch_fill_empty(o, lse, rows, d, o_dtype == ATTN_F32, st);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill launch");
  }
  if (live == 1) {
    for (int i = 0; i < n_blocks; ++i) {
      const attn_kv_block& b = kv_blocks[i];
      if (classify(Nq, b.Nk, causal, q_off, b.k_off, pos_stride) == 0) continue;
      return enqueue_fwd(q_shard, b.k, b.v, o, lse, BH, Nq, b.Nk, d, scale, causal,
                         diag_offset(q_off, b.k_off, pos_stride), in_dtype, o_dtype, st);
    }
  }

  char* ws = reinterpret_cast<char*>(workspace);
  float* acc_o = reinterpret_cast<float*>(ws);
  float* acc_l = reinterpret_cast<float*>(ws + align256(rows * d * 4));
  float* part_o = reinterpret_cast<float*>(ws + align256(rows * d * 4) + align256(rows * 4));
  float* part_l = reinterpret_cast<float*>(ws + 2 * align256(rows * d * 4) + align256(rows * 4));

  int done = 0;
  if (in_dtype == ATTN_BF16) {
    // bf16 inputs: every block after the first merges into the running fp32 result in the attention kernel's
    // epilogue (no partial buffer, no separate merge pass); the last block writes o and lse
    for (int i = 0; i < n_blocks; ++i) {
      const attn_kv_block& b = kv_blocks[i];
      if (classify(Nq, b.Nk, causal, q_off, b.k_off, pos_stride) == 0) continue;
      const int diag = diag_offset(q_off, b.k_off, pos_stride);
      const bool last = (done == live - 1);
      rc = enqueue_fwd(q_shard, b.k, b.v, last ? o : acc_o, last ? lse : acc_l, BH, Nq, b.Nk, d, scale, causal, diag,
                       in_dtype, last ? o_dtype : ATTN_F32, st, ebattn::kNoWindow, 1, done > 0 ? acc_o : nullptr,
                       done > 0 ? acc_l : nullptr);
      if (rc != ATTN_OK) return rc;
      ++done;
    }
    return ATTN_OK;
  }
  for (int i = 0; i < n_blocks; ++i) {
    const attn_kv_block& b = kv_blocks[i];
    if (classify(Nq, b.Nk, causal, q_off, b.k_off, pos_stride) == 0) continue;
    const int diag = diag_offset(q_off, b.k_off, pos_stride);
    if (done == 0) {
      rc = enqueue_fwd(q_shard, b.k, b.v, acc_o, acc_l, BH, Nq, b.Nk, d, scale, causal, diag, in_dtype, ATTN_F32, st);
      if (rc != ATTN_OK) return rc;
    } else {
      rc = enqueue_fwd(q_shard, b.k, b.v, part_o, part_l, BH, Nq, b.Nk, d, scale, causal, diag, in_dtype, ATTN_F32, st);
      if (rc != ATTN_OK) return rc;
      const bool last = (done == live - 1);
      ebattn::MergeArgs m;
      m.o_a = acc_o;
      m.lse_a = acc_l;
      m.o_b = part_o;
      m.lse_b = part_l;
      m.o = last ? o : acc_o;
      m.lse = last ? lse : acc_l;
      m.rows = rows;
      m.d = d;
      const hipError_t e = ebattn::launch_lse_merge(m, 1, last ? (o_dtype == ATTN_F32) : 1, st);
      if (e != hipSuccess) return hip_fail(e, "merge launch");
    }
    ++done;
  }
  return ATTN_OK;
}

// The no-allocation variant's scratch: one array per GPU, in the code object's device memory, that holds the fp32
// accumulator (and, for fp32 inputs, the partial) of ring_local_noalloc. Host code never passes `scratch` itself
// to a kernel or a copy (on the host it names a stand-in, not device memory): it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use), or an error code.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EUNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ATTN_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int ring_local(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse, int B, int H,
               int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride, int in_dtype, int o_dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = '\0';
  return ring_local_run(q_shard, kv_blocks, n_blocks, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride,
                        in_dtype, o_dtype, workspace, workspace_bytes, ring_local_workspace_bytes(B, H, Nq, d), stream);
}

int ring_local_noalloc(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse, int B,
                       int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride, int in_dtype,
                       int o_dtype, void* stream) {
  g_err[0] = '\0';
  if (B < 0 || H < 0 || Nq < 0 || d < 0) return fail(ATTN_EINVAL, "negative size (B=%d H=%d Nq=%d d=%d)", B, H, Nq, d);
  const size_t need = ring_local_bytes_used(B, H, Nq, d, in_dtype);
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_EWORKSPACE, "ring_local_noalloc: this share needs %zu bytes of scratch, above the %zu-byte array",
                need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  int rc = scratch_ptr(&ws);
  if (rc != ATTN_OK) return rc;
  return ring_local_run(q_shard, kv_blocks, n_blocks, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride, in_dtype,
                        o_dtype, ws, (size_t)ATTN_NOALLOC_SCRATCH_BYTES, need, stream);
}

size_t ring_local_pipelined_workspace_bytes(int B, int H, int Nq, int d, int Nk_max) {
  if (B < 0 || H < 0 || Nq < 0 || d < 0 || Nk_max < 0) return 0;
  const size_t rows = (size_t)B * H * Nq, kv = (size_t)B * H * Nk_max * d * 2;
  return align256(rows * d * 4) + align256(rows * 4) + 4 * align256(kv);
}

int ring_local_pipelined(const void* q_shard, const attn_kv_block* kv_blocks, int n_blocks, void* o, float* lse,
                         int B, int H, int Nq, int d, float scale, int causal, int64_t q_off, int pos_stride,
                         int o_dtype, void* workspace, size_t workspace_bytes, void* compute_stream,
                         void* copy_stream) {
  g_err[0] = '\0';
  int rc = check_query_side(q_shard, o, lse, B, H, Nq, d, scale, causal, q_off, pos_stride, ATTN_BF16, o_dtype);
  if (rc != ATTN_OK) return rc;
  if (n_blocks < 0) return fail(ATTN_EINVAL, "negative n_blocks");
  if (n_blocks > 0 && !kv_blocks) return fail(ATTN_EINVAL, "null kv_blocks");
  const int64_t BH = (int64_t)B * H;
  const int64_t rows = BH * Nq;
  int nk_max = 0;
  for (int i = 0; i < n_blocks; ++i) {
    rc = check_kv(kv_blocks[i].k, kv_blocks[i].v, BH, kv_blocks[i].Nk, d, ATTN_BF16, kv_blocks[i].k_off, q_shard, o,
                  lse, Nq, o_dtype, BH);
    if (rc != ATTN_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "block %d: %s", i, g_err);
      return fail(rc, "%s", msg);
    }
    if (i > 0 && kv_blocks[i].Nk > nk_max) nk_max = kv_blocks[i].Nk;
  }
  if (rows == 0) return ATTN_OK;
  rc = check_outputs_disjoint(q_shard, o, lse, rows, d, ATTN_BF16, o_dtype);
  if (rc != ATTN_OK) return rc;
  // live blocks, in ring order; block 0 is resident, every later one arrives through a receive slot
  int live = 0, incoming = 0;
  for (int i = 0; i < n_blocks; ++i) {
    const bool l = classify(Nq, kv_blocks[i].Nk, causal, q_off, kv_blocks[i].k_off, pos_stride) != 0;
    live += l;
    incoming += l && i > 0;
  }
  const size_t need = ring_local_pipelined_workspace_bytes(B, H, Nq, d, nk_max);
  if (live >= 2 || incoming > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
    const Span sw = span(workspace, (int64_t)need);
    if (overlap(sw, span(o, rows * d * elem_bytes(o_dtype))) || overlap(sw, span(lse, rows * 4)) ||
        overlap(sw, span(q_shard, rows * d * 2)))
      return fail(ATTN_EINVAL, "workspace overlaps q, o or lse");
    for (int i = 0; i < n_blocks; ++i) {
      const int64_t kvb = BH * kv_blocks[i].Nk * d * 2;
      if (kv_blocks[i].Nk > 0 && (overlap(sw, span(kv_blocks[i].k, kvb)) || overlap(sw, span(kv_blocks[i].v, kvb))))
        return fail(ATTN_EINVAL, "workspace overlaps block %d", i);
    }
  }
  const hipStream_t cs = reinterpret_cast<hipStream_t>(compute_stream);
  const hipStream_t xs = reinterpret_cast<hipStream_t>(copy_stream);
  (void)hipGetLastError();
  if (live == 0) {
    const hipError_t e = ebattn::launch_fill_empty(o, lse, rows, d, o_dtype == ATTN_F32, cs);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "fill launch");
  }
  char* ws = reinterpret_cast<char*>(workspace);
  float* acc_o = reinterpret_cast<float*>(ws);
  float* acc_l = reinterpret_cast<float*>(ws + align256(rows * d * 4));
  char* slots = ws + align256(rows * d * 4) + align256(rows * 4);
  const size_t kv_slot = align256((size_t)BH * nk_max * d * 2);
  auto slot_k = [&](int s) { return slots + (2 * s) * kv_slot; };
  auto slot_v = [&](int s) { return slots + (2 * s + 1) * kv_slot; };

  // Two receive slots: while the compute stream attends the block in one slot, the copy stream brings the next
  // incoming block into the other. ready[s]: slot s holds its block; freed[s]: the compute that read slot s is
  // done, so the slot may be overwritten. entry: everything enqueued on the compute stream before this call --
  // the producer of an incoming device block, an earlier call still reading the same workspace -- is done; the
  // copy stream waits for it before its first copy.
  hipEvent_t ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr}, entry = nullptr;
  hipError_t e = hipEventCreateWithFlags(&entry, hipEventDisableTiming);
  for (int s = 0; s < 2 && e == hipSuccess; ++s) {
    e = hipEventCreateWithFlags(&ready[s], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&freed[s], hipEventDisableTiming);
  }
  auto release = [&]() {
    for (int s = 0; s < 2; ++s) {
      if (ready[s]) (void)hipEventDestroy(ready[s]);
      if (freed[s]) (void)hipEventDestroy(freed[s]);
    }
    if (entry) (void)hipEventDestroy(entry);
  };
  if (e != hipSuccess) {
    release();
    return hip_fail(e, "event create");
  }
  int inc[ATTN_MAX_RING_BLOCKS];
  int n_inc = 0;
  for (int i = 1; i < n_blocks; ++i)
    if (classify(Nq, kv_blocks[i].Nk, causal, q_off, kv_blocks[i].k_off, pos_stride) != 0) {
      if (n_inc == ATTN_MAX_RING_BLOCKS) {
        release();
        return fail(ATTN_EINVAL, "more than %d live incoming blocks", ATTN_MAX_RING_BLOCKS);
      }
      inc[n_inc++] = i;
    }
  auto copy_in = [&](int j) -> hipError_t {
    const attn_kv_block& b = kv_blocks[inc[j]];
    const int s = j & 1;
    hipError_t r = hipSuccess;
    if (j >= 2) r = hipStreamWaitEvent(xs, freed[s], 0);   // the block two steps back has been consumed
    const size_t bytes = (size_t)BH * b.Nk * d * 2;
    if (r == hipSuccess) r = hipMemcpyAsync(slot_k(s), b.k, bytes, hipMemcpyDefault, xs);
    if (r == hipSuccess) r = hipMemcpyAsync(slot_v(s), b.v, bytes, hipMemcpyDefault, xs);
    if (r == hipSuccess) r = hipEventRecord(ready[s], xs);
    return r;
  };
  int done = 0;
  auto attend = [&](const void* k, const void* v, const attn_kv_block& b) -> int {
    const bool last = (done == live - 1);
    const int r = enqueue_fwd(q_shard, k, v, last ? o : acc_o, last ? lse : acc_l, BH, Nq, b.Nk, d, scale, causal,
                              diag_offset(q_off, b.k_off, pos_stride), ATTN_BF16, last ? o_dtype : ATTN_F32, cs,
                              ebattn::kNoWindow, 1, done > 0 ? acc_o : nullptr, done > 0 ? acc_l : nullptr);
    ++done;
    return r;
  };
  if (n_inc > 0) {
    e = hipEventRecord(entry, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(xs, entry, 0);
    if (e == hipSuccess) e = copy_in(0);
  }
  if (e == hipSuccess && n_blocks > 0 &&
      classify(Nq, kv_blocks[0].Nk, causal, q_off, kv_blocks[0].k_off, pos_stride) != 0) {
    rc = attend(kv_blocks[0].k, kv_blocks[0].v, kv_blocks[0]);
    if (rc != ATTN_OK) {
      release();
      return rc;
    }
  }
  for (int j = 0; j < n_inc && e == hipSuccess; ++j) {
    if (j + 1 < n_inc) e = copy_in(j + 1);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, ready[j & 1], 0);
    if (e != hipSuccess) break;
    rc = attend(slot_k(j & 1), slot_v(j & 1), kv_blocks[inc[j]]);
    if (rc != ATTN_OK) {
      release();
      return rc;
    }
    e = hipEventRecord(freed[j & 1], cs);
  }
  release();
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "ring pipeline");
}

}  // extern "C"
