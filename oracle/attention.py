"""Plain float64 definition of attention, of its masks by global position, and of the log-sum-exp merge.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke check and the bench's
CPU-baseline leg, never by the HIP path.

Sources (page title, then the section on it):
  [A] "深度学习注意力机制优化与FlashAttention实践", §2.1 数学表达式与计算流程 -- standard attention: scores are
      Q times K transposed divided by sqrt(d_k), a softmax over the key axis, then a weighted sum of V.
      Also "Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈", §2.1 (the same formula).
  [B] "架构层解决方案 - Sparse Attention与Ring Attention", section "Ring Attention / 核心创新" -- the softmax of a
      full key set decomposes over key blocks once every block is shifted by one common maximum m.
  [C] "分布式注意力机制突破：长序列处理的全景技术架构与实践指南", §2.2 stage 3 (pairwise LSE) and §3.4 (M-way
      merge: common maximum over the parts, per-part sums rescaled to it, LSE = max + log of the sum).
  [D] "深度学习注意力机制优化与FlashAttention实践", §5.1 -- causal masking must keep the autoregressive property.
  [E] "注意力机制演进", timeline table, row "Striped Attention" (named only; defined here by position).
  [F] "Mosaic多轴注意力分片：突破Transformer长序列处理瓶颈", §3.2 -- after all K/V shards have passed, each device
      holds the complete attention output of its own query shard.
  [G] "架构层解决方案 - Sparse Attention与Ring Attention", sections "Sliding Window Attention" (each token attends
      only to the w most recent tokens) and "MQA与GQA" (query heads split into g groups, each group sharing one
      key/value head; g = number of heads is plain multi-head attention, g = 1 is MQA).
  [H] "深度学习注意力机制优化与FlashAttention实践", §4.1 item 3 and §3.3 -- the backward pass recomputes the
      attention weights instead of storing them (blockwise softmax recomputation).

Readings where the pages are silent or garbled (each also listed in the design notes):
  * lse is the natural log of the sum of exp(scale * q.k) over the visible keys; no additive bias.
  * The pairwise formula printed in [C] §2.2 has the wrong sign in the exponent; the correct identity is
    log(e^a + e^b) = max(a, b) + log(1 + e^{-|a-b|}), which agrees with [C] §3.4's M-way steps.
  * Causal is inclusive: a key at the same global position as the query is visible.
  * Global positions: local query row i sits at q_off + i*stride, local key j at k_off + j*stride. Contiguous
    shards use stride 1; striping over W devices uses stride W with q_off = r, k_off = s ([E], plainest reading).
  * A query row with no visible key gets o = 0 and lse = -inf (no epsilon in the denominator); the merge treats
    lse = -inf as weight zero.
  * The scale is an explicit argument (the workloads pass 1/sqrt(d)).
  * Sliding window ([G]): with a window of w positions a key is visible iff q_pos - w < k_pos <= q_pos, i.e. the w
    most recent positions up to and including the query's own; a window is only defined together with the causal
    mask. w = 0 means no window.
  * Grouped-query attention ([G]): with Hkv key/value heads (Hkv divides H) query head h reads key/value head
    h // (H // Hkv), so consecutive query heads share a key/value head, as in the section's figure.
  * Backward ([H]): the pages name recomputation but give no formulas. The backward here is the exact gradient of
    the forward definition [A] for a scalar loss whose gradient with respect to o is do, obtained by the chain
    rule: o = p v, p = softmax of the scaled scores over the visible keys, s = scale q k^T. A key/value head shared
    by a group of query heads receives the sum of the group's gradients. Rows with no visible key have o = 0
    independent of every input, so they contribute nothing.

The attention here is the definition, not a blockwise algorithm: each query row's scores over ALL keys are
materialised at once (rows are processed in chunks only to bound memory), so this code shares no structure with
a tiled kernel.
"""
from __future__ import annotations

import numpy as np

_CHUNK_ELEMS = 8 << 20   # at most ~64 MB of float64 scores per chunk


def visible(nq: int, nk: int, causal: bool, q_off: int = 0, k_off: int = 0, stride: int = 1,
            rows=None, window: int = 0) -> np.ndarray:
    """Boolean [R, nk]: True where key j is visible to query row i ([D], [E], [G] and the readings above).

    rows: optional query row indices (default: all nq rows). window: sliding window in positions (0 = none;
    requires causal).
    """
    r = np.arange(nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if window and not causal:
        raise ValueError("a sliding window is defined only with the causal mask")
    if not causal:
        return np.ones((r.size, nk), dtype=bool)
    q_pos = int(q_off) + int(stride) * r
    k_pos = int(k_off) + int(stride) * np.arange(nk, dtype=np.int64)
    vis = k_pos[None, :] <= q_pos[:, None]
    if window:
        vis &= k_pos[None, :] > q_pos[:, None] - int(window)
    return vis


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Row softmax of scores s over the visible entries; returns (p, lse). Empty rows: p = 0, lse = -inf."""
    masked = np.where(vis, s, -np.inf)
    m = masked.max(axis=-1, keepdims=True)                  # -inf for an empty row
    has = np.isfinite(m)
    shift = np.where(has, m, 0.0)
    e = np.where(vis, np.exp(masked - shift), 0.0)
    l = e.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(has, shift + np.log(l), -np.inf)
    p = np.where(has, e / np.where(has, l, 1.0), 0.0)
    return p, lse[..., 0]


def attention(q, k, v, scale: float, causal: bool = False, q_off: int = 0, k_off: int = 0, stride: int = 1,
              rows=None, window: int = 0):
    """Exact attention ([A]) with the mask by global position, in float64.

    q: [B, H, Nq, d]; k: [B, Hkv, Nk, d]; v: [B, Hkv, Nk, dv] (any real dtype; widened to float64), Hkv dividing
       H (Hkv = H: multi-head; fewer: grouped-query, [G]).
    rows: optional 1-D indices of the query rows to compute (the same rows for every batch and head). Every
          output row depends only on its own query row and all keys, so a subset is exact.
    window: sliding window in positions (0 = none), with causal only ([G]).
    Returns (o [B, H, R, dv] float64, lse [B, H, R] float64), lse in natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if (k.shape[0] != B or Hkv < 1 or H % Hkv != 0 or v.shape[:3] != (B, Hkv, Nk) or k.shape[3] != d):
        raise ValueError("shape mismatch")
    group = H // Hkv
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    o = np.zeros((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.full((B, H, R), -np.inf, dtype=np.float64)
    chunk = max(1, _CHUNK_ELEMS // max(1, Nk))
    for c0 in range(0, R, chunk):
        rr = rows[c0:c0 + chunk]
        vis = visible(Nq, Nk, causal, q_off, k_off, stride, rows=rr, window=window)
        for b in range(B):
            for h in range(H):
                g = h // group                              # the key/value head of query head h ([G])
                s = scale * (q[b, h, rr] @ k[b, g].T)       # [r, Nk] scores, scaled ([A])
                p, l = _softmax_rows(s, vis)
                o[b, h, c0:c0 + rr.size] = p @ v[b, g]
                lse[b, h, c0:c0 + rr.size] = l
    return o, lse


def lse_merge_many(parts):
    """Merge partial results [(o_i, lse_i), ...] computed over disjoint key sets ([B], [C] §3.4).

    With lse_i = m_i + log s_i (local maximum m_i, local shifted sum s_i), [C] §3.4 takes the common maximum
    m = max_i m_i, the merged sum s = sum_i s_i * exp(m_i - m) and LSE = m + log s. In terms of the stored lse_i
    this is s = sum_i exp(lse_i - m) with m = max_i lse_i; each part's output is weighted by its share
    exp(lse_i - LSE) of the merged normaliser ([B]). Parts with lse = -inf (no visible key) weigh zero; if every
    part is empty the result is (0, -inf).
    """
    os_ = [np.asarray(o, dtype=np.float64) for o, _ in parts]
    ls = [np.asarray(l, dtype=np.float64) for _, l in parts]
    m = ls[0]
    for l in ls[1:]:
        m = np.maximum(m, l)
    has = np.isfinite(m)
    shift = np.where(has, m, 0.0)
    w = [np.where(np.isfinite(l), np.exp(l - shift), 0.0) for l in ls]
    s = sum(w)
    with np.errstate(divide="ignore"):
        lse = np.where(has, shift + np.log(np.where(has, s, 1.0)), -np.inf)
    den = np.where(has, s, 1.0)[..., None]
    o = sum(wi[..., None] * oi for wi, oi in zip(w, os_)) / den
    o = np.where(has[..., None], o, 0.0)
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partials (the two-part case of lse_merge_many)."""
    return lse_merge_many([(o_a, lse_a), (o_b, lse_b)])


def lse_pair(a, b):
    """log(e^a + e^b) by the pairwise form of [C] §2.2 with its exponent sign corrected:
    max(a, b) + log(1 + e^{-|a-b|}); -inf if both are -inf."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = np.maximum(a, b)
    both_empty = np.isneginf(m)
    with np.errstate(invalid="ignore"):
        diff = np.abs(a - b)                    # +inf when exactly one side is -inf: the term below is 0
        out = m + np.log1p(np.exp(-diff))
    return np.where(both_empty, -np.inf, out)


def attention_backward(q, k, v, do, scale: float, causal: bool = False, q_off: int = 0, k_off: int = 0,
                       stride: int = 1, window: int = 0):
    """Gradients of attention ([A], with the masks of [D], [E], [G]) for an output gradient do, in float64 ([H]).

    q: [B, H, Nq, d]; k: [B, Hkv, Nk, d]; v: [B, Hkv, Nk, dv]; do: [B, H, Nq, dv].
    Returns (dq [B, H, Nq, d], dk [B, Hkv, Nk, d], dv [B, Hkv, Nk, dv], delta [B, H, Nq]).

    The chain rule, one query row i at a time (all of its keys at once, as in the forward definition):
      p_i = softmax(s_i) over the visible keys (recomputed from q, k: nothing of the forward is stored),
      dp_ij = do_i . v_j                     (o_i = sum_j p_ij v_j),
      ds_i = J_i^T dp_i with the softmax Jacobian J_i = diag(p_i) - p_i p_i^T, i.e.
      ds_ij = p_ij (dp_ij - delta_i), delta_i = sum_j p_ij dp_ij,
      dq_i = scale sum_j ds_ij k_j,  dk_j += scale ds_ij q_i,  dv_j += p_ij do_i.
    delta is returned as well: it is the per-row quantity a blockwise backward needs besides the saved lse.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if (k.shape[0] != B or Hkv < 1 or H % Hkv != 0 or v.shape[:3] != (B, Hkv, Nk) or k.shape[3] != d
            or do.shape != (B, H, Nq, v.shape[3])):
        raise ValueError("shape mismatch")
    group = H // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((B, H, Nq), dtype=np.float64)
    chunk = max(1, _CHUNK_ELEMS // max(1, Nk))
    for c0 in range(0, Nq, chunk):
        rr = np.arange(c0, min(Nq, c0 + chunk), dtype=np.int64)
        vis = visible(Nq, Nk, causal, q_off, k_off, stride, rows=rr, window=window)
        for b in range(B):
            for h in range(H):
                g = h // group
                s = scale * (q[b, h, rr] @ k[b, g].T)            # [r, Nk]
                p, _ = _softmax_rows(s, vis)                     # recomputed weights ([H]); 0 where masked
                dp = do[b, h, rr] @ v[b, g].T                    # dL/dp
                dl = np.sum(p * dp, axis=1)                      # p_i . dp_i (the rank-one part of J_i)
                ds = p * (dp - dl[:, None])                      # J_i^T dp_i, zero where masked
                dq[b, h, rr] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ q[b, h, rr])
                dv[b, g] += p.T @ do[b, h, rr]
                delta[b, h, rr] = dl
    return dq, dk, dv, delta
