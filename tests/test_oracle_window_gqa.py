"""Pins of the oracle's sliding window and grouped-query attention.

Source: "架构层解决方案 - Sparse Attention与Ring Attention", sections "Sliding Window Attention" (each token attends
only to the w most recent tokens) and "MQA与GQA" (query heads split into groups that share one key/value head).
Readings: a window of w positions keeps keys with q_pos - w < k_pos <= q_pos (the query's own position
included), and query head h reads key/value head h // (H // Hkv).

The pins: a scalar brute force that walks back w positions from each query (a different formulation from the
oracle's comparison of positions), a per-head brute force with the head mapping written out, closed forms
(Q = 0, window 1), invariants (a window wider than the sequence is plain causal attention; Hkv = H is plain
multi-head attention), and planted mistakes in copies of the oracle.
"""
import math

import numpy as np
import pytest

import oracle

INF = float("inf")


def brute_window(q, k, v, scale, q_off, k_off, stride, window):
    """One head: for each query, the visible keys are found by walking back from its position."""
    nq, d = q.shape
    nk, dv = v.shape
    key_at = {k_off + j * stride: j for j in range(nk)}
    o = np.zeros((nq, dv))
    lse = np.full(nq, -INF)
    for i in range(nq):
        qp = q_off + i * stride
        vis = [key_at[p] for p in range(qp, qp - window, -1) if p in key_at]
        if not vis:
            continue
        e = {j: math.exp(scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d))) for j in vis}
        z = math.fsum(e.values())
        for c in range(dv):
            o[i, c] = math.fsum(e[j] * float(v[j, c]) for j in vis) / z
        lse[i] = math.log(z)
    return o, lse


def _compare(o, lse, ob, lb, tol=1e-12):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) < tol
    assert np.max(np.abs(o - ob), initial=0.0) < tol


@pytest.mark.parametrize("nq,nk,q_off,k_off,stride,window", [
    (10, 10, 0, 0, 1, 1), (10, 10, 0, 0, 1, 3), (12, 9, 4, 0, 1, 5), (9, 12, 0, 3, 1, 4),
    (8, 8, 2, 1, 4, 9), (8, 8, 1, 3, 4, 6), (7, 11, -5, 2, 2, 7), (6, 6, 0, 0, 1, 100)])
def test_window_matches_brute_force(nq, nk, q_off, k_off, stride, window):
    rng = np.random.default_rng(nq * 131 + window)
    d, dv = 4, 3
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, dv))
    scale = 0.7
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal=True, q_off=q_off,
                              k_off=k_off, stride=stride, window=window)
    ob, lb = brute_window(q, k, v, scale, q_off, k_off, stride, window)
    _compare(o[0, 0], lse[0, 0], ob, lb)


def test_window_closed_forms():
    # Q = 0: uniform weights over the window; o = mean of the visible v, lse = log(count)
    nq = nk = 20
    w = 6
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 1, nk, 5))
    o, lse = oracle.attention(np.zeros((1, 1, nq, 5)), np.ones((1, 1, nk, 5)), v, 1.0, causal=True, window=w)
    for i in range(nq):
        lo = max(0, i - w + 1)
        assert abs(lse[0, 0, i] - math.log(i - lo + 1)) < 1e-12
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, lo:i + 1].mean(axis=0))) < 1e-12
    # window 1: every row sees exactly its own position
    q, k = rng.standard_normal((1, 1, nq, 5)), rng.standard_normal((1, 1, nk, 5))
    o, lse = oracle.attention(q, k, v, 0.5, causal=True, window=1)
    assert np.max(np.abs(o - v)) < 1e-12
    assert np.max(np.abs(lse[0, 0] - 0.5 * np.einsum("ic,ic->i", q[0, 0], k[0, 0]))) < 1e-12


def test_wide_window_is_causal_and_window_requires_causal():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 3, 15, 4)) for _ in range(3))
    a = oracle.attention(q, k, v, 0.4, causal=True, q_off=3, window=19)
    b = oracle.attention(q, k, v, 0.4, causal=True, q_off=3)
    assert np.max(np.abs(a[0] - b[0])) < 1e-15 and np.array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 0.4, causal=False, window=4)


def brute_gqa(q, k, v, scale, causal):
    """Per query head, attention against the key/value head its group shares, written out head by head."""
    B, H, nq, d = q.shape
    hkv = k.shape[1]
    per = H // hkv
    o = np.zeros((B, H, nq, v.shape[3]))
    lse = np.zeros((B, H, nq))
    for b in range(B):
        for h in range(H):
            g = h // per
            s = scale * q[b, h] @ k[b, g].T
            if causal:
                s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            o[b, h] = (e / z) @ v[b, g]
            lse[b, h] = (m + np.log(z))[:, 0]
    return o, lse


@pytest.mark.parametrize("H,hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (6, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_per_head_brute_force(H, hkv, causal):
    rng = np.random.default_rng(H * 10 + hkv)
    q = rng.standard_normal((2, H, 9, 4))
    k = rng.standard_normal((2, hkv, 9, 4))
    v = rng.standard_normal((2, hkv, 9, 3))
    o, lse = oracle.attention(q, k, v, 0.6, causal=causal)
    ob, lb = brute_gqa(q, k, v, 0.6, causal)
    assert np.max(np.abs(o - ob)) < 1e-12 and np.max(np.abs(lse - lb)) < 1e-12
    # the same heads with their shared key/value heads repeated is plain multi-head attention
    rep = H // hkv
    o2, l2 = oracle.attention(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), 0.6, causal=causal)
    assert np.max(np.abs(o - o2)) < 1e-15 and np.max(np.abs(lse - l2)) < 1e-15


def test_gqa_shape_errors():
    q = np.zeros((1, 6, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, np.zeros((1, 4, 4, 2)), np.zeros((1, 4, 4, 2)), 1.0)   # 4 does not divide 6


# planted mistakes: each must be caught by the pins above
def _window_inclusive_lower(q, k, v, scale, q_off, k_off, stride, window):
    """Mutant: keeps q_pos - w itself (one key too many)."""
    return oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal=True, q_off=q_off,
                            k_off=k_off, stride=stride, window=window + 1)


def _gqa_interleaved(q, k, v, scale, causal):
    """Mutant: query head h reads key/value head h % Hkv (interleaved groups)."""
    H, hkv = q.shape[1], k.shape[1]
    idx = np.arange(H) % hkv
    return oracle.attention(q, k[:, idx], v[:, idx], scale, causal=causal)


def test_planted_window_mistake_is_caught():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((10, 4)), rng.standard_normal((10, 4)), rng.standard_normal((10, 3))
    o, lse = _window_inclusive_lower(q, k, v, 0.7, 0, 0, 1, 3)
    ob, lb = brute_window(q, k, v, 0.7, 0, 0, 1, 3)
    assert np.max(np.abs(lse[0, 0] - lb)) > 1e-3


def test_planted_gqa_mistake_is_caught():
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((1, 8, 6, 4)), rng.standard_normal((1, 2, 6, 4)), rng.standard_normal((1, 2, 6, 3))
    o, lse = _gqa_interleaved(q, k, v, 0.6, False)
    ob, lb = brute_gqa(q, k, v, 0.6, False)
    assert np.max(np.abs(lse - lb)) > 1e-3
