"""Exact work and byte counts used to turn kernel times into TFLOP/s and GB/s.

A "visible pair" is one (query row, key) pair that the mask lets through. Algorithmic FLOPs are 4*d per
visible pair: the two contractions Q.K^T and P.V each do one multiply-add (2 flops) per pair per head
dimension. Bytes are the minimum HBM traffic: every input read once and every output written once.
"""
from __future__ import annotations

import numpy as np


def diag_offset(q_off: int, k_off: int, stride: int) -> int:
    """Causal-by-position reduces to 'key j visible to query i iff j <= i + D'; returns D (floor division)."""
    return (int(q_off) - int(k_off)) // int(stride)


def visible_pairs(Nq: int, Nk: int, causal: bool, q_off: int = 0, k_off: int = 0, stride: int = 1,
                  window: int = 0) -> int:
    """Number of visible (query, key) pairs of one (batch, head); window > 0 (causal only) keeps the keys of the
    `window` most recent positions up to each query's own."""
    if not causal:
        return int(Nq) * int(Nk)
    D = diag_offset(q_off, k_off, stride)
    i = np.arange(Nq, dtype=np.int64)
    hi = np.clip(i + D + 1, 0, Nk)                      # one past the last visible key
    if not window:
        return int(hi.sum())
    lo = np.clip(i + diag_offset(q_off, k_off + window, stride) + 1, 0, Nk)   # first key inside the window
    return int(np.maximum(hi - lo, 0).sum())


def config_pairs(cfg) -> int:
    """Visible pairs of a whole workload (all heads, all key/value blocks)."""
    per_head = sum(visible_pairs(cfg.Nq, nk, cfg.causal, cfg.q_off, ko, cfg.stride) for nk, ko in cfg.blocks)
    return cfg.B * cfg.H * per_head


def attention_flops(pairs: int, d: int) -> float:
    return 4.0 * d * pairs


def attention_backward_flops(pairs: int, d: int) -> float:
    """Algorithmic FLOPs of the backward over `pairs` visible (query, key) pairs: five products of 2*d FLOPs per
    pair (S = QK^T recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q), 2.5 times the forward."""
    return 10.0 * d * pairs


def tensor_bytes(n: int, d: int, elem_bytes: int) -> int:
    """Bytes of one [n, d] matrix (one head's Q, K or V)."""
    return int(n) * int(d) * int(elem_bytes)


def score_matrix_bytes(n: int, elem_bytes: int) -> int:
    """Bytes of the full n x n score matrix that materialised attention stores."""
    return int(n) * int(n) * int(elem_bytes)


def score_pairs(n: int) -> int:
    """Number of score entries of full (unmasked) self-attention over n tokens."""
    return int(n) * int(n)


def attn_fwd_bytes(B, H, Nq, Nk, d, in_bytes, o_bytes) -> int:
    """Minimum HBM bytes of one attention forward: read Q, K, V once, write O and the fp32 lse once."""
    return B * H * ((Nq + 2 * Nk) * d * in_bytes + Nq * d * o_bytes + Nq * 4)


def merge_bytes(rows: int, d: int, part_bytes: int, o_bytes: int) -> int:
    """Minimum HBM bytes of one LSE merge: read two partials (o, lse), write one (o, lse)."""
    return int(rows) * (2 * (d * part_bytes + 4) + d * o_bytes + 4)
