"""GPU parity of attn_fwd_ex (grouped-query heads, sliding window) against the float64 oracle.

The cases run every kernel path: the pipelined d = 128 kernel (4-wave causal and 8-wave unmasked launches),
d = 64 and d = 24 one tile at a time, the fp32 path and the short-sequence path. Windows are chosen to start
inside a tile, at a tile edge, to be 1 (each query sees only its own position), and to be wider than the
sequence (plain causal attention).
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_F32, TOL_LSE, compare, dev_bf16, dev_f32, host_f64, torch
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


# (B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window)
CASES = [
    (1, 8, 2, 300, 300, 128, True, 0, 0, 1, 100),
    (2, 4, 1, 257, 257, 128, False, 0, 0, 1, 0),        # multi-query, unmasked (8-wave launch)
    (1, 4, 4, 700, 700, 128, True, 0, 0, 1, 64),        # window of exactly one tile
    (1, 2, 2, 500, 900, 128, True, 400, 0, 1, 200),     # offset queries
    (1, 2, 1, 200, 200, 128, True, 2, 1, 4, 30),        # striped positions
    (1, 4, 2, 300, 300, 64, True, 0, 0, 1, 1),          # each query sees only itself
    (1, 6, 3, 333, 333, 24, True, 0, 0, 1, 77),
    (1, 3, 3, 129, 129, 128, True, 0, 0, 1, 100000),    # wider than the sequence: plain causal
    (1, 2, 2, 1000, 1000, 128, True, 0, 0, 1, 129),     # window edge moves across workgroups and waves
    (2, 4, 2, 190, 250, 128, False, 0, 0, 1, 0),        # grouped heads, unmasked
]


def _inputs(seed, B, H, Hkv, Nq, Nk, d):
    return (normal_bf16_bits(seed, "q", (B, H, Nq, d)), normal_bf16_bits(seed, "k", (B, Hkv, Nk, d)),
            normal_bf16_bits(seed, "v", (B, Hkv, Nk, d)))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}q{}k{}d{}c{}qo{}ko{}s{}w{}".format(*c))
def test_window_gqa_parity(eb, case):
    t = torch()
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    q, k, v = _inputs(21, B, H, Hkv, Nq, Nk, d)
    print(f"[case] window/gqa {case}", flush=True)
    o, lse = eb.attn_fwd_ex(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=1 / math.sqrt(d), causal=causal,
                            q_off=q_off, k_off=k_off, pos_stride=stride, window=window)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                    1 / math.sqrt(d), causal=causal, q_off=q_off, k_off=k_off, stride=stride,
                                    window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"{case}")


def test_window_gqa_fp32_and_short_paths(eb):
    t = torch()
    # fp32 inputs (vector-ALU path)
    B, H, Hkv, Nq, Nk, d, window = 1, 4, 2, 130, 130, 64, 50
    q, k, v = (normal_f32(22, n, (B, hh, N, d)) for n, hh, N in (("q", H, Nq), ("k", Hkv, Nk), ("v", Hkv, Nk)))
    print("[case] window/gqa fp32 path", flush=True)
    o, lse = eb.attn_fwd_ex(dev_f32(q), dev_f32(k), dev_f32(v), scale=0.125, causal=True, window=window)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, 0.125, causal=True, window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_F32, TOL_F32, what="fp32 path")
    # short sequences (one lane per query row)
    B, H, Hkv, Nq, Nk, d, window = 3, 4, 2, 8, 8, 24, 3
    q, k, v = _inputs(23, B, H, Hkv, Nq, Nk, d)
    print("[case] window/gqa short path", flush=True)
    o, lse = eb.attn_fwd_ex(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=0.2, causal=True, window=window)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 0.2,
                                    causal=True, window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 1e-5, what="short path")


def test_plain_calls_are_unchanged(eb):
    """attn_fwd_ex with Hkv = H and no window reproduces attn_fwd bit for bit."""
    t = torch()
    q, k, v = _inputs(24, 1, 3, 3, 300, 300, 128)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for causal in (False, True):
        a = eb.attn_fwd(qd, kd, vd, causal=causal)
        b = eb.attn_fwd_ex(qd, kd, vd, causal=causal)
        t.cuda.synchronize()
        assert t.equal(a[0], b[0]) and t.equal(a[1], b[1])
