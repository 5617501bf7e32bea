"""GPU parity over a seeded random sweep of shapes and masks, against the float64 oracle.

The hand-picked cases of the other parity tests aim at known edges; this sweep draws the arguments instead
(batch, heads and grouping, sequence lengths on both sides of the tile sizes and of the short-sequence limit,
head dim, causal or not, offsets, stride, window, output dtype), so that combinations nobody picked are covered
too. The draws are fixed by the seed; the bars are the same as in the other tests (bf16 inputs: 2e-2 on o,
1e-3 on lse; fp32 inputs: 1e-5; gradients: 1e-2 normwise and 2e-2 of the largest magnitude).
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_F32, TOL_LSE, compare, dev_bf16, dev_f32, host_f64, torch
from tests.test_gpu_backward import compare_grad
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu


def _draw(rng, short_share=0.2, max_n=320):
    B = int(rng.integers(1, 3))
    H = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([x for x in (1, 2, 4) if H % x == 0]))
    if rng.random() < short_share:
        Nq, Nk = int(rng.integers(1, 17)), int(rng.integers(1, 17))
    else:
        Nq, Nk = int(rng.integers(1, max_n)), int(rng.integers(1, max_n))
    d = int(rng.choice([24, 64, 128]))
    causal = bool(rng.random() < 0.7)
    stride = int(rng.choice([1, 1, 2, 4]))
    q_off = int(rng.integers(-40, 300)) if causal else 0
    k_off = int(rng.integers(-40, 300)) if causal else 0
    window = int(rng.integers(1, 200)) if causal and rng.random() < 0.35 else 0
    return (B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window)


_RNG = np.random.default_rng(20261203)
FWD_CASES = [(_draw(_RNG), str(_RNG.choice(["bf16", "bf16", "f32out", "f32in"]))) for _ in range(40)]
BWD_CASES = [_draw(_RNG, short_share=0.0, max_n=260) for _ in range(16)]


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _case_id(c):
    return "B{}H{}kv{}q{}k{}d{}c{}qo{}ko{}s{}w{}".format(*c)


@pytest.mark.parametrize("i", range(len(FWD_CASES)), ids=[f"{k}-{_case_id(c)}" for c, k in FWD_CASES])
def test_random_forward(eb, i):
    t = torch()
    case, kind = FWD_CASES[i]
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    print(f"[case] random forward {i} {kind} {case}", flush=True)
    mask = dict(causal=causal, q_off=q_off, k_off=k_off, pos_stride=stride, window=window)
    scale = 1 / math.sqrt(d)
    if kind == "f32in":
        q = normal_f32(100 + i, "q", (B, H, Nq, d))
        k = normal_f32(100 + i, "k", (B, Hkv, Nk, d))
        v = normal_f32(100 + i, "v", (B, Hkv, Nk, d))
        o, lse = eb.attn_fwd_ex(dev_f32(q), dev_f32(k), dev_f32(v), scale=scale, **mask)
        tol = TOL_F32
        qr, kr, vr = (x.astype(np.float64) for x in (q, k, v))
    else:
        q = normal_bf16_bits(100 + i, "q", (B, H, Nq, d))
        k = normal_bf16_bits(100 + i, "k", (B, Hkv, Nk, d))
        v = normal_bf16_bits(100 + i, "v", (B, Hkv, Nk, d))
        o, lse = eb.attn_fwd_ex(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale,
                                out_dtype=t.float32 if kind == "f32out" else t.bfloat16, **mask)
        tol = TOL_BF16
        qr, kr, vr = (bf16_bits_to_f64(x) for x in (q, k, v))
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(qr, kr, vr, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride,
                                    window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, tol, TOL_F32 if kind == "f32in" else TOL_LSE,
            what=f"random forward {i} {kind} {case}")


@pytest.mark.parametrize("i", range(len(BWD_CASES)), ids=[_case_id(c) for c in BWD_CASES])
def test_random_backward(eb, i):
    t = torch()
    case = BWD_CASES[i]
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    print(f"[case] random backward {i} {case}", flush=True)
    mask = dict(causal=causal, q_off=q_off, k_off=k_off, pos_stride=stride, window=window)
    scale = 1 / math.sqrt(d)
    q = normal_bf16_bits(200 + i, "q", (B, H, Nq, d))
    k = normal_bf16_bits(200 + i, "k", (B, Hkv, Nk, d))
    v = normal_bf16_bits(200 + i, "v", (B, Hkv, Nk, d))
    do = normal_bf16_bits(200 + i, "do", (B, H, Nq, d))
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    o, lse = eb.attn_fwd_ex(qd, kd, vd, scale=scale, out_dtype=t.float32, **mask)
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, scale=scale, **mask)
    t.cuda.synchronize()
    ref = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                    bf16_bits_to_f64(do), scale, causal=causal, q_off=q_off, k_off=k_off,
                                    stride=stride, window=window)
    for name, g, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        compare_grad(host_f64(g), r, f"random backward {i} {case} {name}")
