"""GPU parity over a seeded random sweep of shapes and masks, against the float64 oracle.

The hand-picked cases of the other parity tests aim at known edges; this sweep draws the arguments instead
(batch, heads and grouping, sequence lengths on both sides of the tile sizes and of the short-sequence limit,
head dim, causal or not, offsets, stride, window, output dtype), so that combinations nobody picked are covered
too: the forward, the backward, the fused merge (a running result over the first keys, a block over the rest)
and the ring share (blocks of a global sequence in a drawn order, contiguous or striped, bf16 or fp32, with and
without the exchange step). The draws are fixed by the seed; the bars are the same as in the other tests (bf16
inputs: 2e-2 on o, 1e-3 on lse; fp32 inputs: 1e-5; gradients: the per-element bound derived from the bf16
arithmetic, delta within the error propagated from the stored o).
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_F32, TOL_LSE, compare, dev_bf16, dev_f32, host_f64, torch
from tests.test_gpu_backward import check_grads
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
MERGE_CASES = []
for _ in range(12):
    _c = _draw(_RNG, short_share=0.0, max_n=300)
    MERGE_CASES.append((_c, int(_RNG.integers(0, _c[4] + 1)), bool(_RNG.random() < 0.5)))
RING_CASES = []
for _ in range(12):
    _nb = int(_RNG.integers(1, 5))
    _f32 = bool(_RNG.random() < 0.25)
    RING_CASES.append(dict(nb=_nb, n=int(_RNG.integers(1, 300)), d=int(_RNG.choice([24, 64, 128])),
                           B=int(_RNG.integers(1, 3)), H=int(_RNG.choice([1, 2, 4])), causal=bool(_RNG.random() < 0.8),
                           striped=bool(_RNG.random() < 0.3), r=int(_RNG.integers(0, _nb)), f32=_f32,
                           pipelined=(not _f32) and bool(_RNG.random() < 0.5),
                           order=[int(x) for x in _RNG.permutation(_nb)]))


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
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (q, k, v, do))
    omask = dict(causal=causal, q_off=q_off, k_off=k_off, stride=stride, window=window)
    ref = oracle.attention_backward(q64, k64, v64, do64, scale, **omask)
    # The drawn shapes include few keys read by many query rows (e.g. 203 rows of two heads on 4 keys), where dk
    # sums hundreds of terms and grows to |dk| ~ 12: one bf16 rounding of dS then moves it by more than a flat
    # 2e-2, so the gradients here are held to the bound derived from the arithmetic, element by element.
    check_grads([host_f64(x) for x in (dq, dk, dv, delta)], ref, f"random backward {i} {case}", q64, k64, v64, do64,
                host_f64(o), host_f64(lse), scale, omask, True, False, abs_bar=False)


@pytest.mark.parametrize("i", range(len(MERGE_CASES)),
                         ids=[f"{_case_id(c)}-split{sp}-{'inplace' if ip else 'out'}" for c, sp, ip in MERGE_CASES])
def test_random_fused_merge(eb, i):
    t = torch()
    case, split, inplace = MERGE_CASES[i]
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    print(f"[case] random fused merge {i} {case} split={split} inplace={inplace}", flush=True)
    scale = 1 / math.sqrt(d)
    q = normal_bf16_bits(300 + i, "q", (B, H, Nq, d))
    k = normal_bf16_bits(300 + i, "k", (B, Hkv, Nk, d))
    v = normal_bf16_bits(300 + i, "v", (B, Hkv, Nk, d))
    qd = dev_bf16(q)
    k1, v1 = dev_bf16(np.ascontiguousarray(k[:, :, :split])), dev_bf16(np.ascontiguousarray(v[:, :, :split]))
    k2, v2 = dev_bf16(np.ascontiguousarray(k[:, :, split:])), dev_bf16(np.ascontiguousarray(v[:, :, split:]))
    run_o, run_l = eb.attn_fwd_ex(qd, k1, v1, scale=scale, causal=causal, q_off=q_off, k_off=k_off, pos_stride=stride,
                                  window=window, out_dtype=t.float32)
    kw = dict(scale=scale, causal=causal, q_off=q_off, k_off=k_off + split * stride, pos_stride=stride, window=window)
    if inplace:
        o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, out=run_o, lse=run_l, **kw)
    else:
        o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, **kw)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale, causal=causal,
                                    q_off=q_off, k_off=k_off, stride=stride, window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"random fused merge {i} {case}")


@pytest.mark.parametrize("i", range(len(RING_CASES)), ids=[
    "nb{nb}-n{n}-d{d}-B{B}H{H}-c{causal}-{striped}-r{r}-f32{f32}-pipe{pipelined}".format(**c) for c in RING_CASES])
def test_random_ring_share(eb, i):
    t = torch()
    c = RING_CASES[i]
    nb, n, d, B, H, causal, r = c["nb"], c["n"], c["d"], c["B"], c["H"], c["causal"], c["r"]
    print(f"[case] random ring share {i} {c}", flush=True)
    scale = 1 / math.sqrt(d)
    if c["striped"]:
        offs, q_off, stride = list(range(nb)), r, nb
    else:
        offs, q_off, stride = [s * n for s in range(nb)], r * n, 1
    if c["f32"]:
        q = normal_f32(400 + i, "q", (B, H, n, d))
        ks = [normal_f32(400 + 17 * s + i, "k", (B, H, n, d)) for s in range(nb)]
        vs = [normal_f32(400 + 17 * s + i, "v", (B, H, n, d)) for s in range(nb)]
        up, wide, tol, tl = dev_f32, (lambda x: x.astype(np.float64)), TOL_F32, TOL_F32
    else:
        q = normal_bf16_bits(400 + i, "q", (B, H, n, d))
        ks = [normal_bf16_bits(400 + 17 * s + i, "k", (B, H, n, d)) for s in range(nb)]
        vs = [normal_bf16_bits(400 + 17 * s + i, "v", (B, H, n, d)) for s in range(nb)]
        up, wide, tol, tl = dev_bf16, bf16_bits_to_f64, TOL_BF16, TOL_LSE
    blocks = [(up(ks[s]), up(vs[s]), offs[s]) for s in c["order"]]
    if c["pipelined"]:
        own = c["order"].index(r)
        blocks = [blocks[own]] + [b for j, b in enumerate(blocks) if j != own]
        o, lse = eb.ring_local_pipelined(up(q), blocks, scale=scale, causal=causal, q_off=q_off, pos_stride=stride)
    else:
        o, lse = eb.ring_local(up(q), blocks, scale=scale, causal=causal, q_off=q_off, pos_stride=stride)
    t.cuda.synchronize()
    # the share's rows of attention over all blocks: each block by the oracle, merged by the oracle's merge
    parts = [oracle.attention(wide(q), wide(ks[s]), wide(vs[s]), scale, causal=causal, q_off=q_off, k_off=offs[s],
                              stride=stride) for s in range(nb)]
    o_ref, l_ref = oracle.lse_merge_many(parts)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, tol, tl, what=f"random ring share {i}")
