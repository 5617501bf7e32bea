"""GPU parity of the HIP path (through the C ABI) against the float64 oracle on seeded inputs.

Small shapes compare every element; they span several 128-row query tiles and 64-key tiles and end in ragged
tails. Edge cases: empty key sets, fully masked rows and blocks, single keys, short sequences, extreme scores.
Tolerances (max-abs): fp32 paths 1e-5; bf16 paths 2e-2 on o; lse 1e-3; -inf rows matched exactly.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import (TOL_BF16, TOL_F32, TOL_LSE, compare, dev_bf16, dev_f32, host_f64, torch)
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _inputs(seed, B, H, Nq, Nk, d):
    q = normal_bf16_bits(seed, "q", (B, H, Nq, d))
    k = normal_bf16_bits(seed, "k", (B, H, Nk, d))
    v = normal_bf16_bits(seed, "v", (B, H, Nk, d))
    return q, k, v


SMALL = [
    # (B, H, Nq, Nk, d, causal, q_off, k_off, stride)
    (1, 1, 128, 128, 128, False, 0, 0, 1),
    (1, 2, 128, 128, 128, True, 0, 0, 1),
    (2, 3, 300, 257, 128, False, 0, 0, 1),
    (2, 3, 300, 257, 128, True, 0, 0, 1),
    (1, 2, 333, 700, 128, True, 400, 0, 1),       # bottom-right style offset: every row sees >= 68 keys
    (1, 2, 256, 256, 128, True, 0, 100, 1),       # first 100 rows see nothing
    (1, 2, 200, 200, 128, True, 2, 1, 4),         # striped, key stripe before query stripe
    (1, 2, 200, 200, 128, True, 1, 3, 4),         # striped, key stripe after: row 0 empty
    (1, 1, 17, 1000, 128, False, 0, 0, 1),
    (1, 4, 1000, 17, 128, True, 5, 0, 1),
    (2, 2, 250, 190, 64, False, 0, 0, 1),
    (2, 2, 250, 190, 64, True, 30, 0, 1),
    (1, 3, 513, 77, 24, False, 0, 0, 1),
    (1, 3, 300, 300, 24, True, 0, 0, 1),
    (1, 2, 129, 65, 128, True, 64, 0, 1),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}q{}k{}d{}c{}qo{}ko{}s{}".format(*c))
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_small_parity(eb, case, out):
    t = torch()
    B, H, Nq, Nk, d, causal, q_off, k_off, stride = case
    q, k, v = _inputs(11, B, H, Nq, Nk, d)
    print(f"[case] small {case} out={out}", flush=True)
    odt = t.bfloat16 if out == "bf16" else t.float32
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=1 / math.sqrt(d), causal=causal, q_off=q_off,
                         k_off=k_off, pos_stride=stride, out_dtype=odt)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(d),
                                    causal=causal, q_off=q_off, k_off=k_off, stride=stride)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"{case} {out}")


@pytest.mark.parametrize("case", [
    (1, 1, 256, 256, 64, False, 0, 0, 1),
    (1, 2, 100, 150, 64, True, 0, 0, 1),
    (2, 1, 70, 33, 128, True, 40, 0, 1),
    (1, 2, 90, 90, 24, True, 1, 2, 4),
])
def test_fp32_path_parity(eb, case):
    B, H, Nq, Nk, d, causal, q_off, k_off, stride = case
    q = normal_f32(1, "q", (B, H, Nq, d))
    k = normal_f32(1, "k", (B, H, Nk, d))
    v = normal_f32(1, "v", (B, H, Nk, d))
    print(f"[case] fp32 {case}", flush=True)
    o, lse = eb.attn_fwd(dev_f32(q), dev_f32(k), dev_f32(v), scale=1 / math.sqrt(d), causal=causal, q_off=q_off,
                         k_off=k_off, pos_stride=stride)
    torch().cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, 1 / math.sqrt(d), causal=causal, q_off=q_off, k_off=k_off, stride=stride)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_F32, TOL_F32, what=f"fp32 {case}")


@pytest.mark.parametrize("case", [
    (3, 5, 8, 8, 24, False, 0, 0, 1),
    (3, 5, 8, 8, 24, True, 0, 0, 1),
    (2, 2, 1, 1, 128, False, 0, 0, 1),
    (2, 3, 16, 16, 64, True, 3, 0, 1),
    (1, 4, 5, 13, 128, True, 0, 4, 1),     # rows 0-3 empty
    (1000, 4, 8, 8, 24, False, 0, 0, 1),  # many slices per workgroup, ragged last workgroup
    (7, 3, 16, 2, 64, True, 5, 0, 1),     # more output than K/V bytes: each lane stores its own row
    (50, 2, 16, 3, 24, False, 0, 0, 1),
])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_short_sequences(eb, case, out):
    t = torch()
    B, H, Nq, Nk, d, causal, q_off, k_off, stride = case
    q, k, v = _inputs(5, B, H, Nq, Nk, d)
    print(f"[case] short {case} {out}", flush=True)
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, q_off=q_off, k_off=k_off,
                         pos_stride=stride, out_dtype=t.bfloat16 if out == "bf16" else t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(d),
                                    causal=causal, q_off=q_off, k_off=k_off, stride=stride)
    # this path keeps P in fp32: the fp32 output is held to a tighter bar than bf16 rounding needs
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16 if out == "bf16" else 1e-5, 1e-5,
            what=f"short {case} {out}")


def test_empty_and_fully_masked(eb):
    t = torch()
    q, k, v = _inputs(3, 1, 2, 200, 100, 128)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    # no key visible to any row: rows hidden by position
    o, lse = eb.attn_fwd(qd, kd, vd, causal=True, q_off=0, k_off=500)
    t.cuda.synchronize()
    assert (host_f64(o) == 0).all() and np.isneginf(host_f64(lse)).all()
    # Nk = 0
    e = t.empty((1, 2, 0, 128), dtype=t.bfloat16, device="cuda")
    o, lse = eb.attn_fwd(qd, e, e)
    t.cuda.synchronize()
    assert (host_f64(o) == 0).all() and np.isneginf(host_f64(lse)).all()
    # Nq = 0 is a no-op
    o, lse = eb.attn_fwd(t.empty((1, 2, 0, 128), dtype=t.bfloat16, device="cuda"), kd, vd)
    assert o.shape == (1, 2, 0, 128)


def test_extreme_scores_no_overflow(eb):
    # q scaled by 32: scores reach hundreds; exp without the running maximum would overflow
    t = torch()
    rng = np.random.default_rng(4)
    from workloads import f32_to_bf16_bits
    q = f32_to_bf16_bits(rng.standard_normal((1, 2, 300, 128)).astype(np.float32) * 32)
    k = f32_to_bf16_bits(rng.standard_normal((1, 2, 300, 128)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((1, 2, 300, 128)).astype(np.float32))
    for causal in (False, True):
        o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, out_dtype=t.float32)
        t.cuda.synchronize()
        o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                        1 / math.sqrt(128), causal=causal)
        # lse of order 1e2: fp32 score rounding is ~1e-5 relative
        compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 5e-3, what=f"extreme causal={causal}")


def _planted_key(seed, N, gain, d=128):
    """q, k, v of N(0,1) bf16 (1 batch, 2 heads, N tokens), with key 1300 of head 0 set to gain times query 1500 of
    head 0: that row's score against it is about gain * sqrt(d), far above anything the first two key tiles show
    any row."""
    from workloads import f32_to_bf16_bits
    q, k, v = _inputs(seed, 1, 2, N, N, d)
    qf = bf16_bits_to_f64(q)
    k = k.copy()
    k[0, 0, 1300] = f32_to_bf16_bits((gain * qf[0, 0, 1500]).astype(np.float32))
    return q, k, v


@pytest.mark.parametrize("gain", [3.0, 20.0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 64, 24])
def test_scores_far_above_the_first_tiles(eb, gain, causal, d):
    # The kernel takes the weights of later tiles against the reference the first two tiles set. With gain 3 the
    # planted score is about 3 sqrt(d) (natural log) above that reference, 21 to 49 in log2 units: the weights
    # grow to about 2^21..2^49 and stay finite. With gain 20 it is 98 to 226 (natural log) above: the weights
    # overflow, and the block must be redone with the row maximum formed at every tile. Both must match the
    # oracle, in the pipelined (d = 128) and the one-tile (d = 64, 24) kernels, and through the fused merge of
    # ring_local.
    t = torch()
    q, k, v = _planted_key(31, 2048, gain, d)
    print(f"[case] planted key gain={gain} causal={causal} d={d}", flush=True)
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, out_dtype=t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(d),
                                    causal=causal)
    # lse up to about 230: fp32 score rounding is ~1e-5 relative
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 5e-3, what=f"planted gain={gain} causal={causal} d={d}")
    if causal:
        n = 512
        blocks = [(dev_bf16(np.ascontiguousarray(k[:, :, s * n:(s + 1) * n])),
                   dev_bf16(np.ascontiguousarray(v[:, :, s * n:(s + 1) * n])), s * n) for s in (3, 1, 0, 2)]
        o, lse = eb.ring_local(dev_bf16(np.ascontiguousarray(q[:, :, 3 * n:])), blocks, causal=True, q_off=3 * n,
                               out_dtype=t.float32)
        t.cuda.synchronize()
        compare(host_f64(o), host_f64(lse), o_ref[:, :, 3 * n:], l_ref[:, :, 3 * n:], TOL_BF16, 5e-3,
                what=f"planted gain={gain} d={d} ring_local")


def test_values_one_give_one(eb):
    # V = 1: every non-empty row of o is exactly a probability-weighted average of ones
    t = torch()
    q, k, _ = _inputs(6, 1, 2, 300, 300, 128)
    ones = np.full((1, 2, 300, 128), 0x3F80, dtype=np.uint16)
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(ones), causal=True, q_off=0, k_off=10, out_dtype=t.float32)
    t.cuda.synchronize()
    oh, lh = host_f64(o), host_f64(lse)
    nonempty = ~np.isneginf(lh)
    assert nonempty.sum() == 2 * 290 and np.isneginf(lh[:, :, :10]).all()
    np.testing.assert_allclose(oh[nonempty], 1.0, rtol=0, atol=3e-3)   # bf16 rounding of P vs fp32 sum
    assert (oh[~nonempty] == 0).all()


def test_deterministic(eb):
    t = torch()
    q, k, v = _inputs(8, 2, 4, 700, 900, 128)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o1, l1 = eb.attn_fwd(qd, kd, vd, causal=True, q_off=200)
    o2, l2 = eb.attn_fwd(qd, kd, vd, causal=True, q_off=200)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16)) and t.equal(l1, l2)


# ------------------------------------------------------------------------------------------------- merge
@pytest.mark.parametrize("rows,d,pt,ot", [(1000, 128, "f32", "f32"), (777, 128, "f32", "bf16"),
                                           (513, 64, "bf16", "bf16"), (300, 24, "f32", "f32"),
                                           (301, 24, "bf16", "f32")])
def test_merge_parity(eb, rows, d, pt, ot):
    t = torch()
    rng = np.random.default_rng(rows)
    oa = rng.standard_normal((rows, d))
    ob = rng.standard_normal((rows, d))
    la = rng.standard_normal(rows) * 20
    lb = rng.standard_normal(rows) * 20
    la[::7] = -np.inf
    lb[::11] = -np.inf
    lb[::5] = la[::5]                       # equal lse
    oa[np.isneginf(la)] = 0
    ob[np.isneginf(lb)] = 0
    if pt == "bf16":
        from workloads import f32_to_bf16_bits
        oa_b, ob_b = f32_to_bf16_bits(oa.astype(np.float32)), f32_to_bf16_bits(ob.astype(np.float32))
        oa, ob = bf16_bits_to_f64(oa_b), bf16_bits_to_f64(ob_b)
        oad, obd = dev_bf16(oa_b), dev_bf16(ob_b)
    else:
        oa, ob = oa.astype(np.float32).astype(np.float64), ob.astype(np.float32).astype(np.float64)
        oad, obd = dev_f32(oa), dev_f32(ob)
    la = la.astype(np.float32).astype(np.float64)
    lb = lb.astype(np.float32).astype(np.float64)
    o, l = eb.attn_lse_merge(oad, dev_f32(la), obd, dev_f32(lb), out_dtype=t.float32 if ot == "f32" else t.bfloat16)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(oa, la, ob, lb)
    compare(host_f64(o), host_f64(l), o_ref, l_ref, TOL_F32 if ot == "f32" else TOL_BF16, TOL_F32,
            what=f"merge {rows}x{d} {pt}->{ot}")


def test_merge_in_place(eb):
    t = torch()
    rng = np.random.default_rng(2)
    oa, ob = rng.standard_normal((4096, 128)), rng.standard_normal((4096, 128))
    la, lb = rng.standard_normal(4096) * 3, rng.standard_normal(4096) * 3
    oa32, ob32 = oa.astype(np.float32), ob.astype(np.float32)
    la32, lb32 = la.astype(np.float32), lb.astype(np.float32)
    oad, lad = dev_f32(oa32), dev_f32(la32)
    eb.attn_lse_merge(oad, lad, dev_f32(ob32), dev_f32(lb32), out=oad, lse_out=lad)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(oa32, la32, ob32, lb32)
    compare(host_f64(oad), host_f64(lad), o_ref, l_ref, TOL_F32, TOL_F32, what="merge in place")


# --------------------------------------------------------------------------------------------- ring_local
@pytest.mark.parametrize("order", [[0, 1, 2, 3], [2, 1, 0, 3], [3, 0, 2, 1]])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_ring_local_contiguous_small(eb, order, out):
    # rank 2 of 4 over a global sequence of 4*160 tokens: the merged share equals rows 320..479 of global
    # causal attention, whatever order the blocks arrive in
    t = torch()
    n, W, H, d = 160, 4, 3, 128
    Q, K, V = _inputs(21, 1, H, n * W, n * W, d)
    r = 2
    kd = [dev_bf16(np.ascontiguousarray(K[:, :, s * n:(s + 1) * n])) for s in range(W)]
    vd = [dev_bf16(np.ascontiguousarray(V[:, :, s * n:(s + 1) * n])) for s in range(W)]
    blocks = [(kd[s], vd[s], s * n) for s in order]
    o, lse = eb.ring_local(dev_bf16(np.ascontiguousarray(Q[:, :, r * n:(r + 1) * n])), blocks, causal=True,
                           q_off=r * n, out_dtype=t.bfloat16 if out == "bf16" else t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(Q), bf16_bits_to_f64(K), bf16_bits_to_f64(V), 1 / math.sqrt(d),
                                    causal=True, rows=np.arange(r * n, (r + 1) * n))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"ring order={order} {out}")


@pytest.mark.parametrize("r", [0, 1, 2, 3])
def test_ring_local_striped_small(eb, r):
    t = torch()
    W, n, H, d = 4, 150, 2, 128
    Q, K, V = _inputs(22, 1, H, n * W, n * W, d)
    blocks = [(dev_bf16(np.ascontiguousarray(K[:, :, s::W])), dev_bf16(np.ascontiguousarray(V[:, :, s::W])), s)
              for s in [(r - i) % W for i in range(W)]]
    o, lse = eb.ring_local(dev_bf16(np.ascontiguousarray(Q[:, :, r::W])), blocks, causal=True, q_off=r, pos_stride=W)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(Q), bf16_bits_to_f64(K), bf16_bits_to_f64(V), 1 / math.sqrt(d),
                                    causal=True, rows=np.arange(r, n * W, W))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"striped r={r}")


def test_ring_local_single_and_no_live_block(eb):
    t = torch()
    Q, K, V = _inputs(23, 1, 2, 100, 300, 64)
    qd = dev_bf16(Q)
    kd, vd = dev_bf16(K), dev_bf16(V)
    # only the first block is visible at all (the second starts after every query position)
    o, lse = eb.ring_local(qd, [(kd, vd, 0), (kd, vd, 10_000)], causal=True, q_off=500)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(Q), bf16_bits_to_f64(K), bf16_bits_to_f64(V), 1 / 8.0,
                                    causal=True, q_off=500)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what="ring single live")
    o, lse = eb.ring_local(qd, [(kd, vd, 10_000), (kd, vd, 20_000)], causal=True, q_off=500)
    t.cuda.synchronize()
    assert (host_f64(o) == 0).all() and np.isneginf(host_f64(lse)).all()


def test_tiny_f32_workload(eb):
    # fp32, B=1 H=1 N=256 d=64, non-causal; also K/V split into 4 blocks of 64, merged by ring_local
    from workloads import CONFIGS
    c = CONFIGS["tiny_f32"]
    q = normal_f32(c.seed, "q", (c.B, c.H, c.Nq, c.d))
    k = normal_f32(c.seed, "k", (c.B, c.H, c.Nk_total, c.d))
    v = normal_f32(c.seed, "v", (c.B, c.H, c.Nk_total, c.d))
    qd, kd, vd = dev_f32(q), dev_f32(k), dev_f32(v)
    o, lse = eb.attn_fwd(qd, kd, vd, scale=c.scale)
    blocks = [(dev_f32(k[:, :, ko:ko + n]), dev_f32(v[:, :, ko:ko + n]), ko) for n, ko in c.blocks]
    om, lm = eb.ring_local(qd, blocks, scale=c.scale)
    torch().cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, c.scale)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_F32, TOL_F32, what="tiny_f32 unsplit")
    compare(host_f64(om), host_f64(lm), o_ref, l_ref, TOL_F32, TOL_F32, what="tiny_f32 4-block merge")
