"""GPU parity of the attention backward (attn_bwd, through the C ABI) against the float64 oracle.

Every case runs the library's forward first (its o and lse are what a training step would save), then the
backward, and compares dq, dk, dv and delta with oracle.attention_backward on the same bf16-exact inputs.

Tolerance: each gradient is a sum of MFMA products in which one factor was rounded to bf16 (the weights P for dv,
the score gradients dS for dq and dk; the inputs are exact bf16 values), and delta uses the forward's o, itself
rounded to bf16 when o is bf16. With the unit roundoff u = 2^-9 of round-to-nearest bf16 and independent
roundings, the normwise relative error is of order u (about 2e-3); the bar is 1e-2 normwise and 2e-2 of the
tensor's largest magnitude elementwise. delta (fp32 products of the stored o and dout) is held to the same bar.
Where the exact gradient is zero everywhere although its terms are not (window 1: dS = P (dout.v - dout.o) with
o = v), only fp32 rounding of dot products of size ~sqrt(d) remains: the bar is 1e-5 absolute. Rows with no
visible key must come back exactly zero in dq and delta.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import dev_bf16, dev_f32, host_f64, torch
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu

TOL_NORM = 1e-2
TOL_MAX = 2e-2


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _inputs(seed, B, H, Hkv, Nq, Nk, d):
    return (normal_bf16_bits(seed, "q", (B, H, Nq, d)), normal_bf16_bits(seed, "k", (B, Hkv, Nk, d)),
            normal_bf16_bits(seed, "v", (B, Hkv, Nk, d)), normal_bf16_bits(seed, "do", (B, H, Nq, d)))


def compare_grad(got, ref, what, tol_norm=None, tol_max=None):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref), initial=0.0))
    nref = float(np.linalg.norm(ref))
    err_max = float(np.max(np.abs(got - ref), initial=0.0))
    err_norm = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got))
    print(f"[parity] {what}: max|err|={err_max:.3e} (max|ref| {scale:.3e}) norm rel={err_norm:.3e}", flush=True)
    if nref == 0:
        assert err_max <= 1e-5, f"{what}: expected zeros up to fp32 rounding, got {err_max}"
        return
    tol_norm = TOL_NORM if tol_norm is None else tol_norm
    tol_max = TOL_MAX if tol_max is None else tol_max
    assert err_norm <= tol_norm, f"{what}: normwise error {err_norm}"
    assert err_max <= tol_max * scale, f"{what}: max error {err_max} > {tol_max} * {scale}"


def run_case(eb, case, seed=31, o_f32=False, grad="f32", q_gain=1):
    t = torch()
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    q, k, v, do = _inputs(seed, B, H, Hkv, Nq, Nk, d)
    if q_gain != 1:   # a power of two: the scaled bf16 values stay exact
        q = (q.astype(np.int32) + (int(round(math.log2(q_gain))) << 7) * (q & 0x7F80 != 0)).astype(np.uint16)
    scale = 1 / math.sqrt(d)
    mask = dict(causal=causal, q_off=q_off, k_off=k_off, pos_stride=stride, window=window)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    o, lse = eb.attn_fwd_ex(qd, kd, vd, scale=scale, out_dtype=t.float32 if o_f32 else t.bfloat16, **mask)
    gdt = t.float32 if grad == "f32" else t.bfloat16
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, scale=scale, grad_dtype=gdt, **mask)
    t.cuda.synchronize()
    ref = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                    bf16_bits_to_f64(do), scale, causal=causal, q_off=q_off, k_off=k_off,
                                    stride=stride, window=window)
    for name, g, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        compare_grad(host_f64(g), r, f"{case} {name}")
    # rows with no visible key: exactly zero
    _, l_ref = oracle.attention(bf16_bits_to_f64(q[:, :1]), bf16_bits_to_f64(k[:, :1]), bf16_bits_to_f64(v[:, :1]),
                                scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride, window=window)
    empty = np.isneginf(l_ref[0, 0])
    if empty.any():
        assert (host_f64(dq)[0, 0][empty] == 0).all() and (host_f64(delta)[0, 0][empty] == 0).all()
    return dq, dk, dv, delta


# (B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window)
CASES = [
    (1, 2, 2, 300, 300, 128, True, 0, 0, 1, 0),          # ragged tails, several tiles each way
    (1, 2, 2, 257, 190, 128, False, 0, 0, 1, 0),
    (2, 4, 2, 200, 200, 64, True, 0, 0, 1, 0),           # grouped heads, d = 64
    (1, 4, 1, 333, 333, 128, True, 0, 0, 1, 100),        # multi-query with a sliding window
    (1, 2, 2, 500, 900, 128, True, 400, 0, 1, 0),        # offset queries (bottom-right causal)
    (1, 2, 2, 200, 200, 128, True, 2, 1, 4, 0),          # striped positions
    (1, 2, 2, 200, 260, 128, True, -50, 0, 1, 0),        # the first 50 rows see no key
    (1, 1, 1, 5, 7, 64, False, 0, 0, 1, 0),              # tiny
    (1, 2, 2, 300, 300, 128, True, 0, 0, 1, 1),          # window 1: each row sees only itself
    (1, 2, 2, 129, 1000, 64, False, 0, 0, 1, 0),
    (1, 2, 2, 1000, 65, 128, True, 5, 0, 1, 0),
    (1, 3, 3, 333, 333, 24, True, 0, 0, 1, 0),           # d = 24 (padded to 32), as the tabular row axis
    (2, 4, 2, 150, 260, 24, False, 0, 0, 1, 0),
    (1, 4, 1, 200, 200, 24, True, 0, 0, 1, 37),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}q{}k{}d{}c{}qo{}ko{}s{}w{}".format(*c))
def test_backward_parity(eb, case):
    print(f"[case] backward {case}", flush=True)
    run_case(eb, case)


@pytest.mark.parametrize("o_f32,grad", [(True, "f32"), (False, "bf16"), (True, "bf16")])
def test_backward_dtypes(eb, o_f32, grad):
    case = (1, 2, 1, 260, 260, 128, True, 0, 0, 1, 0)
    print(f"[case] backward dtypes o_f32={o_f32} grad={grad}", flush=True)
    run_case(eb, case, seed=32, o_f32=o_f32, grad=grad)


@pytest.mark.parametrize("q_gain", [4, 16])
def test_backward_peaked_softmax(eb, q_gain):
    """Scores several times larger than N(0, 1) (q scaled by a power of two, exactly): the weights of a row
    concentrate on a few keys and dS = P (dP - delta) nearly cancels. With o kept in fp32, delta carries no bf16
    rounding of o, and the usual bar holds."""
    case = (1, 2, 2, 300, 300, 128, True, 0, 0, 1, 0)
    print(f"[case] backward peaked softmax q_gain={q_gain}", flush=True)
    run_case(eb, case, seed=34, o_f32=True, q_gain=q_gain)


@pytest.mark.parametrize("d", [24, 64, 128])
def test_backward_reads_nothing_past_the_tensors(eb, d):
    """Partial last tiles (166 query rows, 20 keys) with NaN right after the end of every input: rows past the end
    must read as zeros, so the gradients stay finite and match the oracle. (At d = 24 the tile copies once sized
    their range by the padded LDS row, 64 bytes, instead of the 48-byte row in memory, and read past the end.)"""
    t = torch()
    B, H, Hkv, Nq, Nk = 1, 2, 2, 166, 20
    q, k, v, do = _inputs(35, B, H, Hkv, Nq, Nk, d)
    print(f"[case] backward NaN-padded inputs d={d}", flush=True)

    def padded(bits):
        n = bits.size
        buf = t.full((n + 64 * 128,), float("nan"), dtype=t.bfloat16, device="cuda")
        buf[:n] = dev_bf16(bits).reshape(-1)
        return buf[:n].view(bits.shape)

    qd, kd, vd, dod = padded(q), padded(k), padded(v), padded(do)
    scale = 1 / math.sqrt(d)
    o, lse = eb.attn_fwd(qd, kd, vd, scale=scale, out_dtype=t.float32)
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, scale=scale)
    t.cuda.synchronize()
    ref = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                    bf16_bits_to_f64(do), scale)
    for name, g, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        compare_grad(host_f64(g), r, f"NaN-padded d={d} {name}")


def test_backward_ring_blocks_add_up(eb):
    """One share of a ring: the keys arrive in three blocks; with the global lse and o, the blocks' dq add up
    (accumulate) to the full dq, and each block's dk, dv are the full gradient's rows for its keys."""
    t = torch()
    B, H, N, d = 1, 2, 600, 128
    q, k, v, do = _inputs(33, B, H, H, N, N, d)
    scale = 1 / math.sqrt(d)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    print("[case] backward ring blocks", flush=True)
    o, lse = eb.attn_fwd(qd, kd, vd, scale=scale, causal=True)
    dq = t.zeros((B, H, N, d), dtype=t.float32, device=qd.device)
    dks, dvs = [], []
    for lo, hi in ((0, 200), (200, 450), (450, 600)):
        kb, vb = kd[:, :, lo:hi].contiguous(), vd[:, :, lo:hi].contiguous()
        dk = t.zeros_like(kb, dtype=t.float32)
        dv = t.zeros_like(vb, dtype=t.float32)
        eb.attn_bwd(qd, kb, vb, o, lse, dod, scale=scale, causal=True, k_off=lo, dq=dq, dk=dk, dv=dv,
                    accumulate=True)
        dks.append(dk)
        dvs.append(dv)
    t.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_backward(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v),
                                              bf16_bits_to_f64(do), scale, causal=True)
    compare_grad(host_f64(dq), rq, "ring dq")
    compare_grad(np.concatenate([host_f64(x) for x in dks], axis=2), rk, "ring dk")
    compare_grad(np.concatenate([host_f64(x) for x in dvs], axis=2), rv, "ring dv")


def test_backward_accumulate_adds(eb):
    t = torch()
    case = (1, 2, 2, 200, 200, 64, True, 0, 0, 1, 0)
    print("[case] backward accumulate", flush=True)
    dq, dk, dv, _ = run_case(eb, case, seed=34)
    B, H, Hkv, Nq, Nk, d = case[:6]
    q, k, v, do = _inputs(34, B, H, Hkv, Nq, Nk, d)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    o, lse = eb.attn_fwd(qd, kd, vd, causal=True)
    a = [x.clone() for x in (dq, dk, dv)]
    eb.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, dq=a[0], dk=a[1], dv=a[2], accumulate=True)
    t.cuda.synchronize()
    for x, y in zip(a, (dq, dk, dv)):
        assert t.allclose(x, 2 * y, rtol=1e-6, atol=1e-6)


def test_backward_empty_and_fully_masked(eb):
    t = torch()
    dev = t.device("cuda:0")
    d = 128
    print("[case] backward empty / fully masked", flush=True)
    q, k, v, do = _inputs(35, 1, 2, 2, 100, 50, d)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    # every key after every query: nothing visible -> all gradients zero
    o, lse = eb.attn_fwd(qd, kd, vd, causal=True, k_off=1000)
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, causal=True, k_off=1000)
    # no keys at all
    e = t.empty((1, 2, 0, d), dtype=t.bfloat16, device=dev)
    o0, l0 = eb.attn_fwd(qd, e, e)
    dq0, dk0, dv0, delta0 = eb.attn_bwd(qd, e, e, o0, l0, dod)
    # no queries at all
    eq = t.empty((1, 2, 0, d), dtype=t.bfloat16, device=dev)
    o1, l1 = eb.attn_fwd(eq, kd, vd)
    dq1, dk1, dv1, delta1 = eb.attn_bwd(eq, kd, vd, o1, l1, eq)
    t.cuda.synchronize()
    for x in (dq, dk, dv, delta, dq0, delta0, dk1, dv1):
        assert x.numel() == 0 or bool((x == 0).all())
    assert dk0.numel() == 0 and dq1.numel() == 0


def test_backward_deterministic(eb):
    t = torch()
    case = (1, 4, 2, 300, 300, 128, True, 0, 0, 1, 0)
    B, H, Hkv, Nq, Nk, d = case[:6]
    q, k, v, do = _inputs(36, B, H, Hkv, Nq, Nk, d)
    qd, kd, vd, dod = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(do)
    print("[case] backward deterministic", flush=True)
    o, lse = eb.attn_fwd_ex(qd, kd, vd, causal=True)
    a = eb.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    b = eb.attn_bwd(qd, kd, vd, o, lse, dod, causal=True)
    t.cuda.synchronize()
    for x, y in zip(a, b):
        assert t.equal(x, y)


def test_backward_causal_8k_full_size_heads(eb):
    """The backward at the forward's full workload (causal self-attention B=4, H=32, N=8192, d=128, the launch
    the bench times: fp32 gradients): two whole (batch, head) slices against the oracle, every element."""
    t = torch()
    from workloads import CONFIGS
    c = CONFIGS["causal_8k"]
    shape = (c.B, c.H, c.Nq, c.d)
    Q, K, V, dO = (normal_bf16_bits(c.seed, n, shape) for n in ("q", "k", "v", "do"))
    print("[case] backward causal_8k full size", flush=True)
    qd, kd, vd, dod = dev_bf16(Q), dev_bf16(K), dev_bf16(V), dev_bf16(dO)
    o, lse = eb.attn_fwd(qd, kd, vd, scale=c.scale, causal=True)
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, scale=c.scale, causal=True)
    t.cuda.synchronize()
    for b, h in ((0, 0), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(*(bf16_bits_to_f64(x[sl]) for x in (Q, K, V, dO)), c.scale, causal=True)
        for name, g, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
            compare_grad(host_f64(g[sl]), r, f"causal_8k b{b} h{h} {name}")


# fp32 inputs (the vector-ALU path): fp32 arithmetic throughout, so the bar is 1e-5 normwise and 1e-4 of the
# tensor's largest magnitude elementwise (sums of up to a thousand fp32 products of O(1) terms)
F32_CASES = [
    (1, 2, 2, 150, 170, 128, True, 0, 0, 1, 0),
    (1, 4, 2, 100, 90, 64, False, 0, 0, 1, 0),
    (2, 3, 3, 77, 77, 24, True, 0, 0, 1, 20),
    (1, 2, 1, 100, 200, 64, True, 100, 0, 1, 0),
    (1, 2, 2, 60, 60, 128, True, 1, 3, 4, 0),        # striped: row 0 sees nothing
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "B{}H{}kv{}q{}k{}d{}c{}qo{}ko{}s{}w{}".format(*c))
@pytest.mark.parametrize("grad", ["f32", "bf16"])
def test_backward_fp32_inputs(eb, case, grad):
    t = torch()
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, stride, window = case
    q, k, v, do = (normal_f32(37, n, (B, hh, N, d)) for n, hh, N in
                   (("q", H, Nq), ("k", Hkv, Nk), ("v", Hkv, Nk), ("do", H, Nq)))
    scale = 1 / math.sqrt(d)
    mask = dict(causal=causal, q_off=q_off, k_off=k_off, pos_stride=stride, window=window)
    print(f"[case] backward fp32 {case} grad={grad}", flush=True)
    qd, kd, vd, dod = dev_f32(q), dev_f32(k), dev_f32(v), dev_f32(do)
    o, lse = eb.attn_fwd_ex(qd, kd, vd, scale=scale, **mask)
    dq, dk, dv, delta = eb.attn_bwd(qd, kd, vd, o, lse, dod, scale=scale,
                                    grad_dtype=t.float32 if grad == "f32" else t.bfloat16, **mask)
    t.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, do, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride,
                                    window=window)
    tn, tm = (1e-5, 1e-4) if grad == "f32" else (TOL_NORM, TOL_MAX)
    for name, g, r in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), ref):
        compare_grad(host_f64(g), r, f"fp32 {case} {name}", tn if name != "delta" else 1e-5,
                     tm if name != "delta" else 1e-4)
