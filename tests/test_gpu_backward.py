"""GPU parity of the attention backward (attn_bwd, through the C ABI) against the float64 oracle.

Every case runs the library's forward first (its o and lse are what a training step would save), then the
backward, and compares dq, dk, dv and delta with oracle.attention_backward on the same bf16-exact inputs.

Bars (element-wise):
  * delta = rowsum(dout * o) is formed in fp32 from the o the forward stored. Its error against the oracle is the
    propagation of that o's own error plus the fp32 rounding of a d-term dot product,
        |delta_gpu_i - delta_ref_i| <= sum_c |dout_ic| |o_gpu_ic - o_ref_ic| + d u32 sum_c |dout_ic o_gpu_ic|
    (u32 = 2^-24, o_ref the oracle's forward); the stored o itself must meet the forward's bar (2e-2 max-abs for
    bf16 inputs, 1e-5 for fp32 inputs).
  * dq, dk, dv of bf16 inputs (the MFMA path: P is rounded to bf16 for dv, dS = P (dP - delta) to bf16 for dq
    and dk, every sum is fp32) are held to a first-order bound derived from that arithmetic, per element: with
    u16 = 2^-8 (bf16 round to nearest) and, per visible pair, eps_ij = the relative error of the recomputed P
    (the stored lse's error, the fp32 score's rounding d u32 scale sum_c |q_ic k_jc|, exp2's own 1e-6),
        E_ij  = P_ij eps_ij |dP_ij - delta_i| + P_ij (d u32 sum_c |dout_ic v_jc| + |delta error bound|_i),
        dq_ic : scale (sum_j (E_ij + u16 |dS_ij|) |k_jc| + Nk u32 sum_j |dS_ij k_jc|),
        dk_jc : scale (sum_i (E_ij + u16 |dS_ij|) |q_ic| + Nq u32 sum_i |dS_ij q_ic|)   (summed over a group),
        dv_jc : sum_i P_ij (eps_ij + u16) |dout_ic| + Nq u32 sum_i P_ij |dout_ic|       (summed over a group),
    plus u16 |g| when the gradient is stored as bf16. Second-order terms are covered by a factor 1.1 and 1e-6.
    This bound is the bar of every case. The cases here, all with N(0,1) inputs and gradients of order one, are
    also held to 2e-2 max-abs, except the peaked-softmax ones: they scale q up by 4 and 16, their gradients grow
    with it (|dk| up to 12.6 at q x 4), and one bf16 rounding of dS alone then moves an element by more than
    2e-2. (Gradients also grow when many query rows feed few keys, as in some of the randomly drawn shapes.)
  * fp32 inputs (the vector-ALU path, fp32 throughout): dq, dk, dv and delta within 1e-5 max-abs with fp32
    gradients; stored as bf16 they are within u16 |g| + 1e-5.
Where the exact gradient vanishes everywhere although its terms do not (window 1: dS = P (dout.v - dout.o) with
o = v), only fp32 rounding remains: 1e-5 max-abs. Rows with no visible key must come back exactly zero in dq
and delta.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import dev_bf16, dev_f32, host_f64, torch
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2     # max-abs: the forward's bf16 bar, and the gradients' wherever their arithmetic permits it
TOL_F32 = 1e-5      # max-abs: fp32 inputs with fp32 gradients (and their forward's o)
U32 = 2.0 ** -24    # unit roundoff of fp32
U16 = 2.0 ** -8     # unit roundoff of bf16 (8 significant bits, round to nearest even)


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _inputs(seed, B, H, Hkv, Nq, Nk, d):
    return (normal_bf16_bits(seed, "q", (B, H, Nq, d)), normal_bf16_bits(seed, "k", (B, Hkv, Nk, d)),
            normal_bf16_bits(seed, "v", (B, Hkv, Nk, d)), normal_bf16_bits(seed, "do", (B, H, Nq, d)))


def compare_grad(got, ref, what, tol, bound=None, abs_bar=True):
    """Element-wise: |got - ref| <= 1.1 bound + 1e-6 when a derived bound is given, and <= tol (max-abs) when
    abs_bar is set. Prints the figures."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    nref = float(np.linalg.norm(ref))
    err = np.abs(got - ref)
    err_max = float(np.max(err, initial=0.0))
    err_norm = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got))
    msg = (f"[parity] {what}: max|err|={err_max:.3e} (max|ref| {float(np.max(np.abs(ref), initial=0.0)):.3e}) "
           f"norm rel={err_norm:.3e}")
    if nref == 0:   # the exact gradient vanishes (window 1: dS = P (dout.v - dout.o) with o = v): fp32 rounding only
        tol = min(tol, 1e-5)
    if bound is not None:
        lim = 1.1 * bound + 1e-6
        worst = float(np.max(err / lim, initial=0.0))
        bmax = float(np.max(bound, initial=0.0))
        msg += f"; derived bound max {bmax:.3e}, max err/bound {worst:.3f}"
        print(msg, flush=True)
        assert (err <= lim).all(), f"{what}: error above the derived bound (ratio {worst})"
        if abs_bar:
            assert err_max <= tol, f"{what}: max error {err_max} > {tol}"
        return
    print(msg + f" (bar {tol:g})", flush=True)
    assert err_max <= tol, f"{what}: max error {err_max} > {tol}"


def delta_bound(dout, o_gpu, o_ref):
    """Per-row bound on |delta_gpu - delta_ref| from the stored o's error and the fp32 dot product (see the
    module docstring); dout, o_gpu, o_ref are [..., Nq, d] float64."""
    d = dout.shape[-1]
    prop = np.sum(np.abs(dout) * np.abs(o_gpu - o_ref), axis=-1)
    rnd = d * U32 * np.sum(np.abs(dout * o_gpu), axis=-1)
    return 1.001 * (prop + rnd) + 1e-7


def compare_delta(got, ref, bound, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape == bound.shape, (what, got.shape, ref.shape, bound.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    worst = float(np.max(err / bound, initial=0.0))
    print(f"[parity] {what}: max|err|={float(np.max(err, initial=0.0)):.3e}, max err/bound={worst:.3f} "
          f"(bound from o's error: max {float(np.max(bound, initial=0.0)):.3e})", flush=True)
    assert (err <= bound).all(), f"{what}: delta error exceeds the bound propagated from o (ratio {worst})"


def grad_bounds(q, k, v, do, lse_gpu, o_ref, lse_ref, ddelta, scale, mask):
    """The derived per-element bounds on dq, dk, dv of the bf16 MFMA path (module docstring), from the exact
    float64 quantities of the oracle's own definitions: scores, weights P, dP = dout.v, delta, dS."""
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = H // Hkv
    vis = oracle.visible(Nq, Nk, mask.get("causal", False), mask.get("q_off", 0), mask.get("k_off", 0),
                         mask.get("stride", 1), window=mask.get("window", 0))
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = h // grp
            qa, ka, va, da = np.abs(q[b, h]), np.abs(k[b, g]), np.abs(v[b, g]), np.abs(do[b, h])
            s = scale * (q[b, h] @ k[b, g].T)
            lr = lse_ref[b, h][:, None]
            fin = np.isfinite(lr)
            P = np.where(vis & fin, np.exp(np.where(vis & fin, s - np.where(fin, lr, 0.0), -np.inf)), 0.0)
            dP = do[b, h] @ v[b, g].T
            delta = np.sum(P * dP, axis=1, keepdims=True)
            dS = P * (dP - delta)
            dlse = np.where(fin, np.abs(lse_gpu[b, h][:, None] - np.where(fin, lr, 0.0)), 0.0)
            eps = scale * d * U32 * (qa @ ka.T) + dlse + 1e-6 * (1.0 + np.abs(s))
            E = P * eps * np.abs(dP - delta) + P * (d * U32 * (da @ va.T) + ddelta[b, h][:, None])
            ES = E + U16 * np.abs(dS)
            bq[b, h] = scale * (ES @ ka + Nk * U32 * (np.abs(dS) @ ka))
            bk[b, g] += scale * (ES.T @ qa + grp * Nq * U32 * (np.abs(dS).T @ qa))
            bv[b, g] += (P * (eps + U16)).T @ da + grp * Nq * U32 * (P.T @ da)
    return bq, bk, bv


def check_grads(got, ref, what, q, k, v, dout, o_gpu, lse_gpu, scale, mask, bf16_path, grad_bf16, abs_bar=True):
    """dq, dk, dv against their bars, the stored o against the forward's bar, delta against the bound propagated
    from that o. got = (dq, dk, dv, delta) and every input are float64 arrays of the exact values the GPU saw;
    mask uses the oracle's keywords (causal, q_off, k_off, stride, window)."""
    o_ref, lse_ref = oracle.attention(q, k, v, scale, **mask)
    err_o = float(np.max(np.abs(o_gpu - o_ref), initial=0.0))
    assert err_o <= (TOL_BF16 if bf16_path else TOL_F32), f"{what}: stored o error {err_o}"
    dbound = delta_bound(dout, o_gpu, o_ref)
    compare_delta(got[3], ref[3], dbound, f"{what} delta")
    if bf16_path:
        bounds = grad_bounds(q, k, v, dout, lse_gpu, o_ref, lse_ref, dbound, scale, mask)
        for name, g, r, bnd in zip(("dq", "dk", "dv"), got[:3], ref[:3], bounds):
            if grad_bf16:
                bnd = bnd + U16 * (np.abs(r) + bnd)
            compare_grad(g, r, f"{what} {name}", TOL_BF16, bound=bnd, abs_bar=abs_bar)
    else:
        compare_grad(got[3], ref[3], f"{what} delta", TOL_F32)
        for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
            if grad_bf16:
                compare_grad(g, r, f"{what} {name}", TOL_BF16, bound=U16 * np.abs(r) + TOL_F32)
            else:
                compare_grad(g, r, f"{what} {name}", TOL_F32)


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
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (q, k, v, do))
    omask = dict(causal=causal, q_off=q_off, k_off=k_off, stride=stride, window=window)
    ref = oracle.attention_backward(q64, k64, v64, do64, scale, **omask)
    check_grads([host_f64(x) for x in (dq, dk, dv, delta)], ref, f"{case} o_f32={o_f32} grad={grad} gain={q_gain}",
                q64, k64, v64, do64, host_f64(o), host_f64(lse), scale, omask, True, grad == "bf16",
                abs_bar=q_gain == 1)
    # rows with no visible key: exactly zero
    _, l_ref = oracle.attention(q64[:, :1], k64[:, :1], v64[:, :1], scale, **omask)
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
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (q, k, v, do))
    ref = oracle.attention_backward(q64, k64, v64, do64, scale)
    check_grads([host_f64(x) for x in (dq, dk, dv, delta)], ref, f"NaN-padded d={d}", q64, k64, v64, do64,
                host_f64(o), host_f64(lse), scale, {}, True, False)


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
    q64, k64, v64, do64 = (bf16_bits_to_f64(x) for x in (q, k, v, do))
    o_ref, lse_ref = oracle.attention(q64, k64, v64, scale, causal=True)
    bounds = grad_bounds(q64, k64, v64, do64, host_f64(lse), o_ref, lse_ref, delta_bound(do64, host_f64(o), o_ref),
                         scale, dict(causal=True))
    compare_grad(host_f64(dq), rq, "ring dq", TOL_BF16, bound=bounds[0])
    compare_grad(np.concatenate([host_f64(x) for x in dks], axis=2), rk, "ring dk", TOL_BF16, bound=bounds[1])
    compare_grad(np.concatenate([host_f64(x) for x in dvs], axis=2), rv, "ring dv", TOL_BF16, bound=bounds[2])


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
        q64, k64, v64, do64 = (bf16_bits_to_f64(x[sl]) for x in (Q, K, V, dO))
        ref = oracle.attention_backward(q64, k64, v64, do64, c.scale, causal=True)
        check_grads([host_f64(x[sl]) for x in (dq, dk, dv, delta)], ref, f"causal_8k b{b} h{h}", q64, k64, v64,
                    do64, host_f64(o[sl]), host_f64(lse[sl]), c.scale, dict(causal=True), True, False)


# fp32 inputs (the vector-ALU path): fp32 arithmetic throughout, so the bar is 1e-5 max-abs for fp32 gradients
# (and for delta and the forward's o); gradients stored as bf16 are within their output rounding plus 1e-5
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
    q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    check_grads([host_f64(x) for x in (dq, dk, dv, delta)], ref, f"fp32 {case} grad={grad}", q64, k64, v64, do64,
                host_f64(o), host_f64(lse), scale,
                dict(causal=causal, q_off=q_off, k_off=k_off, stride=stride, window=window), False, grad == "bf16")
