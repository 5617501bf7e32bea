"""GPU parity at the full sizes of the named workloads, in the launch configurations the bench times.

Each output row depends only on its own query row and all keys, so the oracle checks sampled rows exactly
(random rows plus the first/last rows of query tiles and of the sequence). Properties that hold at any size
cover every row: the constructed mask probe (the output of each causal row is the base-64 digits of its own
global position, up to weights of about e^-45 on lower positions and the bf16 rounding of the weight and of the
output) and the Q = 0 closed form (uniform weights: prefix means of V, lse = log(visible count)).
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_LSE, compare, dev_bf16, host_f64, sample_rows, torch
from workloads import CONFIGS, bf16_bits_to_f64, f32_to_bf16_bits, mask_probe_inputs, normal_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _oracle_rows(Q, K, V, heads, rows, scale, **mask):
    """Oracle on selected (b, h) slices and query rows; Q/K/V are bf16 bit arrays [B, H, N, d]."""
    outs = []
    for b, h in heads:
        o, l = oracle.attention(bf16_bits_to_f64(Q[b:b + 1, h:h + 1]), bf16_bits_to_f64(K[b:b + 1, h:h + 1]),
                                bf16_bits_to_f64(V[b:b + 1, h:h + 1]), scale, rows=rows, **mask)
        outs.append((o[0, 0], l[0, 0]))
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def test_causal_8k_sampled(eb):
    t = torch()
    c = CONFIGS["causal_8k"]
    Q = normal_bf16_bits(c.seed, "q", (c.B, c.H, c.Nq, c.d))
    K = normal_bf16_bits(c.seed, "k", (c.B, c.H, c.Nq, c.d))
    V = normal_bf16_bits(c.seed, "v", (c.B, c.H, c.Nq, c.d))
    print("[case] causal_8k full size, bf16 and fp32 outputs", flush=True)
    qd, kd, vd = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    o, lse = eb.attn_fwd(qd, kd, vd, scale=c.scale, causal=True)
    o32, lse32 = eb.attn_fwd(qd, kd, vd, scale=c.scale, causal=True, out_dtype=t.float32)
    t.cuda.synchronize()
    rng = np.random.default_rng(0)
    heads = [(0, 0), (1, 7), (2, 19), (3, 31), (int(rng.integers(4)), int(rng.integers(32)))]
    rows = sample_rows(c.Nq, 128, 160, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, rows, c.scale, causal=True)
    oh = host_f64(o)
    lh = host_f64(lse)
    o_got = np.stack([oh[b, h, rows] for b, h in heads])
    l_got = np.stack([lh[b, h, rows] for b, h in heads])
    compare(o_got, l_got, o_ref, l_ref, TOL_BF16, TOL_LSE, what="causal_8k bf16 out")
    oh = host_f64(o32)
    lh = host_f64(lse32)
    compare(np.stack([oh[b, h, rows] for b, h in heads]), np.stack([lh[b, h, rows] for b, h in heads]), o_ref, l_ref,
            TOL_BF16, TOL_LSE, what="causal_8k fp32 out")


def test_causal_8k_q_zero_closed_form(eb):
    # Q = 0: every visible key has weight 1/(i+1): o_i is the prefix mean of V, lse_i = log(i+1), all rows
    t = torch()
    c = CONFIGS["causal_8k"]
    K = normal_bf16_bits(c.seed, "k", (c.B, c.H, c.Nq, c.d))
    V = normal_bf16_bits(c.seed, "v", (c.B, c.H, c.Nq, c.d))
    Q = np.zeros_like(K)
    o, lse = eb.attn_fwd(dev_bf16(Q), dev_bf16(K), dev_bf16(V), scale=c.scale, causal=True, out_dtype=t.float32)
    t.cuda.synchronize()
    lh = host_f64(lse)
    np.testing.assert_allclose(lh, np.broadcast_to(np.log(np.arange(1, c.Nq + 1)), lh.shape), rtol=0, atol=1e-5)
    oh = host_f64(o)
    for b, h in [(0, 0), (3, 31), (1, 16)]:
        v = bf16_bits_to_f64(V[b, h])
        prefix = np.cumsum(v, axis=0) / np.arange(1, c.Nq + 1)[:, None]
        err = np.abs(oh[b, h] - prefix).max()
        print(f"[parity] q=0 closed form head {(b, h)}: max|do|={err:.3e}", flush=True)
        assert err < 1e-4


def _probe_tensors(B, H, n, d, q_off, k_off, stride):
    q, k, v = mask_probe_inputs(n, n, q_off, k_off, stride)
    def pad(x):
        out = np.zeros((B, H, x.shape[0], d), dtype=np.float32)
        out[:, :, :, :3] = x
        return f32_to_bf16_bits(out)
    return pad(q), pad(k), pad(v)


def _assert_digits(got, want, what):
    # The next-lower visible position carries a weight of about e^-45 (a few 1e-18 in the output), so the row is
    # the last visible key's digits up to rounding: the key's weight enters P.V rounded to bf16 (at most 2^-8
    # relative against the fp32 sum that normalises o) and o is stored as bf16 (2^-8 relative): within
    # 2^-7 |digit| < 0.5. A wrong mask puts a different key's digits here, off by at least 1.
    bad = np.argwhere((np.abs(got - want) > 2.0 ** -7 * np.abs(want) + 1e-6).any(axis=-1))
    if bad.size:
        idx = tuple(bad[0])
        print(f"[probe] {what}: {len(bad)} mismatching rows; first at {idx}: got {got[idx]} want {want[idx]}; "
              f"rows {[tuple(b) for b in bad[:8]]}", flush=True)
    assert bad.size == 0, what


def _digits(pos):
    pos = np.asarray(pos)
    return np.stack([pos // 4096, (pos // 64) % 64, pos % 64], axis=-1).astype(np.float64)


def test_mask_probe_causal_8k_all_rows(eb):
    # every causal row's last visible key is itself: o = digits(own position), to bf16 rounding, in every row
    t = torch()
    n, d = 8192, 128
    Qb, Kb, Vb = _probe_tensors(1, 2, n, d, 0, 0, 1)
    o, lse = eb.attn_fwd(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), scale=1 / math.sqrt(d), causal=True)
    t.cuda.synchronize()
    oh = host_f64(o)
    want = _digits(np.arange(n))
    _assert_digits(oh[:, :, :, :3], np.broadcast_to(want, (1, 2, n, 3)), "causal 8k probe")
    assert (oh[:, :, :, 3:] == 0).all()


def test_mask_probe_ring_rank2_all_rows(eb):
    t = torch()
    n, d, W, r = 32768, 128, 4, 2
    _, Kb, Vb = _probe_tensors(1, 2, W * n, d, 0, 0, 1)
    q, _, _ = mask_probe_inputs(n, 1, 0, 0, 1)
    Qb = np.zeros((1, 2, n, d), dtype=np.float32)
    Qb[:, :, :, :3] = q
    Qb = f32_to_bf16_bits(Qb)
    blocks = [(dev_bf16(np.ascontiguousarray(Kb[:, :, s * n:(s + 1) * n])),
               dev_bf16(np.ascontiguousarray(Vb[:, :, s * n:(s + 1) * n])), s * n) for s in (2, 1, 0, 3)]
    o, lse = eb.ring_local(dev_bf16(Qb), blocks, causal=True, q_off=r * n)
    t.cuda.synchronize()
    oh = host_f64(o)
    want = _digits(np.arange(r * n, (r + 1) * n))
    _assert_digits(oh[:, :, :, :3], np.broadcast_to(want, (1, 2, n, 3)), "ring rank 2 probe")


@pytest.mark.parametrize("r", [0, 3])
def test_mask_probe_striped_all_rows(eb, r):
    t = torch()
    W, n, d = 4, 16384, 128
    _, Kb, Vb = _probe_tensors(1, 1, W * n, d, 0, 0, 1)
    q, _, _ = mask_probe_inputs(n, 1, 0, 0, 1)
    Qb = np.zeros((1, 1, n, d), dtype=np.float32)
    Qb[:, :, :, :3] = q
    Qb = f32_to_bf16_bits(Qb)
    blocks = [(dev_bf16(np.ascontiguousarray(Kb[:, :, s::W])), dev_bf16(np.ascontiguousarray(Vb[:, :, s::W])), s)
              for s in range(W)]
    o, lse = eb.ring_local(dev_bf16(Qb), blocks, causal=True, q_off=r, pos_stride=W)
    t.cuda.synchronize()
    oh = host_f64(o)
    want = _digits(np.arange(r, W * n, W))
    _assert_digits(oh[0, 0, :, :3], want, f"striped r={r} probe")


def test_ring_rank2of4_128k_sampled(eb):
    t = torch()
    c = CONFIGS["ring_rank2of4_128k"]
    n = c.Nq
    print("[case] ring_rank2of4_128k: generating global Q/K/V (N=131072, H=32)", flush=True)
    Q = normal_bf16_bits(c.seed, "q", (c.B, c.H, c.global_N, c.d))
    K = normal_bf16_bits(c.seed, "k", (c.B, c.H, c.global_N, c.d))
    V = normal_bf16_bits(c.seed, "v", (c.B, c.H, c.global_N, c.d))
    qd = dev_bf16(np.ascontiguousarray(Q[:, :, c.q_off:c.q_off + n]))
    kd = [dev_bf16(np.ascontiguousarray(K[:, :, s * n:(s + 1) * n])) for s in range(4)]
    vd = [dev_bf16(np.ascontiguousarray(V[:, :, s * n:(s + 1) * n])) for s in range(4)]
    blocks = [(kd[s], vd[s], s * n) for s in (2, 1, 0, 3)]
    o, lse = eb.ring_local(qd, blocks, scale=c.scale, causal=True, q_off=c.q_off)
    t.cuda.synchronize()
    rng = np.random.default_rng(3)
    heads = [(0, 0), (0, 13), (0, 31)]
    local = sample_rows(n, 128, 96, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, local + c.q_off, c.scale, causal=True)
    oh, lh = host_f64(o), host_f64(lse)
    compare(np.stack([oh[b, h, local] for b, h in heads]), np.stack([lh[b, h, local] for b, h in heads]), o_ref,
            l_ref, TOL_BF16, TOL_LSE, what="ring rank 2 of 4 (global N=131072)")


def test_striped_64k_sampled_all_ranks(eb):
    t = torch()
    c0 = CONFIGS["striped_r0_64k"]
    W = 4
    Q = normal_bf16_bits(c0.seed, "q", (c0.B, c0.H, c0.global_N, c0.d))
    K = normal_bf16_bits(c0.seed, "k", (c0.B, c0.H, c0.global_N, c0.d))
    V = normal_bf16_bits(c0.seed, "v", (c0.B, c0.H, c0.global_N, c0.d))
    kd = [dev_bf16(np.ascontiguousarray(K[:, :, s::W])) for s in range(W)]
    vd = [dev_bf16(np.ascontiguousarray(V[:, :, s::W])) for s in range(W)]
    rng = np.random.default_rng(4)
    heads = [(0, 0), (0, 15)]
    for r in range(W):
        print(f"[case] striped rank {r}", flush=True)
        c = CONFIGS[f"striped_r{r}_64k"]
        blocks = [(kd[s], vd[s], s) for s in [(r - i) % W for i in range(W)]]
        o, lse = eb.ring_local(dev_bf16(np.ascontiguousarray(Q[:, :, r::W])), blocks, scale=c.scale, causal=True,
                               q_off=r, pos_stride=W)
        t.cuda.synchronize()
        local = sample_rows(c.Nq, 128, 64, rng)
        o_ref, l_ref = _oracle_rows(Q, K, V, heads, local * W + r, c.scale, causal=True)
        oh, lh = host_f64(o), host_f64(lse)
        compare(np.stack([oh[b, h, local] for b, h in heads]), np.stack([lh[b, h, local] for b, h in heads]), o_ref,
                l_ref, TOL_BF16, TOL_LSE, what=f"striped r={r}")


def test_tabular_row_and_feature_axes(eb):
    # (batch=1, rows=150000, features=8, heads=4, head_dim=24). Drawn in the row-axis layout
    # [features, heads, rows, d]; the feature-axis layout [rows, heads, features, d] is its permutation.
    t = torch()
    cr = CONFIGS["tabular_rows_150k"]
    Q = normal_bf16_bits(cr.seed, "q", (cr.B, cr.H, cr.Nq, cr.d))
    K = normal_bf16_bits(cr.seed, "k", (cr.B, cr.H, cr.Nq, cr.d))
    V = normal_bf16_bits(cr.seed, "v", (cr.B, cr.H, cr.Nq, cr.d))
    print("[case] tabular row axis N=150000 d=24", flush=True)
    o, lse = eb.attn_fwd(dev_bf16(Q), dev_bf16(K), dev_bf16(V), scale=cr.scale)
    t.cuda.synchronize()
    rng = np.random.default_rng(5)
    heads = [(0, 0), (7, 3), (3, 1)]
    rows = sample_rows(cr.Nq, 128, 64, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, rows, cr.scale)
    oh, lh = host_f64(o), host_f64(lse)
    compare(np.stack([oh[b, h, rows] for b, h in heads]), np.stack([lh[b, h, rows] for b, h in heads]), o_ref, l_ref,
            TOL_BF16, TOL_LSE, what="tabular rows")
    del o, lse
    print("[case] tabular feature axis N=8 d=24, 600000 slices", flush=True)
    perm = lambda x: np.ascontiguousarray(np.transpose(x, (2, 1, 0, 3)))   # -> [rows, heads, features, d]
    Qf, Kf, Vf = perm(Q), perm(K), perm(V)
    o, lse = eb.attn_fwd(dev_bf16(Qf), dev_bf16(Kf), dev_bf16(Vf), scale=cr.scale)
    t.cuda.synchronize()
    sel = np.concatenate([[0, 1, 149999], rng.choice(150000, 200, replace=False)])
    oh, lh = host_f64(o), host_f64(lse)
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(Qf[sel]), bf16_bits_to_f64(Kf[sel]), bf16_bits_to_f64(Vf[sel]),
                                    cr.scale)
    compare(oh[sel], lh[sel], o_ref, l_ref, TOL_BF16, 1e-5, what="tabular features")


@pytest.mark.parametrize("key", ["causal_32k", "causal_128k"])
def test_causal_long_single_call_sampled(eb, key):
    """The long single-call workloads the bench times (B=1, H=32, d=128, causal, N = 32768 and 131072): sampled
    rows of three heads against the oracle."""
    t = torch()
    c = CONFIGS[key]
    print(f"[case] {key}: generating Q/K/V (N={c.Nq}, H={c.H})", flush=True)
    Q, K, V = (normal_bf16_bits(c.seed, n, (c.B, c.H, c.Nq, c.d)) for n in "qkv")
    o, lse = eb.attn_fwd(dev_bf16(Q), dev_bf16(K), dev_bf16(V), scale=c.scale, causal=True)
    t.cuda.synchronize()
    rng = np.random.default_rng(5)
    heads = [(0, 0), (0, 17), (0, 31)]
    rows = sample_rows(c.Nq, 128, 96, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, rows, c.scale, causal=True)
    oh, lh = host_f64(o), host_f64(lse)
    compare(np.stack([oh[b, h, rows] for b, h in heads]), np.stack([lh[b, h, rows] for b, h in heads]), o_ref, l_ref,
            TOL_BF16, TOL_LSE, what=f"{key} single call")


def _unfused_share(eb, qd, blocks, scale, q_off, stride):
    """The share as a chain of library calls: attn_fwd of each K/V block (in ring order) into an fp32 partial,
    each partial folded into the running fp32 result by attn_lse_merge (in place), the last merge writing bf16 o.
    Fully hidden blocks run too: their partial is (0, -inf) rows, which the merge weighs zero."""
    t = torch()
    acc_o = acc_l = None
    for i, (kb, vb, k_off) in enumerate(blocks):
        po, pl = eb.attn_fwd(qd, kb, vb, scale=scale, causal=True, q_off=q_off, k_off=k_off, pos_stride=stride,
                             out_dtype=t.float32)
        if acc_o is None:
            acc_o, acc_l = po, pl
            continue
        last = i == len(blocks) - 1
        out = t.empty(qd.shape, dtype=t.bfloat16, device=qd.device) if last else acc_o
        out_l = t.empty_like(acc_l) if last else acc_l
        acc_o, acc_l = eb.attn_lse_merge(acc_o, acc_l, po, pl, out=out, lse_out=out_l)
    return acc_o, acc_l


def test_ring_rank2of4_128k_unfused_merge_sampled(eb):
    """The ring share (rank 2 of 4, global N = 131072) composed as the workload states it: attn_fwd per K/V block
    into fp32 partials, combined with attn_lse_merge, against the oracle's rows of global causal attention."""
    t = torch()
    c = CONFIGS["ring_rank2of4_128k"]
    n = c.Nq
    print("[case] ring_rank2of4_128k unfused: attn_fwd partials + attn_lse_merge", flush=True)
    Q = normal_bf16_bits(c.seed, "q", (c.B, c.H, c.global_N, c.d))
    K = normal_bf16_bits(c.seed, "k", (c.B, c.H, c.global_N, c.d))
    V = normal_bf16_bits(c.seed, "v", (c.B, c.H, c.global_N, c.d))
    qd = dev_bf16(np.ascontiguousarray(Q[:, :, c.q_off:c.q_off + n]))
    blocks = [(dev_bf16(np.ascontiguousarray(K[:, :, s * n:(s + 1) * n])),
               dev_bf16(np.ascontiguousarray(V[:, :, s * n:(s + 1) * n])), s * n) for s in (2, 1, 0, 3)]
    o, lse = _unfused_share(eb, qd, blocks, c.scale, c.q_off, 1)
    t.cuda.synchronize()
    assert o.dtype == t.bfloat16
    rng = np.random.default_rng(13)
    heads = [(0, 0), (0, 21)]
    local = sample_rows(n, 128, 96, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, local + c.q_off, c.scale, causal=True)
    oh, lh = host_f64(o), host_f64(lse)
    compare(np.stack([oh[b, h, local] for b, h in heads]), np.stack([lh[b, h, local] for b, h in heads]), o_ref,
            l_ref, TOL_BF16, TOL_LSE, what="ring rank 2 of 4 unfused (attn_fwd + attn_lse_merge)")


@pytest.mark.parametrize("r", [1, 2])
def test_striped_64k_unfused_merge_sampled(eb, r):
    """A stripe of the striped workload (N = 65536, H = 16, stride 4) composed as attn_fwd per K/V stripe into
    fp32 partials plus attn_lse_merge; stripe 1's row 0 sees only stripes 0 and 1, so its partials of stripes 2
    and 3 are empty rows."""
    t = torch()
    c = CONFIGS[f"striped_r{r}_64k"]
    W = 4
    print(f"[case] striped r={r} unfused: attn_fwd partials + attn_lse_merge", flush=True)
    Q = normal_bf16_bits(c.seed, "q", (c.B, c.H, c.global_N, c.d))
    K = normal_bf16_bits(c.seed, "k", (c.B, c.H, c.global_N, c.d))
    V = normal_bf16_bits(c.seed, "v", (c.B, c.H, c.global_N, c.d))
    blocks = [(dev_bf16(np.ascontiguousarray(K[:, :, s::W])), dev_bf16(np.ascontiguousarray(V[:, :, s::W])), s)
              for s in [(r - i) % W for i in range(W)]]
    o, lse = _unfused_share(eb, dev_bf16(np.ascontiguousarray(Q[:, :, r::W])), blocks, c.scale, r, W)
    t.cuda.synchronize()
    rng = np.random.default_rng(14 + r)
    heads = [(0, 0), (0, 9)]
    local = sample_rows(c.Nq, 128, 64, rng)
    o_ref, l_ref = _oracle_rows(Q, K, V, heads, local * W + r, c.scale, causal=True)
    oh, lh = host_f64(o), host_f64(lse)
    compare(np.stack([oh[b, h, local] for b, h in heads]), np.stack([lh[b, h, local] for b, h in heads]), o_ref,
            l_ref, TOL_BF16, TOL_LSE, what=f"striped r={r} unfused (attn_fwd + attn_lse_merge)")
