"""GPU parity of attn_fwd_merge (one key/value block's attention merged into a running result in the attention
kernel's epilogue) against the float64 oracle over the union of the keys.

The running result is the library's own fp32 attention over the first part of the keys; the merged result over
both parts must match the oracle's attention over all keys (bf16 bar on o, 1e-3 on lse). Cases cover in-place and
separate outputs, bf16 and fp32 outputs, every head dim, grouped heads and windows, rows that are empty in one
part or in both, and blocks that hide every key.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_LSE, compare, dev_bf16, host_f64, torch
from workloads import bf16_bits_to_f64, normal_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


# (B, H, Hkv, Nq, Nk, split, d, causal, q_off, window)
CASES = [
    (1, 2, 2, 300, 500, 200, 128, False, 0, 0),
    (1, 2, 2, 300, 500, 200, 128, True, 200, 0),      # causal: first part fully visible, second partly
    (2, 4, 2, 257, 257, 100, 128, True, 0, 0),        # rows 0..99 see keys only in the first part
    (1, 4, 1, 333, 333, 129, 64, True, 0, 90),        # window: some rows see keys only in the second part
    (1, 3, 3, 200, 300, 150, 24, False, 0, 0),
    (1, 2, 2, 150, 150, 64, 128, True, -40, 0),       # the first rows see nothing at all
]


def _parts(eb, case, seed, out_f32, in_place):
    t = torch()
    B, H, Hkv, Nq, Nk, split, d, causal, q_off, window = case
    q = normal_bf16_bits(seed, "q", (B, H, Nq, d))
    k = normal_bf16_bits(seed, "k", (B, Hkv, Nk, d))
    v = normal_bf16_bits(seed, "v", (B, Hkv, Nk, d))
    qd = dev_bf16(q)
    k1, v1 = dev_bf16(np.ascontiguousarray(k[:, :, :split])), dev_bf16(np.ascontiguousarray(v[:, :, :split]))
    k2, v2 = dev_bf16(np.ascontiguousarray(k[:, :, split:])), dev_bf16(np.ascontiguousarray(v[:, :, split:]))
    mask = dict(causal=causal, q_off=q_off, window=window, scale=1 / math.sqrt(d))
    run_o, run_l = eb.attn_fwd_ex(qd, k1, v1, out_dtype=t.float32, **mask)
    if in_place:
        o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, k_off=split, out=run_o, lse=run_l, **mask)
    else:
        o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, k_off=split,
                                   out_dtype=t.float32 if out_f32 else t.bfloat16, **mask)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(d),
                                    causal=causal, q_off=q_off, window=window)
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}kv{}q{}k{}s{}d{}c{}qo{}w{}".format(*c))
@pytest.mark.parametrize("mode", ["in_place", "f32", "bf16"])
def test_fused_merge_parity(eb, case, mode):
    print(f"[case] fused merge {case} {mode}", flush=True)
    o, lse, o_ref, l_ref = _parts(eb, case, 41, mode != "bf16", mode == "in_place")
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"{case} {mode}")


def test_fused_merge_with_hidden_or_empty_block_keeps_running(eb):
    t = torch()
    B, H, N, d = 1, 2, 200, 128
    q = normal_bf16_bits(42, "q", (B, H, N, d))
    k = normal_bf16_bits(42, "k", (B, H, N, d))
    v = normal_bf16_bits(42, "v", (B, H, N, d))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    print("[case] fused merge: hidden and empty blocks", flush=True)
    run_o, run_l = eb.attn_fwd(qd, kd, vd, causal=True, out_dtype=t.float32)
    # a block placed after every query: all keys hidden; and a block with no keys at all
    o1, l1 = eb.attn_fwd_merge(qd, kd, vd, run_o, run_l, causal=True, k_off=10 * N)
    e = t.empty((B, H, 0, d), dtype=t.bfloat16, device=qd.device)
    o2, l2 = eb.attn_fwd_merge(qd, e, e, run_o, run_l)
    t.cuda.synchronize()
    for o, lse in ((o1, l1), (o2, l2)):
        assert t.allclose(o, run_o, rtol=1e-6, atol=1e-6) and t.allclose(lse, run_l, rtol=1e-6, atol=1e-6)


def test_ring_local_fused_matches_unfused_merge(eb):
    """ring_local with bf16 inputs merges in the kernel epilogue; the explicit attn_fwd + attn_lse_merge chain
    over the same blocks agrees to fp32 rounding."""
    t = torch()
    B, H, n, d = 1, 2, 256, 128
    q = normal_bf16_bits(43, "q", (B, H, n, d))
    ks = [normal_bf16_bits(43 + s, "k", (B, H, n, d)) for s in range(3)]
    vs = [normal_bf16_bits(43 + s, "v", (B, H, n, d)) for s in range(3)]
    qd = dev_bf16(q)
    kd, vd = [dev_bf16(x) for x in ks], [dev_bf16(x) for x in vs]
    print("[case] ring_local fused vs explicit merge", flush=True)
    blocks = [(kd[s], vd[s], s * n) for s in (2, 0, 1)]
    ws = t.empty(eb.ring_local_workspace_bytes(B, H, n, d), dtype=t.uint8, device=qd.device)
    o, lse = eb.ring_local(qd, blocks, causal=True, q_off=2 * n, out_dtype=t.float32, workspace=ws)
    acc_o, acc_l = eb.attn_fwd(qd, kd[2], vd[2], causal=True, q_off=2 * n, k_off=2 * n, out_dtype=t.float32)
    for s in (0, 1):
        po, pl = eb.attn_fwd(qd, kd[s], vd[s], causal=True, q_off=2 * n, k_off=s * n, out_dtype=t.float32)
        acc_o, acc_l = eb.attn_lse_merge(acc_o, acc_l, po, pl)
    t.cuda.synchronize()
    assert float((o - acc_o).abs().max()) < 1e-5 and float((lse - acc_l).abs().max()) < 1e-5
