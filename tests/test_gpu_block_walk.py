"""GPU parity of the forward when a workgroup computes several query blocks, against the float64 oracle.

The forward's grid is capped at one round of resident workgroups at d = 128 (512 workgroups of 128 rows under a
causal mask, 256 of 256 rows without one) and four rounds at d = 64 (3072). A launch with more query blocks than
that makes each workgroup walk several blocks in snake order. The other parity tests use too few blocks to get
there; these shapes use many heads of short sequences, so that the oracle still finishes in seconds. They cover:
- the XCD-remapped assignment and the plain one (block count not a multiple of 8);
- a last round that only some workgroups reach;
- per-block state that changes between the blocks of one workgroup: head, key/value head under grouping,
  offsets, window, the output row range, and the running result of the fused merge;
- blocks redone after the speculative reference overflowed, next to blocks that were not, in one workgroup.
The bars are those of the other parity tests: 2e-2 on bf16 o, 1e-3 on lse, 1e-5 on fp32 paths.
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_F32, TOL_LSE, compare, dev_bf16, dev_f32, host_f64, torch
from workloads import bf16_bits_to_f64, normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu

# (B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, window, out): query blocks = B*H*ceil(Nq/rows) with rows = 128,
# or 256 for d = 128 without a mask
CASES = {
    # 602 blocks over 512 workgroups, not a multiple of 8: plain assignment, 90 workgroups take a second block
    "d128_causal_plain": (1, 301, 301, 200, 200, 128, True, 0, 0, 0, "bf16"),
    # 640 blocks (remapped, 80 per XCD over 64 slots): grouped heads, offsets and a window change per block
    "d128_causal_gqa_window": (2, 160, 40, 250, 300, 128, True, 60, 0, 150, "bf16"),
    # the same walk with fp32 output rows
    "d128_causal_f32out": (1, 300, 100, 140, 140, 128, True, 0, 0, 0, "f32"),
    # 280 blocks of 256 rows over 256 workgroups (the unmasked 8-wave kernel)
    "d128_full_8wave": (1, 140, 140, 300, 170, 128, False, 0, 0, 0, "bf16"),
    # 3120 blocks over 3072 workgroups (four rounds at d = 64)
    "d64_causal": (1, 1560, 390, 129, 64, 64, True, 5, 0, 0, "bf16"),
}


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


@pytest.mark.parametrize("name", list(CASES))
def test_forward_walks_several_blocks(eb, name):
    t = torch()
    B, H, Hkv, Nq, Nk, d, causal, q_off, k_off, window, out = CASES[name]
    print(f"[case] block walk {name} {CASES[name]}", flush=True)
    seed = 700 + list(CASES).index(name)
    q = normal_bf16_bits(seed, "q", (B, H, Nq, d))
    k = normal_bf16_bits(seed, "k", (B, Hkv, Nk, d))
    v = normal_bf16_bits(seed, "v", (B, Hkv, Nk, d))
    scale = 1 / math.sqrt(d)
    mask = dict(causal=causal, q_off=q_off, k_off=k_off, pos_stride=1, window=window)
    o, lse = eb.attn_fwd_ex(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale,
                            out_dtype=t.float32 if out == "f32" else t.bfloat16, **mask)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale,
                                    causal=causal, q_off=q_off, k_off=k_off, stride=1, window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"block walk {name}")


def test_fused_merge_walks_several_blocks(eb):
    """600 blocks: the running result read and the merged row written belong to each walked block."""
    t = torch()
    B, H, Nq, Nk, d, split = 1, 300, 200, 230, 128, 90
    print(f"[case] block walk fused merge B{B} H{H} Nq{Nq} Nk{Nk} d{d} split{split}", flush=True)
    q = normal_bf16_bits(760, "q", (B, H, Nq, d))
    k = normal_bf16_bits(760, "k", (B, H, Nk, d))
    v = normal_bf16_bits(760, "v", (B, H, Nk, d))
    scale = 1 / math.sqrt(d)
    qd = dev_bf16(q)
    k1, v1 = dev_bf16(np.ascontiguousarray(k[:, :, :split])), dev_bf16(np.ascontiguousarray(v[:, :, :split]))
    k2, v2 = dev_bf16(np.ascontiguousarray(k[:, :, split:])), dev_bf16(np.ascontiguousarray(v[:, :, split:]))
    run_o, run_l = eb.attn_fwd_ex(qd, k1, v1, scale=scale, causal=True, q_off=40, out_dtype=t.float32)
    o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, out=run_o, lse=run_l, scale=scale, causal=True, q_off=40,
                               k_off=split)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale,
                                    causal=True, q_off=40)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what="block walk fused merge")


def test_fp32_inputs_many_blocks(eb):
    """The fp32 vector-ALU path at a block count past the MFMA kernel's cap (it has its own grid)."""
    B, H, Nq, Nk, d = 1, 300, 140, 100, 64
    print(f"[case] many blocks fp32 B{B} H{H} Nq{Nq} Nk{Nk} d{d}", flush=True)
    q = normal_f32(770, "q", (B, H, Nq, d))
    k = normal_f32(770, "k", (B, H, Nk, d))
    v = normal_f32(770, "v", (B, H, Nk, d))
    scale = 1 / math.sqrt(d)
    o, lse = eb.attn_fwd(dev_f32(q), dev_f32(k), dev_f32(v), scale=scale, causal=True, q_off=30)
    torch().cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale,
                                    causal=True, q_off=30)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_F32, TOL_F32, what="many blocks fp32")


def _plant(q, k, heads, key, row, gain=20.0):
    """Key `key` of each head in `heads` set to gain times query `row` of that head: that row's score against it
    lies far above anything the first two key tiles show, so its block overflows the speculative reference and is
    redone; the blocks of the other heads are not."""
    from workloads import f32_to_bf16_bits
    k = k.copy()
    qf = bf16_bits_to_f64(q)
    for h in heads:
        k[0, h, key] = f32_to_bf16_bits((gain * qf[0, h, row]).astype(np.float32))
    return k


@pytest.mark.parametrize("case", ["d128", "d64", "d128_fused_merge"])
def test_walk_with_some_blocks_redone(eb, case):
    # A workgroup that walks several blocks meets redone and plain blocks in either order: the verdict of one block
    # must not leak into the next (it is tagged with the walk round), and a redone block's stores and, with the
    # fused merge, its running result must come out as the oracle's.
    t = torch()
    print(f"[case] block walk with redone blocks {case}", flush=True)
    if case == "d128_fused_merge":
        B, H, Nq, Nk, d, split = 1, 300, 200, 230, 128, 90
        q = normal_bf16_bits(781, "q", (B, H, Nq, d))
        k = normal_bf16_bits(781, "k", (B, H, Nk, d))
        v = normal_bf16_bits(781, "v", (B, H, Nk, d))
        # key 220 (the second part's key 130, in its third tile) against row 190 (position 230 with q_off 40)
        k = _plant(q, k, range(0, H, 7), 220, 190)
        scale = 1 / math.sqrt(d)
        qd = dev_bf16(q)
        k1, v1 = dev_bf16(np.ascontiguousarray(k[:, :, :split])), dev_bf16(np.ascontiguousarray(v[:, :, :split]))
        k2, v2 = dev_bf16(np.ascontiguousarray(k[:, :, split:])), dev_bf16(np.ascontiguousarray(v[:, :, split:]))
        run_o, run_l = eb.attn_fwd_ex(qd, k1, v1, scale=scale, causal=True, q_off=40, out_dtype=t.float32)
        o, lse = eb.attn_fwd_merge(qd, k2, v2, run_o, run_l, out=run_o, lse=run_l, scale=scale, causal=True,
                                   q_off=40, k_off=split)
        mask = dict(causal=True, q_off=40)
    else:
        # d = 128: 602 blocks over 512 workgroups; d = 64: 3200 blocks over 3072 (four rounds)
        B, H, N, d = (1, 301, 200, 128) if case == "d128" else (1, 1600, 200, 64)
        q = normal_bf16_bits(782, "q", (B, H, N, d))
        k = normal_bf16_bits(782, "k", (B, H, N, d))
        v = normal_bf16_bits(782, "v", (B, H, N, d))
        k = _plant(q, k, range(0, H, 7), 150, 190)
        scale = 1 / math.sqrt(d)
        o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), scale=scale, causal=True, out_dtype=t.float32)
        mask = dict(causal=True)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), scale, **mask)
    # lse up to about 230 in the planted rows: fp32 score rounding is ~1e-5 relative
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 5e-3, what=f"block walk redone {case}")
