"""GPU parity of causal calls over 16K keys or more, which the d = 128 forward runs in workgroups of 256 query rows
(eight waves), against the float64 oracle, element by element.

The query rows sit at the end of the keys (bottom-right, as a ring shard's rows do), so their blocks end in the
diagonal tiles, and both lengths are ragged against the 256-row blocks and 64-key tiles. Each case runs with and
without a planted key whose score for one row overflows the weights taken against the first two tiles' maximum:
that block must be computed again with the row maximum formed at every tile. The fused merge of ring_local runs
the same kernel with a running result; grouped query heads run it over a shared key/value head (and, with a
sliding window, the 4-wave kernel). Tolerances (max-abs): bf16 paths 2e-2 on o, lse 1e-3 (5e-3 with the
planted score, whose lse is about 230).
"""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL_BF16, TOL_LSE, compare, dev_bf16, host_f64, torch
from workloads import bf16_bits_to_f64, f32_to_bf16_bits, normal_bf16_bits

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _inputs(seed, Nq, Nk, q_off, k_off, plant):
    """q, k, v of N(0,1) bf16 (1 batch, 2 heads); with `plant`, the key at global position q_off + 150 of head 0
    is 20 times query row 200 of head 0, whose score against it is then about 20 sqrt(d) (natural log)."""
    q = normal_bf16_bits(seed, "q", (1, 2, Nq, D))
    k = normal_bf16_bits(seed, "k", (1, 2, Nk, D))
    v = normal_bf16_bits(seed, "v", (1, 2, Nk, D))
    if plant:
        k = k.copy()
        qf = bf16_bits_to_f64(q)
        k[0, 0, q_off + 150 - k_off] = f32_to_bf16_bits((20.0 * qf[0, 0, 200]).astype(np.float32))
    return q, k, v


LONG = [
    # (Nq, Nk, q_off, k_off)
    (300, 16500, 16200, 0),      # diagonal in the last key tiles; both lengths ragged
    (520, 16384, 15864, 0),      # exactly 16K keys; the rows span three 256-row blocks
    (257, 20000, 19843, 100),    # keys start at position 100
]


@pytest.mark.parametrize("plant", [False, True], ids=["plain", "planted"])
@pytest.mark.parametrize("case", LONG, ids=lambda c: "q{}k{}qo{}ko{}".format(*c))
def test_long_causal_parity(eb, case, plant):
    t = torch()
    Nq, Nk, q_off, k_off = case
    print(f"[case] long causal {case} plant={plant}", flush=True)
    q, k, v = _inputs(41, Nq, Nk, q_off, k_off, plant)
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, q_off=q_off, k_off=k_off,
                         out_dtype=t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(D),
                                    causal=True, q_off=q_off, k_off=k_off)
    if plant:
        assert l_ref[0, 0, 200] > 200.0   # the planted score dominates its row
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 5e-3 if plant else TOL_LSE,
            what=f"long causal {case} plant={plant}")


@pytest.mark.parametrize("plant", [False, True], ids=["plain", "planted"])
def test_long_causal_fused_merge(eb, plant):
    # rows at the end of 33000 keys, in two blocks of 16500: the diagonal block first, then the full block merged
    # into it in the kernel's epilogue (the planted key sits in the merged block)
    t = torch()
    Nq, n, q_off = 300, 16500, 32700
    print(f"[case] long causal fused merge plant={plant}", flush=True)
    q, k, v = _inputs(43, Nq, 2 * n, q_off, 0, False)
    if plant:
        k = k.copy()
        k[0, 0, 5000] = f32_to_bf16_bits((20.0 * bf16_bits_to_f64(q)[0, 0, 200]).astype(np.float32))
    blocks = [(dev_bf16(np.ascontiguousarray(k[:, :, s * n:(s + 1) * n])),
               dev_bf16(np.ascontiguousarray(v[:, :, s * n:(s + 1) * n])), s * n) for s in (1, 0)]
    o, lse = eb.ring_local(dev_bf16(q), blocks, causal=True, q_off=q_off, out_dtype=t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(D),
                                    causal=True, q_off=q_off)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, 5e-3 if plant else TOL_LSE,
            what=f"long causal fused merge plant={plant}")


def test_long_causal_bf16_out(eb):
    t = torch()
    q, k, v = _inputs(47, 300, 16500, 16200, 0, False)
    print("[case] long causal bf16 out", flush=True)
    o, lse = eb.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, q_off=16200, out_dtype=t.bfloat16)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(D),
                                    causal=True, q_off=16200)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what="long causal bf16 out")


@pytest.mark.parametrize("window", [0, 4096], ids=["grouped", "grouped_window"])
def test_long_causal_grouped_heads(eb, window):
    # four query heads over one key/value head, 16500 keys: without a window the 8-wave kernel, with one the
    # 4-wave kernel (both must agree with the oracle)
    t = torch()
    Nq, Nk, q_off = 300, 16500, 16200
    print(f"[case] long causal grouped heads window={window}", flush=True)
    q = normal_bf16_bits(53, "q", (1, 4, Nq, D))
    k = normal_bf16_bits(53, "k", (1, 1, Nk, D))
    v = normal_bf16_bits(53, "v", (1, 1, Nk, D))
    o, lse = eb.attn_fwd_ex(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, q_off=q_off, window=window,
                            out_dtype=t.float32)
    t.cuda.synchronize()
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(D),
                                    causal=True, q_off=q_off, window=window)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"long causal grouped window={window}")
