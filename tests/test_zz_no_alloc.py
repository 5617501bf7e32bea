"""GPU check of ring_local_noalloc (the entry point that allocates nothing: its workspace is the library's
per-GPU scratch array) against ring_local (a caller workspace), through the C ABI directly.

Two calls in a row on one GPU, the second with a smaller share, for bf16 and fp32 inputs: each result must equal
ring_local's over the same blocks bit for bit (same kernels, same merge order), and the scratch array keeps the
first call's contents when the second one runs. Shares too large for the array are refused before any launch.
"""
import ctypes
import math

import numpy as np
import pytest

from tests.gpu_util import dev_bf16, dev_f32, torch
from workloads import normal_bf16_bits, normal_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eb():
    import exact_blockwise_attention_amd as m
    return m


def _share(dtype, seed, B, H, n, P, d):
    """Rank P-1 of a P-way contiguous ring (every block live), blocks of n keys, in ring order."""
    t = torch()
    if dtype == "bf16":
        Q, K, V = (normal_bf16_bits(seed, x, (B, H, P * n, d)) for x in "qkv")
        up = lambda a: dev_bf16(np.ascontiguousarray(a))         # noqa: E731
    else:
        Q, K, V = (normal_f32(seed, x, (B, H, P * n, d)) for x in "qkv")
        up = lambda a: dev_f32(np.ascontiguousarray(a))          # noqa: E731
    r = P - 1
    qd = up(Q[:, :, r * n:(r + 1) * n])
    blocks = [(up(K[:, :, s * n:(s + 1) * n]), up(V[:, :, s * n:(s + 1) * n]), s * n) for s in
              [(r - i) % P for i in range(P)]]
    o = t.empty_like(qd)
    lse = t.empty((B, H, n), dtype=t.float32, device=qd.device)
    return qd, blocks, o, lse, r * n


def _call_noalloc(eb, qd, blocks, o, lse, q_off):
    t = torch()
    B, H, Nq, d = qd.shape
    arr, nb = eb._blocks(blocks)
    code = eb.ATTN_BF16 if qd.dtype == t.bfloat16 else eb.ATTN_F32
    return eb.lib.ring_local_noalloc(qd.data_ptr(), arr, nb, o.data_ptr(), lse.data_ptr(), B, H, Nq, d,
                                     ctypes.c_float(1 / math.sqrt(d)), 1, q_off, 1, code, code,
                                     t.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("dtype,shapes", [
    ("bf16", [(1, 8, 1000, 4, 128), (1, 2, 300, 3, 64)]),
    ("f32", [(1, 4, 500, 3, 128), (1, 1, 130, 2, 24)]),
    ("bf16", [(1, 2, 16500, 2, 128), (1, 1, 300, 2, 128)]),   # blocks over 16K keys: the 8-wave causal kernel
])
def test_noalloc_matches_ring_local_twice(eb, dtype, shapes):
    t = torch()
    runs = []
    for i, (B, H, n, P, d) in enumerate(shapes):
        print(f"[case] ring_local_noalloc {dtype} call {i}: B={B} H={H} n={n} P={P} d={d}", flush=True)
        qd, blocks, o, lse, q_off = _share(dtype, 80 + i, B, H, n, P, d)
        rc = _call_noalloc(eb, qd, blocks, o, lse, q_off)
        assert rc == eb.ATTN_OK, eb.last_error()
        runs.append((qd, blocks, o, lse, q_off))
    t.cuda.synchronize()
    for i, (qd, blocks, o, lse, q_off) in enumerate(runs):
        o1, l1 = eb.ring_local(qd, blocks, causal=True, q_off=q_off)
        t.cuda.synchronize()
        assert t.equal(o1, o) and t.equal(l1, lse), f"{dtype} call {i}: ring_local_noalloc differs from ring_local"


def test_noalloc_rejects_a_share_above_the_scratch(eb):
    t = torch()
    d, n = 128, 8
    B, H = 1, (eb.NOALLOC_SCRATCH_BYTES // (n * (d + 1) * 4)) + 1
    q = t.zeros((B, H, n, d), dtype=t.bfloat16, device="cuda")
    blocks = [(q, q, 0), (q, q, n)]
    o = t.empty_like(q)
    lse = t.empty((B, H, n), dtype=t.float32, device="cuda")
    rc = _call_noalloc(eb, q, blocks, o, lse, 2 * n)
    assert rc == eb.ATTN_EWORKSPACE, (rc, eb.last_error())
    assert "scratch" in eb.last_error()
