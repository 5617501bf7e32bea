"""GPU parity of ring_local_pipelined: one device's share of Ring Attention with the exchange step overlapped
(incoming K/V blocks copied into receive slots on a second stream while the compute stream attends).

The result must equal ring_local over the same blocks bit for bit (same kernels, same merge order) and the
float64 oracle over the union of the keys to the bf16 bar. Incoming blocks come from pinned host memory (the
stand-in for the link to the neighbouring device) and from device memory; runs of many small blocks make each
receive slot be refilled several times.
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


def _host_bf16(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).pin_memory()


def _run(eb, P, r, n, H, d, stride_mode, source, seed):
    """Rank r of P, block size n: contiguous (q_off = r*n, k_off = s*n) or striped (stride P)."""
    t = torch()
    N = P * n
    Q = normal_bf16_bits(seed, "q", (1, H, N, d))
    K = normal_bf16_bits(seed, "k", (1, H, N, d))
    V = normal_bf16_bits(seed, "v", (1, H, N, d))
    if stride_mode:
        sel = [np.arange(s, N, P) for s in range(P)]
        q_off, stride, offs = r, P, list(range(P))
    else:
        sel = [np.arange(s * n, (s + 1) * n) for s in range(P)]
        q_off, stride, offs = r * n, 1, [s * n for s in range(P)]
    qd = dev_bf16(np.ascontiguousarray(Q[:, :, sel[r]]))
    order = [(r - i) % P for i in range(P)]                    # the ring's arrival order, own block first
    blocks_dev, blocks_pipe = [], []
    for i, s in enumerate(order):
        kb, vb = np.ascontiguousarray(K[:, :, sel[s]]), np.ascontiguousarray(V[:, :, sel[s]])
        kd, vd = dev_bf16(kb), dev_bf16(vb)
        blocks_dev.append((kd, vd, offs[s]))
        if i > 0 and (source == "host" or (source == "mixed" and i % 2 == 1)):
            blocks_pipe.append((_host_bf16(kb), _host_bf16(vb), offs[s]))
        else:
            blocks_pipe.append((kd, vd, offs[s]))
    scale = 1 / math.sqrt(d)
    o1, l1 = eb.ring_local(qd, blocks_dev, scale=scale, causal=True, q_off=q_off, pos_stride=stride)
    o2, l2 = eb.ring_local_pipelined(qd, blocks_pipe, scale=scale, causal=True, q_off=q_off, pos_stride=stride)
    t.cuda.synchronize()
    assert t.equal(o1, o2) and t.equal(l1, l2), "pipelined ring differs from ring_local"
    # the oracle over the union of the blocks: each block by its own positions, merged by the oracle's merge
    qf = bf16_bits_to_f64(Q[:, :, sel[r]])
    parts = [oracle.attention(qf, bf16_bits_to_f64(K[:, :, sel[s]]), bf16_bits_to_f64(V[:, :, sel[s]]), scale,
                              causal=True, q_off=q_off, k_off=offs[s], stride=stride) for s in range(P)]
    o_ref, l_ref = oracle.lse_merge_many(parts)
    compare(host_f64(o2), host_f64(l2), o_ref, l_ref, TOL_BF16, TOL_LSE, what=f"P{P} r{r} {source}")


@pytest.mark.parametrize("P,r,stride_mode", [(4, 2, False), (4, 3, False), (4, 0, False), (4, 1, True),
                                             (3, 2, True)])
@pytest.mark.parametrize("source", ["host", "device", "mixed"])
def test_pipelined_ring_share(eb, P, r, stride_mode, source):
    print(f"[case] pipelined ring P={P} r={r} striped={stride_mode} source={source}", flush=True)
    _run(eb, P, r, 160, 2, 128, stride_mode, source, 51)


def test_pipelined_ring_many_small_blocks(eb):
    """Eight ranks, the last one (every block live): each receive slot is refilled several times; twice in a row."""
    for rep in range(2):
        print(f"[case] pipelined ring P=8 r=7 rep={rep}", flush=True)
        _run(eb, 8, 7, 64, 2, 64, False, "mixed", 52 + rep)


def test_pipelined_ring_edge_blocks(eb):
    t = torch()
    H, n, d = 2, 100, 128
    q = normal_bf16_bits(53, "q", (1, H, n, d))
    k = normal_bf16_bits(53, "k", (1, H, n, d))
    v = normal_bf16_bits(53, "v", (1, H, n, d))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    print("[case] pipelined ring edge blocks", flush=True)
    # only the resident block
    o, lse = eb.ring_local_pipelined(qd, [(kd, vd, 0)], causal=True)
    o_ref, l_ref = oracle.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), 1 / math.sqrt(d),
                                    causal=True)
    t.cuda.synchronize()
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what="resident only")
    # resident block hidden (after every query), one incoming live block from the host
    o, lse = eb.ring_local_pipelined(qd, [(kd, vd, 10 * n), (_host_bf16(k), _host_bf16(v), 0)], causal=True)
    t.cuda.synchronize()
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, TOL_BF16, TOL_LSE, what="resident hidden")
    # every block hidden
    o, lse = eb.ring_local_pipelined(qd, [(kd, vd, 10 * n), (_host_bf16(k), _host_bf16(v), 20 * n)], causal=True)
    t.cuda.synchronize()
    assert bool((o == 0).all()) and bool(t.isneginf(lse).all())


def test_pipelined_ring_back_to_back_on_one_workspace(eb):
    """Calls in a row on ONE workspace, different blocks every call, no synchronisation between them:
    * the first incoming block is a device tensor produced on the current stream just before the call, behind a
      long attention launch (the copy stream must wait for it);
    * the next call's copies must not overwrite receive slots the previous call's kernels still read;
    * the host blocks are dropped right after each call and fresh pinned buffers of other values are allocated
      (the binding keeps the dropped ones alive until the compute stream has passed the call).
    Every result must equal ring_local over the same blocks, bit for bit."""
    t = torch()
    P, r, n, H, d = 4, 3, 2048, 8, 128         # rank 3 of 4: every block live, three incoming
    dev = t.device("cuda:0")
    ws = t.empty(eb.ring_local_pipelined_workspace_bytes(1, H, n, d, n), dtype=t.uint8, device=dev)
    busy = [dev_bf16(normal_bf16_bits(70, x, (1, 32, 8192, 128))) for x in "qkv"]
    scale = 1 / math.sqrt(d)
    runs = []
    for it in range(4):
        print(f"[case] pipelined ring back to back, call {it}", flush=True)
        seed = 71 + it
        Q, K, V = (normal_bf16_bits(seed, x, (1, H, P * n, d)) for x in "qkv")
        blk = lambda X, s: np.ascontiguousarray(X[:, :, s * n:(s + 1) * n])    # noqa: E731
        qd = dev_bf16(blk(Q, r))
        order = [(r - i) % P for i in range(P)]
        ref_blocks = [(dev_bf16(blk(K, s)), dev_bf16(blk(V, s)), s * n) for s in order]
        eb.attn_fwd(*busy, causal=False)                                   # a long kernel on the current stream
        k_in, v_in = ref_blocks[1][0] * 1, ref_blocks[1][1] * 1            # produced behind it, same stream
        pipe = [ref_blocks[0], (k_in, v_in, ref_blocks[1][2])]
        pipe += [(_host_bf16(blk(K, s)), _host_bf16(blk(V, s)), s * n) for s in order[2:]]
        o, lse = eb.ring_local_pipelined(qd, pipe, scale=scale, causal=True, q_off=r * n, workspace=ws)
        del pipe, k_in, v_in
        junk = [t.full((1, H, n, d), float(it + 2), dtype=t.bfloat16).pin_memory() for _ in range(4)]
        runs.append((qd, ref_blocks, o, lse, junk))
    t.cuda.synchronize()
    for it, (qd, ref_blocks, o, lse, _) in enumerate(runs):
        o1, l1 = eb.ring_local(qd, ref_blocks, scale=scale, causal=True, q_off=r * n)
        t.cuda.synchronize()
        assert t.equal(o1, o) and t.equal(l1, lse), f"call {it}: pipelined result differs from ring_local"
