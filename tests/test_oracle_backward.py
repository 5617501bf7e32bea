"""Pins of the oracle's backward pass (gradients of exact attention with respect to q, k and v).

Source: "深度学习注意力机制优化与FlashAttention实践", §4.1 item 3 and §3.3 (the backward recomputes the attention
weights). The pages give no gradient formulas; the oracle's reading is the exact gradient of the forward
definition. It is pinned here by facts that do not use its formulas:
  * central finite differences of the forward oracle (a different computation: only forward evaluations),
  * torch autograd through a float64 softmax attention written with library calls,
  * closed forms (window 1: o_i = v_i; constant value rows: o does not depend on q or k; q = 0: uniform weights),
  * invariants (the key gradients of a row sum to zero; q.dq = k.dk from the bilinear scores, equal to
    scale * dL/dscale; linearity in do; delta_i = do_i . o_i),
  * planted mistakes: each is a one-line change to the oracle's own source, and a pin above must fail on it.
"""
import importlib
import inspect
import math

import numpy as np
import pytest

import oracle

oracle_attention_module = importlib.import_module("oracle.attention")


def _loss(q, k, v, do, scale, **mask):
    o, _ = oracle.attention(q, k, v, scale, **mask)
    return math.fsum((o * do).ravel())


def _finite_diff(q, k, v, do, scale, h=1e-5, **mask):
    """Central differences of L = sum(do * o) for every element of q, k and v."""
    grads = []
    for which in range(3):
        xs = [q.copy(), k.copy(), v.copy()]
        x = xs[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(*xs, do, scale, **mask)
            x[idx] = x0 - h
            lm = _loss(*xs, do, scale, **mask)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def _inputs(seed, B, H, Hkv, nq, nk, d, dv):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, nq, d)), rng.standard_normal((B, Hkv, nk, d)),
            rng.standard_normal((B, Hkv, nk, dv)), rng.standard_normal((B, H, nq, dv)))


# (B, H, Hkv, nq, nk, d, dv, mask kwargs)
FD_CASES = [
    (1, 1, 1, 4, 5, 3, 2, {}),
    (1, 2, 2, 5, 5, 3, 3, {"causal": True}),
    (1, 2, 1, 6, 4, 2, 3, {"causal": True, "q_off": 2, "k_off": 0}),
    (1, 1, 1, 5, 5, 3, 2, {"causal": True, "q_off": 1, "k_off": 3, "stride": 4}),   # striped; row 0 sees nothing
    (1, 1, 1, 6, 7, 3, 2, {"causal": True, "q_off": -2, "k_off": 0}),               # first rows empty
    (1, 4, 2, 6, 6, 2, 2, {"causal": True, "window": 3}),
    (2, 3, 1, 4, 6, 2, 2, {}),                                                     # multi-query
]


@pytest.mark.parametrize("idx", range(len(FD_CASES)))
def test_backward_matches_finite_differences(idx):
    B, H, Hkv, nq, nk, d, dv, mask = FD_CASES[idx]
    q, k, v, do = _inputs(100 + idx, B, H, Hkv, nq, nk, d, dv)
    scale = 0.8
    dq, dk, dvv, _ = oracle.attention_backward(q, k, v, do, scale, **mask)
    fq, fk, fv = _finite_diff(q, k, v, do, scale, **mask)
    for got, ref in ((dq, fq), (dk, fk), (dvv, fv)):
        assert np.max(np.abs(got - ref)) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    B, H, nq, nk, d = 2, 3, 9, 9, 4
    q, k, v, do = _inputs(11 + causal, B, H, H, nq, nk, d, d)
    scale = 0.45
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(~torch.ones(nq, nk, dtype=torch.bool).tril(), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dvv, _ = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    for got, ref in ((dq, tq), (dk, tk), (dvv, tv)):
        assert np.max(np.abs(got - ref.grad.numpy())) < 1e-12


def test_backward_closed_forms():
    rng = np.random.default_rng(4)
    n, d = 7, 3
    q, k, v, do = _inputs(5, 1, 1, 1, n, n, d, d)
    # window 1: o_i = v_i exactly, so dv = do and q, k receive nothing
    dq, dk, dvv, _ = oracle.attention_backward(q, k, v, do, 0.7, causal=True, window=1)
    assert np.max(np.abs(dvv - do)) < 1e-15 and np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15
    # every value row equal: o is that row whatever the weights, so q and k receive nothing
    vc = np.broadcast_to(rng.standard_normal(d), (1, 1, n, d)).copy()
    dq, dk, dvv, _ = oracle.attention_backward(q, k, vc, do, 0.7, causal=True)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # q = 0: weights are uniform over the visible keys, dv_j = sum over the rows i that see j of do_i / (i + 1)
    dq, dk, dvv, _ = oracle.attention_backward(np.zeros_like(q), k, v, do, 0.7, causal=True)
    for j in range(n):
        ref = sum(do[0, 0, i] / (i + 1) for i in range(j, n))
        assert np.max(np.abs(dvv[0, 0, j] - ref)) < 1e-13


@pytest.mark.parametrize("mask", [{}, {"causal": True, "q_off": 3}, {"causal": True, "window": 4},
                                  {"causal": True, "q_off": -3}])
def test_backward_invariants(mask):
    B, H, Hkv, nq, nk, d, dv = 2, 4, 2, 8, 10, 5, 3
    q, k, v, do = _inputs(6, B, H, Hkv, nq, nk, d, dv)
    scale = 0.6
    dq, dk, dvv, delta = oracle.attention_backward(q, k, v, do, scale, **mask)
    # each row's score gradients sum to zero, so the key gradients of every key/value head sum to zero
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    # the scores are bilinear in q and k: q.dq = k.dk = scale * dL/dscale (Euler's identity)
    qdq, kdk = math.fsum((q * dq).ravel()), math.fsum((k * dk).ravel())
    h = 1e-6
    dscale = (_loss(q, k, v, do, scale + h, **mask) - _loss(q, k, v, do, scale - h, **mask)) / (2 * h)
    assert abs(qdq - kdk) < 1e-12 and abs(qdq - scale * dscale) < 1e-7
    # delta_i = do_i . o_i
    o, _ = oracle.attention(q, k, v, scale, **mask)
    assert np.max(np.abs(delta - np.sum(do * o, axis=-1))) < 1e-13
    # linear in do
    do2 = np.random.default_rng(7).standard_normal(do.shape)
    g1 = oracle.attention_backward(q, k, v, do, scale, **mask)
    g2 = oracle.attention_backward(q, k, v, do2, scale, **mask)
    g3 = oracle.attention_backward(q, k, v, do + 2 * do2, scale, **mask)
    for a, b, c in zip(g1, g2, g3):
        assert np.max(np.abs(a + 2 * b - c)) < 1e-12


# planted mistakes: one-line edits of the oracle's own source; the finite-difference pin must catch each
MUTATIONS = [
    ("ds = p * (dp - dl[:, None])", "ds = p * dp"),                                  # Jacobian rank-one part dropped
    ("ds = p * (dp - dl[:, None])", "ds = p * (dp + dl[:, None])"),                  # wrong sign
    ("dq[b, h, rr] = scale * (ds @ k[b, g])", "dq[b, h, rr] = ds @ k[b, g]"),        # scale dropped
    ("dk[b, g] += scale * (ds.T @ q[b, h, rr])", "dk[b, g] = scale * (ds.T @ q[b, h, rr])"),   # group not summed
    ("dv[b, g] += p.T @ do[b, h, rr]", "dv[b, g] += (p.T @ do[b, h, rr]) / max(1, rr.size)"),
    ("dl = np.sum(p * dp, axis=1)", "dl = np.mean(dp, axis=1)"),                      # unweighted row mean
    ("dp = do[b, h, rr] @ v[b, g].T", "dp = do[b, h, rr] @ v[b, 0].T"),               # wrong value head
]


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[str(i) for i in range(len(MUTATIONS))])
def test_planted_backward_mistakes_are_caught(old, new):
    src = inspect.getsource(oracle_attention_module.attention_backward)
    assert src.count(old) == 1
    ns = dict(vars(oracle_attention_module))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mutant = ns["attention_backward"]
    B, H, Hkv, nq, nk, d, dv, mask = (1, 4, 2, 5, 5, 2, 2, {"causal": True})
    q, k, v, do = _inputs(9, B, H, Hkv, nq, nk, d, dv)
    fq, fk, fv = _finite_diff(q, k, v, do, 0.8, **mask)
    dq, dk, dvv, _ = mutant(q, k, v, do, 0.8, **mask)
    err = max(np.max(np.abs(dq - fq)), np.max(np.abs(dk - fk)), np.max(np.abs(dvv - fv)))
    assert err > 1e-4
