"""Pins of the float64 oracle against facts outside itself.

The pages print no worked numeric attention example, so the oracle is pinned by: a pure-Python brute force of
the textbook softmax (no max shift, math.fsum), hand-derived closed forms, invariants (probability rows,
shift invariance, permutation invariance), special cases that reduce to a library routine (torch's float64
scaled_dot_product_attention), the LSE identity (merging the partials of any key partition equals the unsplit
result), and a constructed mask probe whose output is an integer position. The last group plants plausible
mistakes in copies of the oracle and checks that these pins catch each of them.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import mask_probe_inputs

INF = float("inf")


# ----------------------------------------------------------------------------------------------------------
# brute force: textbook softmax written as scalar loops
def brute_attention(q, k, v, scale, causal, q_off, k_off, stride):
    """Per query row: weights e^{s_ij} / sum_visible e^{s_ik}; lse = log of that sum (no max shift)."""
    nq, d = q.shape
    nk, dv = v.shape
    o = np.zeros((nq, dv))
    lse = np.full(nq, -INF)
    for i in range(nq):
        vis = [j for j in range(nk) if (not causal) or (k_off + j * stride <= q_off + i * stride)]
        if not vis:
            continue
        e = {j: math.exp(scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(d))) for j in vis}
        z = math.fsum(e.values())
        for c in range(dv):
            o[i, c] = math.fsum(e[j] * float(v[j, c]) for j in vis) / z
        lse[i] = math.log(z)
    return o, lse


def _cases():
    rng = np.random.default_rng(1234)
    shapes = [(1, 1, 1, 1), (5, 7, 3, 3), (8, 3, 4, 2), (12, 12, 8, 8), (6, 14, 2, 5)]
    out = []
    for nq, nk, d, dv in shapes:
        for causal in (False, True):
            for q_off, k_off, stride in [(0, 0, 1), (3, 0, 1), (0, 4, 1), (2, 1, 4), (1, 3, 4),
                                         (int(rng.integers(-20, 21)), int(rng.integers(-20, 21)), 2)]:
                out.append((nq, nk, d, dv, causal, q_off, k_off, stride))
    return out


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def check_against_brute(impl, case, seed=0):
    nq, nk, d, dv, causal, q_off, k_off, stride = case
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, dv)
    scale = 1.0 / math.sqrt(d)
    o, lse = impl(q[None, None], k[None, None], v[None, None], scale, causal, q_off, k_off, stride)
    ob, lb = brute_attention(q, k, v, scale, causal, q_off, k_off, stride)
    same_inf = np.array_equal(np.isneginf(lse[0, 0]), np.isneginf(lb))
    fin = np.isfinite(lb)
    err_l = np.max(np.abs(lse[0, 0][fin] - lb[fin]), initial=0.0)
    err_o = np.max(np.abs(o[0, 0] - ob), initial=0.0)
    return same_inf, max(err_l, err_o)


def _oracle_impl(q, k, v, scale, causal, q_off, k_off, stride):
    return oracle.attention(q, k, v, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride)


@pytest.mark.parametrize("case", _cases())
def test_oracle_matches_brute_force(case):
    same_inf, err = check_against_brute(_oracle_impl, case)
    assert same_inf
    assert err < 1e-13


# ----------------------------------------------------------------------------------------------------------
# hand-derived closed forms
def test_hand_worked_d1():
    # d=1, scale=1, queries [1, 1], keys [0, ln 3], values [0, 1]: the two scores of a query are 0 and ln 3,
    # so the softmax weights are 1/4 and 3/4. Non-causal: every row gives o = 3/4, lse = ln 4. Causal: row 0
    # sees only key 0 (o = 0, lse = 0); row 1 sees both (o = 3/4, lse = ln 4). Merging the two single-key
    # partials of row 1, (0, 0) and (1, ln 3), gives (3/4, ln 4) again.
    q = np.array([1.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    v = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    o, lse = oracle.attention(q, k, v, 1.0, causal=False)
    np.testing.assert_allclose(o[0, 0, :, 0], [0.75, 0.75], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [math.log(4.0)] * 2, rtol=0, atol=1e-15)
    o, lse = oracle.attention(q, k, v, 1.0, causal=True)
    np.testing.assert_allclose(o[0, 0, :, 0], [0.0, 0.75], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [0.0, math.log(4.0)], rtol=0, atol=1e-15)
    om, lm = oracle.lse_merge(np.array([0.0]), np.array([0.0]), np.array([1.0]), np.array([math.log(3.0)]))
    assert abs(om[0] - 0.75) < 1e-15 and abs(lm[0] - math.log(4.0)) < 1e-15


def test_q_zero_uniform_weights():
    # Q = 0: all scores 0, the weights are uniform over the visible keys: o_i is the mean of the visible values
    # (a prefix mean for causal) and lse_i = log(number of visible keys).
    rng = np.random.default_rng(7)
    n, d = 40, 6
    v = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    q = np.zeros((n, d))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3, causal=True)
    counts = np.arange(1, n + 1)
    prefix_mean = np.cumsum(v, axis=0) / counts[:, None]
    np.testing.assert_allclose(o[0, 0], prefix_mean, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=0, atol=1e-14)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3, causal=False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v.mean(axis=0), (n, d)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.full(n, math.log(n)), rtol=0, atol=1e-14)


def test_single_key_and_first_causal_row():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 5, 4))
    k = rng.standard_normal((1, 1, 1, 4))
    v = rng.standard_normal((1, 1, 1, 3))
    o, lse = oracle.attention(q, k, v, 0.5, causal=False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (5, 3)), rtol=0, atol=1e-15)
    for i in range(5):
        assert abs(lse[0, 0, i] - 0.5 * math.fsum(q[0, 0, i] * k[0, 0, 0])) < 1e-14
    k2 = rng.standard_normal((1, 1, 9, 4))
    v2 = rng.standard_normal((1, 1, 9, 3))
    o, _ = oracle.attention(q, k2, v2, 0.5, causal=True)
    np.testing.assert_allclose(o[0, 0, 0], v2[0, 0, 0], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------------------------------------
# invariants
@pytest.mark.parametrize("causal,q_off,k_off,stride", [(False, 0, 0, 1), (True, 0, 0, 1), (True, 2, 5, 1),
                                                       (True, 1, 3, 4), (True, 3, 1, 4)])
def test_probability_rows(causal, q_off, k_off, stride):
    # With V the identity (dv = Nk), row i of the output IS row i of the attention matrix P: entries are
    # non-negative, zero on masked keys, and each non-empty row sums to 1; empty rows are all zero, lse -inf.
    rng = np.random.default_rng(9)
    nq, nk, d = 11, 13, 5
    q, k = rng.standard_normal((nq, d)), rng.standard_normal((nk, d))
    o, lse = oracle.attention(q[None, None], k[None, None], np.eye(nk)[None, None], 0.7, causal, q_off, k_off,
                              stride)
    p = o[0, 0]
    vis = np.array([[(not causal) or (k_off + j * stride <= q_off + i * stride) for j in range(nk)]
                    for i in range(nq)])
    assert (p >= 0).all()
    assert (p[~vis] == 0).all()
    nonempty = vis.any(axis=1)
    np.testing.assert_allclose(p[nonempty].sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (p[~nonempty] == 0).all() and np.isneginf(lse[0, 0][~nonempty]).all()
    assert np.isfinite(lse[0, 0][nonempty]).all()


def test_shift_invariance_large_scores():
    # Adding a constant c to every score of a row leaves o unchanged and shifts lse by exactly c. Realised by
    # an extra dimension (q_extra = c / scale, k_extra = 1). With c = 900 a textbook exp would overflow.
    rng = np.random.default_rng(10)
    nq, nk, d = 9, 17, 4
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, 3))
    scale, c = 0.5, 900.0
    o0, l0 = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal=True)
    q1 = np.concatenate([q, np.full((nq, 1), c / scale)], axis=1)
    k1 = np.concatenate([k, np.ones((nk, 1))], axis=1)
    o1, l1 = oracle.attention(q1[None, None], k1[None, None], v[None, None], scale, causal=True)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1 - c, l0, rtol=0, atol=1e-11)


def test_permutation_invariance_noncausal():
    rng = np.random.default_rng(11)
    q, k, v = rng.standard_normal((7, 5)), rng.standard_normal((19, 5)), rng.standard_normal((19, 4))
    perm = rng.permutation(19)
    o0, l0 = oracle.attention(q[None, None], k[None, None], v[None, None], 0.4)
    o1, l1 = oracle.attention(q[None, None], k[perm][None, None], v[perm][None, None], 0.4)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-14)


def test_row_subset_is_exact():
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((2, 3, 20, 4)), rng.standard_normal((2, 3, 25, 4)), rng.standard_normal(
        (2, 3, 25, 4))
    rows = np.array([0, 3, 19, 7])
    o, l = oracle.attention(q, k, v, 0.5, causal=True, q_off=5)
    os_, ls = oracle.attention(q, k, v, 0.5, causal=True, q_off=5, rows=rows)
    np.testing.assert_array_equal(os_, o[:, :, rows])
    np.testing.assert_array_equal(ls, l[:, :, rows])


# ----------------------------------------------------------------------------------------------------------
# a library routine as a third opinion
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    B, H, nq, nk, d = 2, 3, 17, 23, 8
    q, k, v = rng.standard_normal((B, H, nq, d)), rng.standard_normal((B, H, nk, d)), rng.standard_normal(
        (B, H, nk, d))
    q_off = nk  # every query row sees at least one key
    mask = torch.from_numpy(oracle.visible(nq, nk, causal, q_off=q_off - 10, k_off=0))
    scale = 1 / math.sqrt(d)
    t = lambda x: torch.from_numpy(x)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=scale)
    s = torch.matmul(t(q), t(k).transpose(-1, -2)) * scale
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -float("inf")), dim=-1)
    o, lse = oracle.attention(q, k, v, scale, causal=causal, q_off=q_off - 10, k_off=0)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------------------------------------
# the merge
def _partition_check(merge_many, attn, causal, stride, q_off, splits, seed=14, n_total=None):
    """Attention over the whole key set vs the merge of attention over a partition of it."""
    rng = np.random.default_rng(seed)
    nk = sum(splits)
    nq, d = 9, 6
    q, k, v = rng.standard_normal((1, 2, nq, d)), rng.standard_normal((1, 2, nk, d)), rng.standard_normal(
        (1, 2, nk, 5))
    o_full, l_full = attn(q, k, v, 0.45, causal=causal, q_off=q_off, k_off=0, stride=stride)
    parts, start = [], 0
    for n in splits:
        parts.append(attn(q, k[:, :, start:start + n], v[:, :, start:start + n], 0.45, causal=causal, q_off=q_off,
                          k_off=start * stride, stride=stride))
        start += n
    order = np.random.default_rng(seed + 1).permutation(len(parts))
    o_m, l_m = merge_many([parts[i] for i in order])
    same_inf = np.array_equal(np.isneginf(l_m), np.isneginf(l_full))
    fin = np.isfinite(l_full)
    return same_inf, max(np.max(np.abs(o_m - o_full)), np.max(np.abs(l_m[fin] - l_full[fin]), initial=0.0))


def _attn(q, k, v, scale, causal, q_off, k_off, stride):
    if k.shape[2] == 0:
        B, H, nq, _ = q.shape
        return np.zeros((B, H, nq, v.shape[3])), np.full((B, H, nq), -INF)
    return oracle.attention(q, k, v, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride)


@pytest.mark.parametrize("causal,stride,q_off", [(False, 1, 0), (True, 1, 0), (True, 1, 6), (True, 2, 3),
                                                 (True, 1, -3)])
@pytest.mark.parametrize("splits", [[7], [3, 4], [1, 5, 0, 8, 2], [10, 1, 1, 3]])
def test_lse_identity(causal, stride, q_off, splits):
    same_inf, err = _partition_check(oracle.lse_merge_many, _attn, causal, stride, q_off, splits)
    assert same_inf and err < 1e-13


def test_merge_with_empty_is_identity_and_pairwise_agrees():
    rng = np.random.default_rng(15)
    o, l = rng.standard_normal((6, 4)), rng.standard_normal(6) * 5
    z, zl = np.zeros((6, 4)), np.full(6, -INF)
    om, lm = oracle.lse_merge(o, l, z, zl)
    np.testing.assert_array_equal(om, o)
    np.testing.assert_array_equal(lm, l)
    om, lm = oracle.lse_merge(z, zl, z, zl)
    assert (om == 0).all() and np.isneginf(lm).all()
    a, b = rng.standard_normal(50) * 30, rng.standard_normal(50) * 30
    _, lm = oracle.lse_merge(np.zeros((50, 1)), a, np.zeros((50, 1)), b)
    np.testing.assert_allclose(lm, oracle.lse_pair(a, b), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lm, np.logaddexp(a, b), rtol=0, atol=1e-13)


def test_ring_and_stripe_shares_equal_global_rows():
    # One ring rank's share (contiguous blocks, global offsets) and one stripe's share (stride W) merged over
    # their K/V blocks equal the rows of plain causal attention over the global sequence at the shard's
    # global positions.
    rng = np.random.default_rng(16)
    N, W, d = 64, 4, 8
    Q, K, V = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    o_g, l_g = oracle.attention(Q, K, V, 0.35, causal=True)
    n = N // W
    for r in range(W):
        # contiguous: rank r holds rows [r*n, (r+1)*n), blocks s hold keys [s*n, (s+1)*n)
        parts = [oracle.attention(Q[:, :, r * n:(r + 1) * n], K[:, :, s * n:(s + 1) * n], V[:, :, s * n:(s + 1) * n],
                                  0.35, causal=True, q_off=r * n, k_off=s * n) for s in range(W)]
        o, l = oracle.lse_merge_many(parts)
        np.testing.assert_allclose(o, o_g[:, :, r * n:(r + 1) * n], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_g[:, :, r * n:(r + 1) * n], rtol=0, atol=1e-13)
        # striped: stripe r holds tokens t = W*i + r
        parts = [oracle.attention(Q[:, :, r::W], K[:, :, s::W], V[:, :, s::W], 0.35, causal=True, q_off=r, k_off=s,
                                  stride=W) for s in range(W)]
        o, l = oracle.lse_merge_many(parts)
        np.testing.assert_allclose(o, o_g[:, :, r::W], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, l_g[:, :, r::W], rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------------------------------------
# constructed mask probe: the output is the digits of the last visible key position
@pytest.mark.parametrize("nq,nk,q_off,k_off,stride", [(20, 30, 0, 0, 1), (16, 16, 2, 1, 4), (16, 16, 1, 3, 4),
                                                      (10, 40, 100, 90, 1), (12, 12, 0, 20, 1)])
def test_mask_probe(nq, nk, q_off, k_off, stride):
    q, k, v = mask_probe_inputs(nq, nk, q_off, k_off, stride)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 1 / math.sqrt(128), causal=True,
                              q_off=q_off, k_off=k_off, stride=stride)
    for i in range(nq):
        q_pos = q_off + i * stride
        vis = [k_off + j * stride for j in range(nk) if k_off + j * stride <= q_pos]
        if not vis:
            assert np.isneginf(lse[0, 0, i]) and (o[0, 0, i] == 0).all()
            continue
        p = max(vis)
        np.testing.assert_allclose(o[0, 0, i], [p // 4096, (p // 64) % 64, p % 64], rtol=0, atol=1e-9)


# ----------------------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
def _mutant_transposed(q, k, v, scale, causal, q_off, k_off, stride):
    # scores from K.Q^T instead of Q.K^T (only shape-compatible when nq == nk)
    return oracle.attention(k, q, v, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride)


def _mutant_strict_causal(q, k, v, scale, causal, q_off, k_off, stride):
    # diagonal excluded: equivalent to shifting every key one position later
    return oracle.attention(q, k, v, scale, causal=causal, q_off=q_off, k_off=k_off + 1, stride=stride)


def _mutant_no_scale(q, k, v, scale, causal, q_off, k_off, stride):
    return oracle.attention(q, k, v, 1.0, causal=causal, q_off=q_off, k_off=k_off, stride=stride)


def _mutant_log2_lse(q, k, v, scale, causal, q_off, k_off, stride):
    o, l = oracle.attention(q, k, v, scale, causal=causal, q_off=q_off, k_off=k_off, stride=stride)
    return o, l / math.log(2.0)


@pytest.mark.parametrize("mutant", [_mutant_transposed, _mutant_strict_causal, _mutant_no_scale, _mutant_log2_lse])
def test_planted_attention_mistakes_are_caught(mutant):
    caught = False
    for case in _cases():
        nq, nk, d, dv, causal, *_ = case
        if mutant is _mutant_transposed and nq != nk:
            continue
        if mutant is _mutant_strict_causal and not causal:
            continue
        same_inf, err = check_against_brute(mutant, case)
        if (not same_inf) or err > 1e-6:
            caught = True
            break
    assert caught


def _merge_garbled_sign(parts):
    # the pairwise formula exactly as printed, with +|a-b| in the exponent, folded over the parts
    (o, l), rest = parts[0], parts[1:]
    for o2, l2 in rest:
        with np.errstate(invalid="ignore", over="ignore"):
            new = np.maximum(l, l2) + np.log1p(np.exp(np.abs(l - l2)))
        new = np.where(np.isneginf(np.maximum(l, l2)), -INF, new)
        wa = np.where(np.isfinite(l), np.exp(l - np.where(np.isfinite(new), new, 0)), 0)
        wb = np.where(np.isfinite(l2), np.exp(l2 - np.where(np.isfinite(new), new, 0)), 0)
        o = wa[..., None] * o + wb[..., None] * o2
        l = new
    return o, l


def _merge_no_rescale(parts):
    # sums of the partial outputs weighted by exp(lse) without the common maximum -- and no division
    o = sum(np.exp(np.where(np.isfinite(l), l, -INF))[..., None] * o for o, l in parts)
    l = np.log(sum(np.exp(l) for _, l in parts))
    return o, l


def _blockwise_without_rescale(q, k, v, scale, causal, q_off, k_off, stride, block=3):
    """The blockwise forward with the accumulator never rescaled when the running maximum grows."""
    B, H, nq, _ = q.shape
    nk = k.shape[2]
    o = np.zeros((B, H, nq, v.shape[3]))
    m = np.full((B, H, nq), -INF)
    s_run = np.zeros((B, H, nq))
    vis_all = oracle.visible(nq, nk, causal, q_off, k_off, stride)
    for j0 in range(0, nk, block):
        s = scale * np.einsum("bhid,bhjd->bhij", q, k[:, :, j0:j0 + block])
        vis = vis_all[:, j0:j0 + block]
        s = np.where(vis, s, -INF)
        new_m = np.maximum(m, s.max(axis=-1))
        sh = np.where(np.isfinite(new_m), new_m, 0)
        s_run = np.where(np.isfinite(m), np.exp(m - sh), 0) * s_run + np.exp(s - sh[..., None]).sum(-1)
        m = new_m
        o = o + np.exp(s - sh[..., None]) @ v[:, :, j0:j0 + block]       # no rescale of o
    with np.errstate(divide="ignore", invalid="ignore"):
        return o / s_run[..., None], np.where(np.isfinite(m), m + np.log(s_run), -INF)


@pytest.mark.parametrize("merge", [_merge_garbled_sign, _merge_no_rescale])
def test_planted_merge_mistakes_are_caught(merge):
    results = []
    for splits in ([3, 4], [1, 5, 0, 8, 2]):
        with np.errstate(all="ignore"):
            same_inf, err = _partition_check(merge, _attn, False, 1, 0, splits)
        results.append((not same_inf) or not (err < 1e-6))
    assert any(results)


def test_planted_missing_rescale_is_caught():
    caught = False
    for case in _cases():
        same_inf, err = check_against_brute(_blockwise_without_rescale, case)
        if (not same_inf) or not (err < 1e-6):
            caught = True
            break
    assert caught
