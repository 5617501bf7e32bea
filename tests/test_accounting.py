"""Pins of the FLOP/byte accounting: the pages' printed closed forms, and brute-force pair counts."""
import os

import numpy as np
import pytest

import oracle
from workloads import accounting as acc
from workloads.configs import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_closed_forms.txt")


def _golden_lines():
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


@pytest.mark.parametrize("fields", list(_golden_lines()), ids=lambda f: " ".join(f))
def test_pages_closed_forms(fields):
    name, *args = fields
    args = [int(a) for a in args]
    expected = args[-1]
    if name == "score_matrix_gib_rounded":
        got = round(acc.score_matrix_bytes(args[0], args[1]) / 2 ** 30)
    else:
        got = getattr(acc, name)(*args[:-1])
    assert got == expected


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_off,k_off,stride", [(0, 0, 1), (5, 0, 1), (0, 7, 1), (3, 1, 4), (1, 3, 4),
                                                (-9, 4, 2), (40, 0, 1), (0, 40, 1)])
def test_visible_pairs_brute_force(causal, q_off, k_off, stride):
    for nq, nk in [(1, 1), (7, 5), (16, 16), (13, 29)]:
        brute = int(oracle.visible(nq, nk, causal, q_off, k_off, stride).sum())
        assert acc.visible_pairs(nq, nk, causal, q_off, k_off, stride) == brute


def test_config_pair_counts():
    # closed forms: causal self-attention n(n+1)/2 per head; ring rank 2 of 4 sees 2 full blocks plus a
    # diagonal block; stripe r sees 2n^2 + n(r-1) pairs per head over the four stripes.
    c2 = CONFIGS["causal_8k"]
    assert acc.config_pairs(c2) == 4 * 32 * 8192 * 8193 // 2
    c3 = CONFIGS["ring_rank2of4_128k"]
    n = 32768
    assert acc.config_pairs(c3) == 32 * (2 * n * n + n * (n + 1) // 2)
    for r in range(4):
        c4 = CONFIGS[f"striped_r{r}_64k"]
        n = 16384
        assert acc.config_pairs(c4) == 16 * (2 * n * n + n * (r - 1))
    c1 = CONFIGS["tiny_f32"]
    assert acc.config_pairs(c1) == 256 * 256
    assert acc.attention_flops(acc.config_pairs(c2), 128) == pytest.approx(2.199e12, rel=1e-3)


def test_merge_and_fwd_bytes():
    # c3 merge: 1,048,576 rows of fp32 partials with d=128 -> 1548 bytes per row
    assert acc.merge_bytes(1, 128, 4, 4) == 1548
    assert acc.merge_bytes(32 * 32768, 128, 4, 4) == 1548 * 1048576
    assert acc.attn_fwd_bytes(1, 1, 10, 10, 4, 2, 2) == 10 * 4 * 2 * 3 + 10 * 4 * 2 + 40
    assert np.isclose(acc.merge_bytes(32 * 32768, 128, 4, 4) / 1e9, 1.623, atol=1e-3)


@pytest.mark.parametrize("nq,nk,q_off,k_off,stride,window", [
    (20, 20, 0, 0, 1, 5), (16, 30, 3, 0, 1, 7), (9, 9, 2, 1, 4, 9), (12, 12, 1, 3, 4, 2), (50, 40, -7, 3, 2, 11),
    (10, 10, 0, 0, 1, 100), (33, 33, 0, 0, 1, 1)])
def test_windowed_pair_counts_brute_force(nq, nk, q_off, k_off, stride, window):
    brute = sum(1 for i in range(nq) for j in range(nk)
                if q_off + i * stride - window < k_off + j * stride <= q_off + i * stride)
    assert acc.visible_pairs(nq, nk, True, q_off, k_off, stride, window=window) == brute


def test_windowed_pair_count_closed_form():
    # self-attention over N tokens with a window of w <= N: w(w+1)/2 pairs for the first w rows, w per row after
    n, w = 32768, 4096
    assert acc.visible_pairs(n, n, True, window=w) == w * (w + 1) // 2 + (n - w) * w
