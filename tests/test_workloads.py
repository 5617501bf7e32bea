"""Input generator checks: bfloat16 rounding, determinism, per-head regeneration, mask-probe exactness."""
import math

import numpy as np

import oracle
from workloads import (CONFIGS, bf16_bits_to_f64, f32_to_bf16_bits, mask_probe_inputs, normal_bf16_bits,
                       normal_f32)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0, -0.0,
                  float("inf"), 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties -> even (1+2^-6 pattern 0x3F82)
    assert list(bits[:7]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000]
    assert bits[7] == 0x7F80
    assert bits[8] == 0x7F62  # 3e38 rounds within range
    assert np.isnan(bf16_bits_to_f64(f32_to_bf16_bits(np.array([np.nan], dtype=np.float32)))[0])


def test_generation_is_seeded_and_per_head():
    a = normal_bf16_bits(2, "q", (2, 3, 16, 8))
    b = normal_bf16_bits(2, "q", (2, 3, 16, 8))
    assert np.array_equal(a, b)
    c = normal_bf16_bits(2, "q", (2, 3, 16, 8), heads=[(1, 2)])
    assert np.array_equal(c[1, 2], a[1, 2]) and not c[0, 0].any()
    assert not np.array_equal(normal_bf16_bits(2, "k", (2, 3, 16, 8)), a)
    x = normal_f32(1, "v", (1, 1, 20000, 4))
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_single_slab_draw_matches_the_full_tensor():
    from workloads import normal_bf16_slab
    full = normal_bf16_bits(11, "v", (2, 3, 40, 24))
    for b, h in ((0, 0), (1, 2), (0, 1)):
        assert np.array_equal(normal_bf16_slab(11, "v", b, h, (40, 24)), full[b, h])


def test_mask_probe_values_exact_in_bf16():
    q, k, v = mask_probe_inputs(8, 64, 131000, 131000 - 70, 1)
    for a in (q, k, v):
        assert np.array_equal(bf16_bits_to_f64(f32_to_bf16_bits(a)), a.astype(np.float64))


def test_config1_split_merge_equals_unsplit_on_oracle():
    c = CONFIGS["tiny_f32"]
    q = normal_f32(c.seed, "q", (c.B, c.H, c.Nq, c.d)).astype(np.float64)
    k = normal_f32(c.seed, "k", (c.B, c.H, c.Nk_total, c.d)).astype(np.float64)
    v = normal_f32(c.seed, "v", (c.B, c.H, c.Nk_total, c.d)).astype(np.float64)
    o, l = oracle.attention(q, k, v, c.scale)
    parts = [oracle.attention(q, k[:, :, ko:ko + n], v[:, :, ko:ko + n], c.scale) for n, ko in c.blocks]
    om, lm = oracle.lse_merge_many(parts)
    assert np.max(np.abs(om - o)) < 1e-13 and np.max(np.abs(lm - l)) < 1e-13
    assert c.scale == 1 / math.sqrt(64)
