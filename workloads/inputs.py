"""Seeded input generators.

Every tensor is drawn per (tensor, batch, head) slab from its own ``numpy.random.SeedSequence`` so that any
single head can be regenerated alone (the parity tests recompute only the heads they sample) and so that slabs
can be drawn in parallel threads (numpy releases the GIL while filling).

Values are iid standard normal in float32. bfloat16 inputs are the round-to-nearest-even bfloat16 of those
float32 draws; the HIP path receives these 16-bit patterns and the oracle receives the same values widened
exactly to float64, so input quantisation is never counted as error.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Stable small integers naming the tensors that a workload draws; part of every slab's seed.
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "o_a": 4, "o_b": 5, "lse_a": 6, "lse_b": 7, "do": 8}

_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even; returns the uint16 bit patterns.

    NaN inputs stay NaN (quiet bit forced); infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _slab_rng(seed: int, tensor: str, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), TENSOR_IDS[tensor], b, h])))


def _draw(seed: int, tensor: str, shape, heads=None) -> np.ndarray:
    """float32 N(0,1) array of ``shape`` = (B, H, *slab); slab (b, h) comes from its own seed.

    ``heads``: optional list of (b, h) pairs; only those slabs are drawn, the rest stay zero.
    """
    shape = tuple(int(s) for s in shape)
    B, H = shape[0], shape[1]
    slab = shape[2:]
    out = np.zeros(shape, dtype=np.float32)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)

    def fill(bh):
        b, h = bh
        out[b, h] = _slab_rng(seed, tensor, b, h).standard_normal(slab, dtype=np.float32)

    if len(todo) == 1:
        fill(todo[0])
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, todo))
    return out


def normal_f32(seed: int, tensor: str, shape, heads=None) -> np.ndarray:
    """Seeded iid N(0,1) float32 tensor of shape (B, H, ...)."""
    return _draw(seed, tensor, shape, heads)


def normal_bf16_bits(seed: int, tensor: str, shape, heads=None) -> np.ndarray:
    """Seeded iid N(0,1) tensor of shape (B, H, ...), rounded to bfloat16; returns uint16 bit patterns."""
    x = _draw(seed, tensor, shape, heads)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24

    def conv(i):
        out[i:i + step] = f32_to_bf16_bits(flat[i:i + step])

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(conv, range(0, flat.size, step)))
    return out.reshape(x.shape)


def normal_bf16_slab(seed: int, tensor: str, b: int, h: int, slab_shape) -> np.ndarray:
    """The (b, h) slab of normal_bf16_bits(seed, tensor, (B, H, *slab_shape)) alone, drawn from the same seed
    (uint16 bit patterns of shape slab_shape)."""
    x = _slab_rng(seed, tensor, b, h).standard_normal(tuple(int(s) for s in slab_shape), dtype=np.float32)
    return f32_to_bf16_bits(x)


def mask_probe_inputs(nq: int, nk: int, q_off: int, k_off: int, stride: int, alpha: float = 512.0):
    """Constructed inputs whose attention output names the last visible key position.

    Key j at global position p = k_off + j*stride carries the base-64 digits (a, b, c) of p (p < 64**3) in
    both its key vector and its value vector; every query is (4096*alpha, 64*alpha, alpha), so the score of key
    j is alpha*p exactly. All values are integers of at most 12 significant bits, hence exact in bfloat16.
    With alpha*scale large, the softmax puts all but a negligible weight on the largest visible position, so
    the output row equals that key's digits. Returns float32 arrays q [nq,3], k [nk,3], v [nk,3].
    """
    pos = k_off + stride * np.arange(nk, dtype=np.int64)
    if pos.min() < 0 or pos.max() >= 64 ** 3:
        raise ValueError("mask probe positions must lie in [0, 64**3)")
    digits = np.stack([pos // 4096, (pos // 64) % 64, pos % 64], axis=1).astype(np.float32)
    q = np.tile(np.array([4096 * alpha, 64 * alpha, alpha], dtype=np.float32), (nq, 1))
    return q, digits.copy(), digits.copy()
