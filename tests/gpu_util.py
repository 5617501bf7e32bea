"""Helpers shared by the GPU tests: move seeded host arrays to the device and results back, and compare
against the float64 oracle with the tolerances of the parity bar."""
from __future__ import annotations

import numpy as np

from workloads import bf16_bits_to_f64

# Parity bar: fp32 paths 1e-5 max-abs; bf16 paths 2e-2 max-abs on o; lse 1e-3; -inf rows matched exactly.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE = 1e-3


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(t.bfloat16)


def dev_f32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t_) -> np.ndarray:
    t = torch()
    if t_.dtype == t.bfloat16:
        return bf16_bits_to_f64(t_.contiguous().view(t.int16).cpu().numpy().view(np.uint16))
    return t_.cpu().numpy().astype(np.float64)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, tol_o, tol_l=TOL_LSE, what=""):
    """Element-wise comparison; -inf lse rows must match exactly (and their o rows be 0)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape and lse_gpu.shape == lse_ref.shape, (o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite output"
    ref_empty = np.isneginf(lse_ref)
    got_empty = np.isneginf(lse_gpu)
    assert np.array_equal(ref_empty, got_empty), f"{what}: -inf rows differ ({ref_empty.sum()} vs {got_empty.sum()})"
    assert (o_gpu[got_empty] == 0).all(), f"{what}: empty rows must be 0"
    fin = ~ref_empty
    err_o = float(np.max(np.abs(o_gpu - o_ref), initial=0.0))
    err_l = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]), initial=0.0))
    print(f"[parity] {what}: max|do|={err_o:.3e} (tol {tol_o:g}) max|dlse|={err_l:.3e} (tol {tol_l:g})", flush=True)
    assert err_o <= tol_o, f"{what}: o error {err_o} > {tol_o}"
    assert err_l <= tol_l, f"{what}: lse error {err_l} > {tol_l}"
    return err_o, err_l


def sample_rows(n: int, tile: int, count: int, rng, extra=()) -> np.ndarray:
    """Random rows plus structurally risky ones: 0-7, the last 8, first/last row of every query tile
    (for up to 64 tiles spread over the range), and any caller-given rows."""
    rows = set(int(x) for x in rng.choice(n, size=min(count, n), replace=False))
    rows.update(range(min(8, n)))
    rows.update(range(max(0, n - 8), n))
    n_t = (n + tile - 1) // tile
    for t in np.linspace(0, n_t - 1, num=min(n_t, 64)).astype(int):
        rows.add(int(t * tile))
        rows.add(int(min(n - 1, t * tile + tile - 1)))
    rows.update(int(r) for r in extra if 0 <= r < n)
    return np.array(sorted(rows), dtype=np.int64)
