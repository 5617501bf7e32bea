"""The C ABI on the CPU: the library loads, exports every declared function, validates its arguments before
touching the device, and plans ring blocks on the host exactly as the oracle's mask says."""
import ctypes
import subprocess

import numpy as np
import pytest

import oracle

eb = pytest.importorskip("exact_blockwise_attention_amd")
lib = eb.lib
A = 1 << 20          # fake, well-aligned "device" addresses: validation must reject before any use
B16 = 1 << 24


def test_every_declared_symbol_is_exported():
    names = eb.declared_symbols()
    assert set(names) >= {"attn_fwd", "attn_lse_merge", "ring_local", "ring_local_workspace_bytes",
                          "ring_local_plan", "attn_last_error", "attn_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", eb.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.attn_version() == 100


def test_workspace_bytes():
    def a256(x):
        return (x + 255) // 256 * 256
    for B, H, Nq, d in [(1, 32, 32768, 128), (1, 1, 256, 64), (3, 5, 7, 24), (0, 1, 1, 128)]:
        rows = B * H * Nq
        assert eb.ring_local_workspace_bytes(B, H, Nq, d) == 2 * (a256(rows * d * 4) + a256(rows * 4))
    assert eb.ring_local_workspace_bytes(-1, 1, 1, 1) == 0


def fwd(**kw):
    args = dict(q=A, k=A + B16, v=A + 2 * B16, o=A + 3 * B16, lse=A + 4 * B16, B=1, H=2, Nq=64, Nk=64, d=128,
                scale=0.125, causal=1, q_off=0, k_off=0, stride=1, it=eb.ATTN_BF16, ot=eb.ATTN_BF16, stream=None)
    args.update(kw)
    return lib.attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"], args["Nq"],
                        args["Nk"], args["d"], args["scale"], args["causal"], args["q_off"], args["k_off"],
                        args["stride"], args["it"], args["ot"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), eb.ATTN_EINVAL),
    (dict(o=None), eb.ATTN_EINVAL),
    (dict(lse=None), eb.ATTN_EINVAL),
    (dict(k=None), eb.ATTN_EINVAL),
    (dict(B=-1), eb.ATTN_EINVAL),
    (dict(Nq=-3), eb.ATTN_EINVAL),
    (dict(Nk=-3), eb.ATTN_EINVAL),
    (dict(Nq=(1 << 28) + 1), eb.ATTN_EINVAL),
    (dict(causal=2), eb.ATTN_EINVAL),
    (dict(stride=0), eb.ATTN_EINVAL),
    (dict(scale=0.0), eb.ATTN_EINVAL),
    (dict(scale=-1.0), eb.ATTN_EINVAL),
    (dict(scale=float("nan")), eb.ATTN_EINVAL),
    (dict(scale=float("inf")), eb.ATTN_EINVAL),
    (dict(it=7), eb.ATTN_EINVAL),
    (dict(d=32), eb.ATTN_EUNSUPPORTED),
    (dict(d=256), eb.ATTN_EUNSUPPORTED),
    (dict(it=eb.ATTN_F32, ot=eb.ATTN_BF16), eb.ATTN_EUNSUPPORTED),
    (dict(q=A + 8), eb.ATTN_EINVAL),                 # misaligned
    (dict(v=A + 2 * B16 + 4), eb.ATTN_EINVAL),
    (dict(lse=A + 4 * B16 + 2), eb.ATTN_EINVAL),
    (dict(o=A + 16), eb.ATTN_EINVAL),                # o overlaps q
    (dict(lse=A + 3 * B16 + 64), eb.ATTN_EINVAL),    # lse overlaps o
    (dict(o=A + B16 + 256), eb.ATTN_EINVAL),         # o overlaps k
    (dict(q_off=(1 << 62) + 1), eb.ATTN_EINVAL),
    (dict(k_off=-(1 << 62) - 1), eb.ATTN_EINVAL),
])
def test_attn_fwd_validation(kw, code):
    assert fwd(**kw) == code
    assert eb.last_error() != ""


def test_zero_sized_calls_are_noops():
    assert fwd(B=0) == eb.ATTN_OK
    assert fwd(H=0, q=None, o=None, lse=None) == eb.ATTN_OK
    assert fwd(Nq=0) == eb.ATTN_OK
    assert eb.last_error() == ""


def merge(**kw):
    args = dict(oa=A, la=A + B16, ob=A + 2 * B16, lb=A + 3 * B16, o=A + 4 * B16, l=A + 5 * B16, rows=100, d=128,
                pt=eb.ATTN_F32, ot=eb.ATTN_F32)
    args.update(kw)
    return lib.attn_lse_merge(args["oa"], args["la"], args["ob"], args["lb"], args["o"], args["l"], args["rows"],
                              args["d"], args["pt"], args["ot"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), eb.ATTN_EINVAL),
    (dict(d=0), eb.ATTN_EINVAL),
    (dict(d=6), eb.ATTN_EUNSUPPORTED),
    (dict(d=12, pt=eb.ATTN_BF16), eb.ATTN_EUNSUPPORTED),
    (dict(d=260), eb.ATTN_EUNSUPPORTED),
    (dict(pt=3), eb.ATTN_EINVAL),
    (dict(oa=None), eb.ATTN_EINVAL),
    (dict(o=A + 64), eb.ATTN_EINVAL),                  # partial overlap with o_a
    (dict(o=A, ot=eb.ATTN_BF16), eb.ATTN_EINVAL),     # in place needs the same dtype
    (dict(o=A, ob=A), eb.ATTN_EINVAL),                # all three the same buffer
    (dict(l=A + B16 + 4), eb.ATTN_EINVAL),            # partial overlap with lse_a
    (dict(l=A + 4 * B16 + 128), eb.ATTN_EINVAL),      # lse inside o
    (dict(o=A + 8), eb.ATTN_EINVAL),                  # misaligned
])
def test_merge_validation(kw, code):
    assert merge(**kw) == code


def test_merge_zero_rows_is_noop():
    assert merge(rows=0) == eb.ATTN_OK


def _blocks(spec):
    arr = (eb.KVBlock * max(1, len(spec)))()
    for i, (nk, ko) in enumerate(spec):
        arr[i] = eb.KVBlock(A + (2 * i + 8) * B16, A + (2 * i + 9) * B16, nk, ko)
    return arr


def ring(spec, ws=A + 40 * B16, ws_bytes=None, **kw):
    args = dict(q=A, o=A + B16, l=A + 2 * B16, B=1, H=2, Nq=64, d=64, scale=0.125, causal=1, q_off=128, stride=1,
                it=eb.ATTN_BF16, ot=eb.ATTN_BF16)
    args.update(kw)
    if ws_bytes is None:
        ws_bytes = eb.ring_local_workspace_bytes(args["B"], args["H"], args["Nq"], args["d"])
    arr = _blocks(spec)
    return lib.ring_local(args["q"], arr, len(spec), args["o"], args["l"], args["B"], args["H"], args["Nq"], args["d"],
                          args["scale"], args["causal"], args["q_off"], args["stride"], args["it"], args["ot"], ws,
                          ws_bytes, None)


def test_ring_local_validation():
    spec = [(64, 0), (64, 64), (64, 128)]
    assert ring(spec, ws=None) == eb.ATTN_EWORKSPACE
    assert ring(spec, ws_bytes=100) == eb.ATTN_EWORKSPACE
    assert ring(spec, ws=A + 40 * B16 + 16) == eb.ATTN_EINVAL           # misaligned workspace
    assert ring(spec, ws=A + 8 * B16 + 256) == eb.ATTN_EINVAL           # workspace inside block 0's k
    assert ring([(64, 0), (-1, 5)]) == eb.ATTN_EINVAL
    assert ring(spec, stride=0) == eb.ATTN_EINVAL
    assert ring(spec, d=48) == eb.ATTN_EUNSUPPORTED
    assert "workspace" in eb.last_error() or eb.last_error() != ""
    assert ring([], Nq=0) == eb.ATTN_OK


def _brute_kind(nq, nk, causal, q_off, k_off, stride):
    vis = oracle.visible(nq, nk, causal, q_off, k_off, stride)
    if nk == 0 or not vis.any():
        return 0
    return 1 if vis.all() else 2


@pytest.mark.parametrize("causal", [0, 1])
def test_ring_plan_matches_oracle_mask(causal):
    rng = np.random.default_rng(3)
    for _ in range(200):
        nq = int(rng.integers(1, 40))
        stride = int(rng.choice([1, 2, 4]))
        q_off = int(rng.integers(-50, 50))
        spec = [(int(rng.integers(0, 40)), int(rng.integers(-80, 80))) for _ in range(int(rng.integers(1, 5)))]
        live, kinds = eb.ring_local_plan(nq, spec, causal=causal, q_off=q_off, pos_stride=stride)
        want = [_brute_kind(nq, nk, causal, q_off, ko, stride) for nk, ko in spec]
        assert kinds == want
        assert live == sum(k != 0 for k in want)


def test_ring_plan_at_extreme_offsets():
    """Offsets at the accepted limit (|offset| <= 2^62): q_off - k_off reaches 2^63, past int64, and must still
    classify correctly (the host forms it in 128 bits)."""
    big = 1 << 62
    cases = [(big, -big, 1), (-big, big, 0), (big, big - 5, 2), (big - 3, big, 2), (big, big - 100, 1),
             (-big, -big + 100, 0)]
    for q_off, k_off, want in cases:
        for stride in (1, 3, 4):
            live, kinds = eb.ring_local_plan(16, [(16, k_off)], causal=1, q_off=q_off, pos_stride=stride)
            ref = _brute_kind(16, 16, 1, q_off, k_off, stride)
            assert kinds == [ref], (q_off, k_off, stride)
            if stride == 1:
                assert kinds == [want], (q_off, k_off)


def test_binding_rejects_integers_wider_than_the_abi():
    """ctypes reduces an int modulo 2^bits without complaint (2^64 + 5 would reach the library as 5); the binding
    must refuse such values instead of passing a different, valid-looking argument."""
    with pytest.raises(ValueError, match="k_off"):
        eb.ring_local_plan(16, [(16, (1 << 64) + 5)], causal=1)
    with pytest.raises(ValueError, match="q_off"):
        eb.ring_local_plan(16, [(16, 0)], causal=1, q_off=-(1 << 63) - 1)
    with pytest.raises(ValueError, match="pos_stride"):
        eb.ring_local_plan(16, [(16, 0)], causal=1, pos_stride=(1 << 32) + 1)
    with pytest.raises(ValueError, match="Nk"):
        eb.ring_local_plan(16, [((1 << 32) + 16, 0)], causal=1)
    with pytest.raises(ValueError, match="Nq"):
        eb.ring_local_plan(1 << 31, [(16, 0)], causal=1)
    with pytest.raises(ValueError, match="Nk_max"):
        eb.ring_local_pipelined_workspace_bytes(1, 1, 64, 64, 1 << 40)
    # a value that fits reaches the library unchanged, which answers with its own range check (|offset| <= 2^62)
    with pytest.raises(eb.AttnError, match="k_off out of range"):
        eb.ring_local_plan(16, [(16, (1 << 63) - 1)], causal=1)


def test_ring_plan_named_workloads():
    n = 32768
    live, kinds = eb.ring_local_plan(n, [(n, 0), (n, n), (n, 2 * n), (n, 3 * n)], causal=True, q_off=2 * n)
    assert (live, kinds) == (3, [1, 1, 2, 0])
    for r in range(4):
        live, kinds = eb.ring_local_plan(16384, [(16384, s) for s in range(4)], causal=True, q_off=r, pos_stride=4)
        assert (live, kinds) == (4, [2, 2, 2, 2])
    assert eb.ring_local_plan(256, [(64, 64 * i) for i in range(4)], causal=False) == (4, [1, 1, 1, 1])


def fwd_ex(**kw):
    args = dict(q=A, k=A + B16, v=A + 2 * B16, o=A + 3 * B16, lse=A + 4 * B16, B=1, H=8, Hkv=2, Nq=64, Nk=64,
                d=128, scale=0.125, causal=1, q_off=0, k_off=0, stride=1, window=16, it=eb.ATTN_BF16,
                ot=eb.ATTN_BF16, stream=None)
    args.update(kw)
    return lib.attn_fwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"],
                           args["Hkv"], args["Nq"], args["Nk"], args["d"], args["scale"], args["causal"],
                           args["q_off"], args["k_off"], args["stride"], args["window"], args["it"], args["ot"],
                           args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=3), eb.ATTN_EINVAL),                   # 3 does not divide 8
    (dict(Hkv=0), eb.ATTN_EINVAL),
    (dict(Hkv=16), eb.ATTN_EINVAL),
    (dict(window=-1), eb.ATTN_EINVAL),
    (dict(window=4, causal=0), eb.ATTN_EINVAL),       # a window needs the causal mask
    (dict(window=(1 << 62) + 1), eb.ATTN_EINVAL),
    (dict(q=None), eb.ATTN_EINVAL),
    (dict(d=32), eb.ATTN_EUNSUPPORTED),
    (dict(o=A + B16 + 16384), eb.ATTN_EINVAL),        # k holds Hkv = 2 heads (32 KiB): o 16 KiB into it overlaps
])
def test_attn_fwd_ex_validation(kw, code):
    assert fwd_ex(**kw) == code
    assert eb.last_error() != ""


def test_attn_fwd_ex_zero_sized_and_kv_sizing():
    assert fwd_ex(B=0) == eb.ATTN_OK
    assert fwd_ex(Nq=0) == eb.ATTN_OK
    assert fwd_ex(H=0, Hkv=0) == eb.ATTN_OK
    assert fwd_ex(q=None, B=0) == eb.ATTN_OK
    # the outputs are sized by the 8 query heads (o: 8 * 64 * 128 bf16 = 128 KiB): lse 64 KiB into o overlaps
    assert fwd_ex(lse=A + 3 * B16 + 65536) == eb.ATTN_EINVAL


def bwd(**kw):
    args = dict(q=A, k=A + B16, v=A + 2 * B16, o=A + 3 * B16, lse=A + 4 * B16, do=A + 5 * B16, dq=A + 6 * B16,
                dk=A + 7 * B16, dv=A + 8 * B16, delta=A + 9 * B16, B=1, H=8, Hkv=2, Nq=64, Nk=64, d=128,
                scale=0.125, causal=1, q_off=0, k_off=0, stride=1, window=0, it=eb.ATTN_BF16, ot=eb.ATTN_BF16,
                gt=eb.ATTN_F32, acc=0, stream=None)
    args.update(kw)
    return lib.attn_bwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["do"], args["dq"], args["dk"],
                        args["dv"], args["delta"], args["B"], args["H"], args["Hkv"], args["Nq"], args["Nk"],
                        args["d"], args["scale"], args["causal"], args["q_off"], args["k_off"], args["stride"],
                        args["window"], args["it"], args["ot"], args["gt"], args["acc"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), eb.ATTN_EINVAL),
    (dict(do=None), eb.ATTN_EINVAL),
    (dict(delta=None), eb.ATTN_EINVAL),
    (dict(dk=None), eb.ATTN_EINVAL),
    (dict(Hkv=3), eb.ATTN_EINVAL),
    (dict(Nk=-1), eb.ATTN_EINVAL),
    (dict(causal=2), eb.ATTN_EINVAL),
    (dict(acc=2), eb.ATTN_EINVAL),
    (dict(acc=1, gt=eb.ATTN_BF16), eb.ATTN_EINVAL),        # accumulation needs fp32 gradients
    (dict(window=8, causal=0), eb.ATTN_EINVAL),
    (dict(scale=0.0), eb.ATTN_EINVAL),
    (dict(stride=0), eb.ATTN_EINVAL),
    (dict(it=eb.ATTN_F32), eb.ATTN_EINVAL),                 # fp32 inputs need an fp32 o
    (dict(it=7), eb.ATTN_EINVAL),
    (dict(d=32), eb.ATTN_EUNSUPPORTED),
    (dict(dq=A + 1), eb.ATTN_EINVAL),                       # misaligned
    (dict(delta=A + 2), eb.ATTN_EINVAL),
    (dict(dq=A + 3 * B16 + 4096), eb.ATTN_EINVAL),          # dq overlaps o
    (dict(dv=A + 7 * B16 + 4096), eb.ATTN_EINVAL),          # dv overlaps dk (2 heads x 64 x 128 fp32 = 64 KiB)
    (dict(delta=A + 6 * B16 + 8), eb.ATTN_EINVAL),          # delta inside dq
    (dict(dk=A + 4 * B16), eb.ATTN_EINVAL),                 # dk over lse
])
def test_attn_bwd_validation(kw, code):
    assert bwd(**kw) == code
    assert eb.last_error() != ""


def test_attn_bwd_zero_sized_calls_are_noops():
    assert bwd(B=0) == eb.ATTN_OK
    assert bwd(H=0, Hkv=0) == eb.ATTN_OK
    assert bwd(Nq=0, Nk=0) == eb.ATTN_OK
    assert bwd(B=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None, delta=None) == eb.ATTN_OK
    # with Nq = 0 the query-side pointers are not needed, but dk and dv still are
    assert bwd(Nq=0, dk=None) == eb.ATTN_EINVAL


def fwd_merge(**kw):
    args = dict(q=A, k=A + B16, v=A + 2 * B16, ro=A + 3 * B16, rl=A + 4 * B16, o=A + 5 * B16, lse=A + 6 * B16, B=1,
                H=8, Hkv=2, Nq=64, Nk=64, d=128, scale=0.125, causal=1, q_off=0, k_off=0, stride=1, window=0,
                it=eb.ATTN_BF16, ot=eb.ATTN_F32, stream=None)
    args.update(kw)
    return lib.attn_fwd_merge(args["q"], args["k"], args["v"], args["ro"], args["rl"], args["o"], args["lse"],
                              args["B"], args["H"], args["Hkv"], args["Nq"], args["Nk"], args["d"], args["scale"],
                              args["causal"], args["q_off"], args["k_off"], args["stride"], args["window"], args["it"],
                              args["ot"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ro=None), eb.ATTN_EINVAL),
    (dict(rl=None), eb.ATTN_EINVAL),
    (dict(ro=A + 3 * B16 + 4), eb.ATTN_EINVAL),                  # misaligned running o
    (dict(it=eb.ATTN_F32), eb.ATTN_EUNSUPPORTED),                 # bf16 inputs only
    (dict(Hkv=3), eb.ATTN_EINVAL),
    (dict(window=4, causal=0), eb.ATTN_EINVAL),
    (dict(o=A + 3 * B16, ot=eb.ATTN_BF16), eb.ATTN_EINVAL),     # in place needs an fp32 output
    (dict(o=A + 3 * B16 + 1024), eb.ATTN_EINVAL),                # o overlaps run_o without being it
    (dict(lse=A + 4 * B16 + 8), eb.ATTN_EINVAL),                 # lse overlaps run_lse without being it
    (dict(rl=A + 3 * B16 + 4096), eb.ATTN_EINVAL),               # run_lse inside run_o
    (dict(ro=A + B16), eb.ATTN_EINVAL),                          # run_o over k
    (dict(d=32), eb.ATTN_EUNSUPPORTED),
])
def test_attn_fwd_merge_validation(kw, code):
    assert fwd_merge(**kw) == code
    assert eb.last_error() != ""


def test_attn_fwd_merge_zero_sized():
    assert fwd_merge(B=0) == eb.ATTN_OK
    assert fwd_merge(Nq=0, ro=None, rl=None) == eb.ATTN_OK


def test_ring_local_pipelined_workspace_and_validation():
    def a256(x):
        return (x + 255) // 256 * 256
    for B, H, Nq, d, nk in [(1, 32, 32768, 128, 32768), (2, 3, 100, 64, 7), (1, 1, 1, 24, 0)]:
        rows, kv = B * H * Nq, B * H * nk * d * 2
        assert eb.ring_local_pipelined_workspace_bytes(B, H, Nq, d, nk) == a256(rows * d * 4) + a256(rows * 4) + 4 * a256(kv)
    assert eb.ring_local_pipelined_workspace_bytes(1, 1, 1, 1, -1) == 0
    blocks = (eb.KVBlock * 3)(eb.KVBlock(A + B16, A + 2 * B16, 64, 0), eb.KVBlock(A + 3 * B16, A + 4 * B16, 64, 64),
                              eb.KVBlock(A + 5 * B16, A + 6 * B16, 64, 128))
    P = dict(q=A, o=A + 7 * B16, lse=A + 8 * B16)

    def call(blocks_, n, ws, ws_bytes, **kw):
        a = dict(P, B=1, H=2, Nq=64, d=128, scale=0.1, causal=0, q_off=0, stride=1, ot=eb.ATTN_BF16)
        a.update(kw)
        return lib.ring_local_pipelined(a["q"], blocks_, n, a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["d"],
                                        a["scale"], a["causal"], a["q_off"], a["stride"], a["ot"], ws, ws_bytes,
                                        None, None)
    assert call(blocks, 3, None, 0) == eb.ATTN_EWORKSPACE                     # two incoming blocks need the slots
    assert call(blocks, 3, A + 9 * B16, 1024) == eb.ATTN_EWORKSPACE
    assert call(blocks, 3, A + 9 * B16 + 8, 1 << 24) == eb.ATTN_EINVAL          # misaligned workspace
    assert call(blocks, 3, A + 7 * B16, 1 << 24) == eb.ATTN_EINVAL              # workspace over o
    assert call(blocks, -1, None, 0) == eb.ATTN_EINVAL
    assert call(None, 2, None, 0) == eb.ATTN_EINVAL
    assert call(blocks, 3, None, 0, d=32) == eb.ATTN_EUNSUPPORTED
    assert call(blocks, 3, None, 0, B=0) == eb.ATTN_OK


def test_import_without_the_library_fails_loudly(tmp_path):
    """The package has no fallback: a copy of its Python files without the built library refuses to import."""
    import os
    import shutil
    import sys
    pkg = os.path.dirname(eb.__file__)
    dst = tmp_path / "exact_blockwise_attention_amd"
    dst.mkdir()
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            shutil.copy(os.path.join(pkg, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import exact_blockwise_attention_amd"], cwd=tmp_path,
                       capture_output=True, text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is missing" in r.stderr and "no fallback" in r.stderr
