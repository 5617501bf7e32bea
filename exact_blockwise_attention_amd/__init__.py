"""Python binding of libebattn (exact blockwise attention and the log-sum-exp merge on MI355X).

Argument marshalling only: every step of the computation runs in the library's HIP kernels. PyTorch provides
device memory (outputs are allocated with ``torch.empty`` when not given) and the stream (the current torch
stream of the tensors' device). Importing this package fails loudly if the shared library is not built; there
is no fallback implementation.

Names and semantics follow the C ABI in include/ebattn.h:

    o, lse = attn_fwd(q, k, v, scale=..., causal=..., q_off=..., k_off=..., pos_stride=...)
    o, lse = attn_lse_merge(o_a, lse_a, o_b, lse_b)
    o, lse = attn_fwd_merge(q, k, v, run_o, run_lse, ...)     # one block's attention merged in its epilogue
    dq, dk, dv, delta = attn_bwd(q, k, v, o, lse, dout, scale=..., causal=..., window=...)
    o, lse = ring_local(q_shard, [(k0, v0, k_off0), (k1, v1, k_off1), ...], scale=..., causal=..., q_off=...)
    o, lse = ring_local_pipelined(q_shard, blocks, ..., copy_stream=s)   # incoming blocks copied while computing
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libebattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ebattn.h")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EHIP = -3
ATTN_EWORKSPACE = -4
ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_MAX_SEQ = 1 << 28


class AttnError(RuntimeError):
    """A non-zero status returned by the library, with its attn_last_error() message."""

    def __init__(self, code: int, message: str):
        super().__init__(f"ebattn error {code}: {message}")
        self.code = code
        self.message = message


class KVBlock(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("Nk", ctypes.c_int), ("k_off", ctypes.c_int64)]


def _load() -> ctypes.CDLL:
    # PyTorch-ROCm ships its own HIP runtime whose soname (libamdhip64.so.7) matches this library's dependency.
    # Loading torch first lets the dynamic linker satisfy that dependency with torch's runtime, so the process
    # has one HIP runtime and torch's device memory and streams are valid here. Loading this library first
    # would bring in a second runtime next to torch's.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python exact_blockwise_attention_amd/build.py` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I64, I64, I, I, I, P]
    lib.attn_fwd.restype = I
    lib.attn_fwd_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, I64, I64, I, I64, I, I, P]
    lib.attn_fwd_ex.restype = I
    lib.attn_fwd_merge.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I64, I64, I, I64, I, I, P]
    lib.attn_fwd_merge.restype = I
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I64, I64, I, I64, I, I, I, I, P]
    lib.attn_bwd.restype = I
    lib.attn_lse_merge.argtypes = [P, P, P, P, P, P, I64, I, I, I, P]
    lib.attn_lse_merge.restype = I
    lib.ring_local.argtypes = [P, ctypes.POINTER(KVBlock), I, P, P, I, I, I, I, F, I, I64, I, I, I, P, SZ, P]
    lib.ring_local.restype = I
    lib.ring_local_noalloc.argtypes = [P, ctypes.POINTER(KVBlock), I, P, P, I, I, I, I, F, I, I64, I, I, I, P]
    lib.ring_local_noalloc.restype = I
    lib.ring_local_workspace_bytes.argtypes = [I, I, I, I]
    lib.ring_local_workspace_bytes.restype = SZ
    lib.ring_local_pipelined.argtypes = [P, ctypes.POINTER(KVBlock), I, P, P, I, I, I, I, F, I, I64, I, I, P, SZ, P, P]
    lib.ring_local_pipelined.restype = I
    lib.ring_local_pipelined_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.ring_local_pipelined_workspace_bytes.restype = SZ
    lib.ring_local_plan.argtypes = [ctypes.POINTER(KVBlock), I, I, I, I64, I, ctypes.POINTER(I)]
    lib.ring_local_plan.restype = I
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = I
    return lib


lib = _load()


def declared_symbols() -> List[str]:
    """Names of the functions declared in include/ebattn.h."""
    with open(HEADER_PATH, encoding="utf-8") as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)


def last_error() -> str:
    return (lib.attn_last_error() or b"").decode("utf-8", "replace")


def _check(rc: int):
    if rc != ATTN_OK:
        raise AttnError(rc, last_error())


def _torch():
    import torch
    return torch


def _code(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return ATTN_BF16
    if dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def _arg(name: str, value, bits: int = 32) -> int:
    """value as a C integer argument of the given width (ctypes would wrap an out-of-range int silently)."""
    v = int(value)
    lim = 1 << (bits - 1)
    if not -lim <= v < lim:
        raise ValueError(f"{name} = {v} does not fit the {bits}-bit argument of the C ABI")
    return v


def _dims(**sizes) -> None:
    for name, v in sizes.items():
        _arg(name, v)


def _need_cuda(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = {t.device for t in ts if t is not None}
    if len(dev) > 1:
        raise ValueError("tensors are on different devices")


def version() -> int:
    return lib.attn_version()


def attn_fwd(q, k, v, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0, k_off: int = 0,
             pos_stride: int = 1, out=None, lse=None, out_dtype=None) -> Tuple[object, object]:
    """Exact attention of q [B,H,Nq,d] against k, v [B,H,Nk,d]; returns (o [B,H,Nq,d], lse [B,H,Nq] fp32).

    scale defaults to 1/sqrt(d). Causal masking is by global position (q_off + i*pos_stride vs
    k_off + j*pos_stride, inclusive). out_dtype defaults to q.dtype.
    """
    torch = _torch()
    _need_cuda(q, k, v, out, lse)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H, d")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("out must be [B,H,Nq,d] and lse fp32 [B,H,Nq]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Nq=Nq, Nk=Nk, d=d)
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, scale, int(causal),
                        _arg("q_off", q_off, 64), _arg("k_off", k_off, 64), _arg("pos_stride", pos_stride),
                        _code(q.dtype), _code(out.dtype), _stream(q)))
    return out, lse


def attn_fwd_ex(q, k, v, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0, k_off: int = 0,
                pos_stride: int = 1, window: int = 0, out=None, lse=None, out_dtype=None) -> Tuple[object, object]:
    """attn_fwd with grouped-query heads and a sliding window: q [B,H,Nq,d], k, v [B,Hkv,Nk,d] with Hkv dividing H
    (query head h reads key/value head h // (H // Hkv)); window > 0 keeps, for each query, the keys of the
    window most recent positions up to its own (causal only). Returns (o [B,H,Nq,d], lse [B,H,Nq] fp32)."""
    torch = _torch()
    _need_cuda(q, k, v, out, lse)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    out_dtype = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("out must be [B,H,Nq,d] and lse fp32 [B,H,Nq]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d)
    _check(lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, Nq, Nk, d, scale,
                           int(causal), _arg("q_off", q_off, 64), _arg("k_off", k_off, 64),
                           _arg("pos_stride", pos_stride), _arg("window", window, 64), _code(q.dtype),
                           _code(out.dtype), _stream(q)))
    return out, lse


def attn_fwd_merge(q, k, v, run_o, run_lse, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0,
                   k_off: int = 0, pos_stride: int = 1, window: int = 0, out=None, lse=None,
                   out_dtype=None) -> Tuple[object, object]:
    """attn_fwd_ex of one key/value block merged with the running fp32 result (run_o [B,H,Nq,d], run_lse
    [B,H,Nq]) inside the attention kernel. out / lse may be run_o / run_lse themselves (in place; out fp32).
    out_dtype defaults to float32. Returns (o, lse)."""
    torch = _torch()
    _need_cuda(q, k, v, run_o, run_lse, out, lse)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if tuple(run_o.shape) != (B, H, Nq, d) or tuple(run_lse.shape) != (B, H, Nq):
        raise ValueError("run_o must be [B,H,Nq,d] and run_lse [B,H,Nq]")
    if run_o.dtype != torch.float32 or run_lse.dtype != torch.float32:
        raise TypeError("run_o and run_lse must be float32")
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float32)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("out must be [B,H,Nq,d] and lse fp32 [B,H,Nq]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d)
    _check(lib.attn_fwd_merge(_ptr(q), _ptr(k), _ptr(v), _ptr(run_o), _ptr(run_lse), _ptr(out), _ptr(lse), B, H, Hkv,
                              Nq, Nk, d, scale, int(causal), _arg("q_off", q_off, 64), _arg("k_off", k_off, 64),
                              _arg("pos_stride", pos_stride), _arg("window", window, 64),
                              _code(q.dtype), _code(out.dtype), _stream(q)))
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0,
             k_off: int = 0, pos_stride: int = 1, window: int = 0, grad_dtype=None, accumulate: bool = False,
             dq=None, dk=None, dv=None, delta=None) -> Tuple[object, object, object, object]:
    """Gradients of attn_fwd_ex: q, dout [B,H,Nq,d] bf16, k, v [B,Hkv,Nk,d] bf16, o [B,H,Nq,d] (bf16 or fp32) and
    lse [B,H,Nq] from the forward over the full key set. Returns (dq, dk, dv, delta) with dq [B,H,Nq,d],
    dk, dv [B,Hkv,Nk,d] in grad_dtype (default fp32, or the dtype of the given dq) and delta = rowsum(dout * o)
    [B,H,Nq] fp32. accumulate=True adds into the given fp32 dq, dk, dv."""
    torch = _torch()
    _need_cuda(q, k, v, o, lse, dout, dq, dk, dv, delta)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    if tuple(o.shape) != (B, H, Nq, d) or tuple(dout.shape) != (B, H, Nq, d) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o and dout must be [B,H,Nq,d] and lse [B,H,Nq]")
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("q, k, v and dout must share a dtype")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if grad_dtype is None:
        grad_dtype = dq.dtype if dq is not None else torch.float32
    if accumulate and any(t is None for t in (dq, dk, dv)):
        raise ValueError("accumulate=True needs dq, dk and dv")
    if dq is None:
        dq = torch.empty((B, H, Nq, d), dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty((B, Hkv, Nk, d), dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty((B, Hkv, Nk, d), dtype=grad_dtype, device=q.device)
    if delta is None:
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if (tuple(dq.shape) != (B, H, Nq, d) or tuple(dk.shape) != (B, Hkv, Nk, d) or tuple(dv.shape) != (B, Hkv, Nk, d)
            or tuple(delta.shape) != (B, H, Nq)):
        raise ValueError("dq must be [B,H,Nq,d], dk and dv [B,Hkv,Nk,d], delta [B,H,Nq]")
    if dq.dtype != grad_dtype or dk.dtype != grad_dtype or dv.dtype != grad_dtype or delta.dtype != torch.float32:
        raise TypeError("dq, dk, dv must share grad_dtype and delta must be float32")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d)
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(delta), B, H, Hkv, Nq, Nk, d, scale, int(causal), _arg("q_off", q_off, 64),
                        _arg("k_off", k_off, 64), _arg("pos_stride", pos_stride), _arg("window", window, 64),
                        _code(q.dtype), _code(o.dtype), _code(grad_dtype), int(accumulate), _stream(q)))
    return dq, dk, dv, delta


def attn_lse_merge(o_a, lse_a, o_b, lse_b, *, out=None, lse_out=None, out_dtype=None) -> Tuple[object, object]:
    """Merges two partials over disjoint key sets; o_* are [..., d], lse_* the matching [...] fp32.

    out may be o_a or o_b (same dtype) and lse_out may be lse_a or lse_b for an in-place merge.
    """
    torch = _torch()
    _need_cuda(o_a, lse_a, o_b, lse_b, out, lse_out)
    if o_a.shape != o_b.shape or o_a.dtype != o_b.dtype:
        raise ValueError("o_a and o_b must match in shape and dtype")
    if lse_a.shape != o_a.shape[:-1] or lse_b.shape != o_a.shape[:-1]:
        raise ValueError("lse_a/lse_b must have o's shape without the last axis")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise TypeError("lse tensors must be fp32")
    d = o_a.shape[-1]
    rows = o_a.numel() // d if d else 0
    out_dtype = out_dtype or (out.dtype if out is not None else o_a.dtype)
    if out is None:
        out = torch.empty(o_a.shape, dtype=out_dtype, device=o_a.device)
    if lse_out is None:
        lse_out = torch.empty(lse_a.shape, dtype=torch.float32, device=o_a.device)
    if out.shape != o_a.shape or lse_out.shape != lse_a.shape:
        raise ValueError("out / lse_out shapes do not match the partials")
    _dims(d=d)
    _check(lib.attn_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out), _ptr(lse_out), rows, d,
                              _code(o_a.dtype), _code(out.dtype), _stream(o_a)))
    return out, lse_out


def ring_local_workspace_bytes(B: int, H: int, Nq: int, d: int) -> int:
    _dims(B=B, H=H, Nq=Nq, d=d)
    return int(lib.ring_local_workspace_bytes(B, H, Nq, d))


def _blocks(kv_blocks) -> Tuple[ctypes.Array, int]:
    arr = (KVBlock * max(1, len(kv_blocks)))()
    for i, (k, v, k_off) in enumerate(kv_blocks):
        if hasattr(k, "data_ptr"):
            arr[i] = KVBlock(_ptr(k), _ptr(v), _arg("Nk", k.shape[2]), _arg("k_off", k_off, 64))
        else:  # (k_ptr, v_ptr, Nk, k_off) raw form is not accepted here; use explicit ints via KVBlock
            raise TypeError("kv_blocks entries are (k, v, k_off) with k, v tensors")
    return arr, len(kv_blocks)


def ring_local_plan(Nq: int, blocks: Sequence[Tuple[int, int]], *, causal: bool, q_off: int = 0,
                    pos_stride: int = 1) -> Tuple[int, List[int]]:
    """Host-only: classifies blocks given as (Nk, k_off). Returns (live count, kinds) with kinds 0 = skipped,
    1 = fully visible, 2 = partly visible."""
    arr = (KVBlock * max(1, len(blocks)))()
    for i, (nk, ko) in enumerate(blocks):
        arr[i] = KVBlock(None, None, _arg("Nk", nk), _arg("k_off", ko, 64))
    kinds = (ctypes.c_int * max(1, len(blocks)))()
    live = lib.ring_local_plan(arr, len(blocks), _arg("Nq", Nq), int(causal), _arg("q_off", q_off, 64),
                               _arg("pos_stride", pos_stride), kinds)
    if live < 0:
        raise AttnError(live, last_error())
    return live, [kinds[i] for i in range(len(blocks))]


def ring_local(q_shard, kv_blocks, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0,
               pos_stride: int = 1, out=None, lse=None, out_dtype=None, workspace=None) -> Tuple[object, object]:
    """One device's share of Ring Attention: q_shard [B,H,Nq,d] against kv_blocks = [(k, v, k_off), ...]
    processed in the given (ring) order and merged; returns (o, lse) of attention over all blocks.

    workspace: optional uint8 device tensor of at least ring_local_workspace_bytes(B, H, Nq, d) bytes;
    allocated here when needed and not given.
    """
    torch = _torch()
    _need_cuda(q_shard, out, lse, workspace)
    for k, v, _ in kv_blocks:
        _need_cuda(q_shard, k, v)
        if k.dtype != q_shard.dtype or v.dtype != q_shard.dtype:
            raise TypeError("blocks must share the query dtype")
        if k.shape[:2] != q_shard.shape[:2] or k.shape != v.shape or k.shape[3] != q_shard.shape[3]:
            raise ValueError("each block is k, v [B, H, Nk, d] with the query's B, H, d")
    B, H, Nq, d = q_shard.shape
    out_dtype = out_dtype or (out.dtype if out is not None else q_shard.dtype)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q_shard.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q_shard.device)
    live, _ = ring_local_plan(Nq, [(k.shape[2], ko) for k, _, ko in kv_blocks], causal=causal, q_off=q_off,
                              pos_stride=pos_stride)
    need = ring_local_workspace_bytes(B, H, Nq, d)
    if workspace is None and live > 1:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_shard.device)
    arr, n = _blocks(kv_blocks)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Nq=Nq, d=d)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.ring_local(_ptr(q_shard), arr, n, _ptr(out), _ptr(lse), B, H, Nq, d, scale, int(causal),
                          _arg("q_off", q_off, 64), _arg("pos_stride", pos_stride), _code(q_shard.dtype),
                          _code(out.dtype), ws_ptr, ws_bytes, _stream(q_shard)))
    return out, lse


# Host (pinned) blocks handed to ring_local_pipelined are read by the copy engines after the call returns. Each
# call's host tensors stay referenced here, with an event recorded on the compute stream after the call, until that
# event has completed: torch's pinned-memory cache cannot hand their pages to a new tensor while a copy still reads
# them.
_inflight_host_blocks: List[Tuple[object, List[object]]] = []


def _retire_host_blocks() -> None:
    _inflight_host_blocks[:] = [(ev, ts) for ev, ts in _inflight_host_blocks if not ev.query()]


# ATTN_NOALLOC_SCRATCH_BYTES of include/ebattn.h: the per-GPU scratch array behind ring_local_noalloc
NOALLOC_SCRATCH_BYTES = 256 << 20


def ring_local_noalloc(q_shard, kv_blocks, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0,
                       pos_stride: int = 1, out=None, lse=None) -> Tuple[object, object]:
    """ring_local without a caller workspace: the library's per-GPU scratch array holds the accumulator, and the
    call allocates no device memory when `out` and `lse` are given (a share needs at most NOALLOC_SCRATCH_BYTES of
    scratch). Calls whose work overlaps on one GPU race on that array; calls on one stream are ordered."""
    torch = _torch()
    _need_cuda(q_shard, out, lse)
    for k, v, _ in kv_blocks:
        _need_cuda(q_shard, k, v)
        if k.dtype != q_shard.dtype or v.dtype != q_shard.dtype:
            raise TypeError("blocks must share the query dtype")
        if k.shape[:2] != q_shard.shape[:2] or k.shape != v.shape or k.shape[3] != q_shard.shape[3]:
            raise ValueError("each block is k, v [B, H, Nk, d] with the query's B, H, d")
    B, H, Nq, d = q_shard.shape
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=q_shard.dtype, device=q_shard.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q_shard.device)
    arr, n = _blocks(kv_blocks)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Nq=Nq, d=d)
    with torch.cuda.device(q_shard.device):   # the scratch array is looked up on the current device
        _check(lib.ring_local_noalloc(_ptr(q_shard), arr, n, _ptr(out), _ptr(lse), B, H, Nq, d, scale, int(causal),
                                      _arg("q_off", q_off, 64), _arg("pos_stride", pos_stride), _code(q_shard.dtype),
                                      _code(out.dtype), _stream(q_shard)))
    return out, lse


def ring_local_pipelined_workspace_bytes(B: int, H: int, Nq: int, d: int, Nk_max: int) -> int:
    _dims(B=B, H=H, Nq=Nq, d=d, Nk_max=Nk_max)
    return int(lib.ring_local_pipelined_workspace_bytes(B, H, Nq, d, Nk_max))


def ring_local_pipelined(q_shard, kv_blocks, *, scale: Optional[float] = None, causal: bool = False, q_off: int = 0,
                         pos_stride: int = 1, out=None, lse=None, out_dtype=None, workspace=None,
                         copy_stream=None) -> Tuple[object, object]:
    """ring_local with the ring's exchange step on this device: kv_blocks[0] = (k, v, k_off) is resident (a GPU
    tensor); every later block is copied into a receive slot on `copy_stream` while the current torch stream
    attends the block before it. Incoming k, v may be pinned CPU tensors (the stand-in for the link) or GPU
    tensors. bf16 only. copy_stream: a torch.cuda.Stream of default priority (one is created when None)."""
    torch = _torch()
    _need_cuda(q_shard, out, lse, workspace)
    if q_shard.dim() != 4:
        raise ValueError("q_shard must be [B, H, Nq, d]")
    B, H, Nq, d = q_shard.shape
    if q_shard.dtype != torch.bfloat16:
        raise TypeError("ring_local_pipelined takes bf16 tensors")
    for i, (k, v, _) in enumerate(kv_blocks):
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
            raise TypeError("blocks must be bf16")
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("blocks must be contiguous")
        if i == 0 and not (k.is_cuda and v.is_cuda):
            raise ValueError("block 0 is read in place and must be on the GPU")
        if not k.is_cuda and not (k.is_pinned() and v.is_pinned()):
            raise ValueError("a CPU block must be in pinned memory")
        if tuple(k.shape) != (B, H, k.shape[2], d) or tuple(v.shape) != tuple(k.shape):
            raise ValueError("each block must be [B, H, Nk, d] matching q_shard")
    out_dtype = out_dtype or (out.dtype if out is not None else q_shard.dtype)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q_shard.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q_shard.device)
    nk_max = max([k.shape[2] for k, _, _ in kv_blocks[1:]] or [0])
    need = ring_local_pipelined_workspace_bytes(B, H, Nq, d, nk_max)
    if workspace is None and len(kv_blocks) > 1:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_shard.device)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=q_shard.device)
    arr, n = _blocks(kv_blocks)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _dims(B=B, H=H, Nq=Nq, d=d)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _retire_host_blocks()
    with torch.cuda.device(q_shard.device):   # the call creates its events on the current device
        _check(lib.ring_local_pipelined(_ptr(q_shard), arr, n, _ptr(out), _ptr(lse), B, H, Nq, d, scale,
                                        int(causal), _arg("q_off", q_off, 64), _arg("pos_stride", pos_stride),
                                        _code(out.dtype), _ptr(workspace), ws_bytes, _stream(q_shard),
                                        copy_stream.cuda_stream))
        host = [t for k, v, _ in kv_blocks for t in (k, v) if not t.is_cuda]
        if host:
            ev = torch.cuda.Event()
            ev.record(torch.cuda.current_stream(q_shard.device))
            _inflight_host_blocks.append((ev, host))
    return out, lse
