"""Python binding of libfa.so: argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libfa.so``; this
module only checks tensor properties, allocates outputs with torch (device
memory and streams are torch's), and passes raw pointers plus the current HIP
stream through the C ABI declared in ``include/fa.h``.  There is no fallback:
if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None
_lock = threading.Lock()

# exported symbols and their C signatures (include/fa.h)
_c_int, _c_float, _c_size_t, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "fa_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp]),
    "fa_fwd_f32": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp]),
    "fa_fwd_fp16": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp]),
    "fa_bwd_fp16": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float,
                             _c_int, _vp, _c_size_t, _vp]),
    "fa_bwd_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "fa_bwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float,
                        _c_int, _vp, _c_size_t, _vp]),
    "fa_bwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float,
                                _c_int, _vp]),
    "fa_probe_mfma_bf16": (_c_int, [_c_int, _c_int, _vp, _vp]),
    "fa_fwd_splitkv_parts": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "fa_fwd_splitkv_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "fa_fwd_splitkv": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int,
                                _vp, _c_size_t, _vp]),
    "fa_lse_merge": (_c_int, [_vp, _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "fa_fwd_window": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int,
                               _vp]),
    "fa_fwd_blocksparse": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _vp,
                                    _c_int, _vp]),
    "fa_fwd_dropout": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_float,
                                ctypes.c_ulonglong, _vp]),
    "fa_bwd_dropout": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float,
                                _c_int, _c_float, ctypes.c_ulonglong, _vp, _c_size_t, _vp]),
    "fa_bwd_window": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_float,
                               _c_int, _c_int, _vp, _c_size_t, _vp]),
    "fa_bwd_blocksparse": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _vp, _c_int, _vp, _c_size_t, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
}
# the float16 versions of the key split, the merge, the masks and dropout take
# the same arguments as the bf16 ones
for _name in ("fa_fwd_splitkv", "fa_lse_merge", "fa_fwd_window", "fa_bwd_window", "fa_fwd_blocksparse",
              "fa_bwd_blocksparse", "fa_fwd_dropout", "fa_bwd_dropout"):
    SIGNATURES[_name + "_fp16"] = SIGNATURES[_name]


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: str | None = None):
    """Load libfa.so (once) and bind its symbols; raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or _LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built: run `python -m aware_exact_attention_amd.build` first")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B,H,N,d]")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: float | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Forward attention of ``[B,H,N,d]`` tensors; returns ``(o, lse)``.

    bf16 inputs run ``fa_fwd``, float16 ``fa_fwd_fp16``, float32 ``fa_fwd_f32``.  ``scale``
    defaults to ``1/sqrt(d)``.  ``out``/``lse`` may be passed preallocated.
    """
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise TypeError(f"unsupported dtype {dtype}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dtype, (B, H, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dtype, (B, H, N, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    name = {torch.bfloat16: "fa_fwd", torch.float16: "fa_fwd_fp16", torch.float32: "fa_fwd_f32"}[dtype]
    st = getattr(lib, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                            float(scale), int(bool(causal)), _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, workspace=None, out=None):
    """Backward attention (bf16 or float16, ``fa_bwd`` / ``fa_bwd_fp16``); returns ``(dq, dk, dv)``.

    ``o`` and ``lse`` must be what ``fwd`` returned for the same inputs, scale
    and causal flag.  ``workspace`` (a uint8 GPU tensor of at least
    ``bwd_workspace_bytes`` bytes) is allocated if not given; ``out`` may hold
    preallocated ``(dq, dk, dv)``.
    """
    lib = load()
    B, H, N, d = q.shape
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"unsupported dtype {dtype}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dtype, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _check(t, n, dtype, (B, H, N, d))
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    name = "fa_bwd" if dtype == torch.bfloat16 else "fa_bwd_fp16"
    st = getattr(lib, name)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                            workspace.data_ptr(), workspace.numel(), _stream())
    if st != 0:
        raise FAError(st, name)
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, out, causal: bool = False, scale: float | None = None):
    """bf16 backward through ``fa_bwd_noalloc``: the library's own per-GPU
    scratch replaces the workspace, and ``out = (dq, dk, dv)`` must be
    preallocated, so the call allocates nothing.  Calls that overlap on one
    GPU share that scratch and must be ordered by the caller."""
    lib = load()
    B, H, N, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, torch.bfloat16, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = out
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, torch.bfloat16, (B, H, N, d))
    st = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale),
                            int(bool(causal)), _stream())
    if st != 0:
        raise FAError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def probe_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor) -> None:
    """Enqueue the MFMA-rate probe (``fa_probe_mfma_bf16``); FLOP = workgroups*4*iters*4*32768."""
    _check(sink, "sink", torch.float32)
    if sink.numel() < workgroups * 256:
        raise ValueError("sink needs workgroups*256 floats")
    st = load().fa_probe_mfma_bf16(int(workgroups), int(iters), sink.data_ptr(), _stream())
    if st != 0:
        raise FAError(st, "fa_probe_mfma_bf16")


def splitkv_parts(B: int, H: int, N: int, d: int, num_splits: int = 0) -> int:
    return int(load().fa_fwd_splitkv_parts(B, H, N, d, int(num_splits)))


def splitkv_workspace_bytes(B: int, H: int, N: int, d: int, num_splits: int = 0) -> int:
    return int(load().fa_fwd_splitkv_workspace_bytes(B, H, N, d, int(num_splits)))


def _half(q):
    """The 16-bit element type of q (bf16 or float16); the entry points for float16 carry the suffix _fp16."""
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"unsupported dtype {q.dtype}: bf16 or float16")
    return q.dtype


def _sym(lib, name, dt):
    full = name if dt == torch.bfloat16 else name + "_fp16"
    return full, getattr(lib, full)


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0,
                workspace=None, out=None, lse=None):
    """bf16 or float16 forward with the keys split into parallel parts merged by Eq. (2); returns ``(o, lse)``.

    ``num_splits <= 0`` lets the library choose.  ``workspace`` (uint8 GPU
    tensor of at least ``splitkv_workspace_bytes`` bytes) is allocated if not
    given.
    """
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt, (B, H, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dt, (B, H, N, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    need = splitkv_workspace_bytes(B, H, N, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
    name, fn = _sym(lib, "fa_fwd_splitkv", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
            float(scale), int(bool(causal)), int(num_splits),
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def lse_merge(o_parts, lse_parts, out=None, lse=None, dtype=torch.bfloat16):
    """Eq. (2) merge of ``o_parts`` float32 ``[S,B,H,N,d]`` and ``lse_parts`` float32 ``[S,B,H,N]``.

    Returns ``(o, lse)``: ``dtype`` (bf16 or float16; that of ``out`` when given)
    ``[B,H,N,d]`` and float32 ``[B,H,N]``.
    """
    lib = load()
    dt = out.dtype if out is not None else dtype
    if dt not in (torch.bfloat16, torch.float16):
        raise TypeError(f"unsupported output dtype {dt}")
    if o_parts.dim() != 5:
        raise ValueError("o_parts must be [S,B,H,N,d]")
    S, B, H, N, d = o_parts.shape
    _check(o_parts, "o_parts", torch.float32, (S, B, H, N, d))
    _check(lse_parts, "lse_parts", torch.float32, (S, B, H, N))
    if out is None:
        out = torch.empty((B, H, N, d), dtype=dt, device=o_parts.device)
    else:
        _check(out, "out", dt, (B, H, N, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    name, fn = _sym(lib, "fa_lse_merge", dt)
    st = fn(o_parts.data_ptr(), lse_parts.data_ptr(), S, out.data_ptr(), lse.data_ptr(), B, H, N, d, _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def _fwd_outputs(q, out, lse):
    B, H, N, d = q.shape
    dt = q.dtype
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dt, (B, H, N, d))
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, H, N))
    return out, lse


def fwd_window(q, k, v, window_left: int, window_right: int, scale: float | None = None, out=None, lse=None):
    """bf16 or float16 sliding-window forward: key j visible to query i iff i-left <= j <= i+right
    (negative = unlimited); returns ``(o, lse)``."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt, (B, H, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _fwd_outputs(q, out, lse)
    name, fn = _sym(lib, "fa_fwd_window", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
            float(scale), int(window_left), int(window_right), _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """bf16 or float16 block-sparse forward over 64 x 64 blocks; ``block_mask`` is a uint8 GPU tensor
    ``[H, nb, nb]`` or ``[nb, nb]`` (shared by all heads), nb = ceil(N/64); returns ``(o, lse)``."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt, (B, H, N, d))
    nb = (N + 63) // 64
    if block_mask.dim() == 3:
        _check(block_mask, "block_mask", torch.uint8, (H, nb, nb))
        per_head = 1
    else:
        _check(block_mask, "block_mask", torch.uint8, (nb, nb))
        per_head = 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _fwd_outputs(q, out, lse)
    name, fn = _sym(lib, "fa_fwd_blocksparse", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N,
            d, float(scale), int(bool(causal)), block_mask.data_ptr(), per_head, _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def _bwd_args(q, k, v, o, lse, do, scale, workspace, out):
    """Shared checks and allocations of the masked backward calls (bf16 or float16)."""
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dt, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", torch.uint8)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _check(t, n, dt, (B, H, N, d))
    return (B, H, N, d), float(scale), workspace, (dq, dk, dv)


def bwd_window(q, k, v, o, lse, do, window_left: int, window_right: int, scale: float | None = None,
               workspace=None, out=None):
    """bf16 or float16 backward of ``fwd_window`` (``fa_bwd_window``); returns ``(dq, dk, dv)``."""
    lib = load()
    dt = _half(q)
    (B, H, N, d), scale, workspace, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, scale, workspace, out)
    name, fn = _sym(lib, "fa_bwd_window", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale, int(window_left),
            int(window_right), workspace.data_ptr(), workspace.numel(), _stream())
    if st != 0:
        raise FAError(st, name)
    return dq, dk, dv


def bwd_blocksparse(q, k, v, o, lse, do, block_mask, causal: bool = False, scale: float | None = None,
                    workspace=None, out=None):
    """bf16 or float16 backward of ``fwd_blocksparse`` (``fa_bwd_blocksparse``); returns ``(dq, dk, dv)``."""
    lib = load()
    dt = _half(q)
    (B, H, N, d), scale, workspace, (dq, dk, dv) = _bwd_args(q, k, v, o, lse, do, scale, workspace, out)
    nb = (N + 63) // 64
    if block_mask.dim() == 3:
        _check(block_mask, "block_mask", torch.uint8, (H, nb, nb))
        per_head = 1
    else:
        _check(block_mask, "block_mask", torch.uint8, (nb, nb))
        per_head = 0
    name, fn = _sym(lib, "fa_bwd_blocksparse", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, scale,
            int(bool(causal)), block_mask.data_ptr(), per_head, workspace.data_ptr(),
            workspace.numel(), _stream())
    if st != 0:
        raise FAError(st, name)
    return dq, dk, dv


def fwd_dropout(q, k, v, dropout_p: float, seed: int, causal: bool = False, scale: float | None = None,
                out=None, lse=None):
    """bf16 or float16 forward with dropout on P (Philox4x32-10 mask from ``seed``); returns ``(o, lse)``."""
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d]")
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, dt, (B, H, N, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _fwd_outputs(q, out, lse)
    name, fn = _sym(lib, "fa_fwd_dropout", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
            float(scale), int(bool(causal)), float(dropout_p), int(seed) & (2**64 - 1), _stream())
    if st != 0:
        raise FAError(st, name)
    return out, lse


def bwd_dropout(q, k, v, o, lse, do, dropout_p: float, seed: int, causal: bool = False,
                scale: float | None = None, workspace=None, out=None):
    """bf16 or float16 backward through the same dropout mask as ``fwd_dropout``; returns ``(dq, dk, dv)``."""
    lib = load()
    B, H, N, d = q.shape
    dt = _half(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, dt, (B, H, N, d))
    _check(lse, "lse", torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", torch.uint8)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _check(t, n, dt, (B, H, N, d))
    name, fn = _sym(lib, "fa_bwd_dropout", dt)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
            float(dropout_p), int(seed) & (2**64 - 1), workspace.data_ptr(), workspace.numel(),
            _stream())
    if st != 0:
        raise FAError(st, name)
    return dq, dk, dv
