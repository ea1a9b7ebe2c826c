"""Thin Python binding of ``libgated_rmsnorm.so`` (C ABI in include/gated_rmsnorm.h).

Argument marshalling only: each function checks torch-level facts the C ABI
cannot see (device, dtype, contiguity, shapes), passes raw device pointers
and torch's current HIP stream, and turns a non-zero status into
``GatedRMSNormError``.  Every step of the computation runs in the HIP
kernels; there is no fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import pathlib
import threading

import torch

_PKG = pathlib.Path(__file__).resolve().parent
_LIB_NAME = "libgated_rmsnorm.so"
_lock = threading.Lock()
_lib = None

GRN_DTYPE_BF16 = 0
GRN_DTYPE_F16 = 1
GRN_DTYPE_F32 = 2
_DTYPE_CODES = {torch.bfloat16: GRN_DTYPE_BF16, torch.float16: GRN_DTYPE_F16,
                torch.float32: GRN_DTYPE_F32}
SUPPORTED_D = (64, 128, 256)
D_DEFAULT = 128


class GatedRMSNormError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> pathlib.Path:
    return _PKG / _LIB_NAME


# Every symbol the header declares, with its ctypes signature.
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIGS = {
    "gated_rmsnorm_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32]),
    "gated_rmsnorm_chunk_rows": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32,
                                                   ctypes.c_int32]),
    "gated_rmsnorm_fwd": (ctypes.c_int32, [_VP, _VP, _VP, _VP, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_int32, _VP]),
    "gated_rmsnorm_bwd": (ctypes.c_int32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            ctypes.c_size_t, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_int32, ctypes.c_int32, _VP]),
    "gated_rmsnorm_ckpt_step": (ctypes.c_int32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                  _VP, _VP, ctypes.c_size_t,
                                                  ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_float, ctypes.c_int32,
                                                  ctypes.c_int32, _VP]),
    "gated_rmsnorm_fwd_strided": (ctypes.c_int32, [_VP, _I64, _VP, _I64, _VP, _VP, _I64,
                                                    _I64, ctypes.c_int32, ctypes.c_float,
                                                    ctypes.c_int32, _VP]),
    "gated_rmsnorm_bwd_strided": (ctypes.c_int32, [_VP, _I64, _VP, _I64, _VP, _VP, _I64,
                                                    _VP, _I64, _VP, _I64, _VP, _VP,
                                                    ctypes.c_size_t, _I64, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32, _VP]),
    "gated_rmsnorm_ckpt_step_strided": (ctypes.c_int32, [_VP, _I64, _VP, _I64, _VP, _VP,
                                                          _I64, _VP, _I64, _VP, _I64, _VP,
                                                          _I64, _VP, _VP, ctypes.c_size_t,
                                                          _I64, ctypes.c_int32,
                                                          ctypes.c_float, ctypes.c_int32,
                                                          ctypes.c_int32, ctypes.c_int32,
                                                          _VP]),
    "gated_rmsnorm_bwd_noalloc": (ctypes.c_int32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                    ctypes.c_int64, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_int32,
                                                    ctypes.c_int32, _VP]),
    "gated_rmsnorm_workspace_init": (ctypes.c_int32, [_VP, ctypes.c_size_t, _VP]),
    "gated_rmsnorm_workspace_init_bytes": (ctypes.c_size_t, []),
    "gated_rmsnorm_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
}


def load_library(path=None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = pathlib.Path(path) if path is not None else library_path()
        if not p.exists():
            raise RuntimeError(
                f"{p} is missing: build it with `python -m silu_gated_rmsnorm_amd.build`"
                " (the HIP kernels are the only implementation)")
        lib = ctypes.CDLL(str(p))
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().gated_rmsnorm_status_string(status).decode()
        raise GatedRMSNormError(status, msg)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"expected bfloat16, float16 or float32, got {t.dtype}")
    return code


def _act(name: str, t: torch.Tensor, like=None):
    """(pointer, row stride in elements) of a [rows, D] activation.

    Rows may be strided (a column slice of a wider buffer, e.g. one half of a
    fused projection) as long as the elements of a row are contiguous.  With
    `like` (the input x), the dtype and shape must match it."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name}: expected a GPU tensor")
    if t.dtype not in _DTYPE_CODES:
        raise TypeError(f"{name}: expected bfloat16, float16 or float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[1] not in SUPPORTED_D:
        raise ValueError(f"{name}: expected shape [rows, D], D in {SUPPORTED_D}, "
                         f"got {tuple(t.shape)}")
    if like is not None:
        if t.device != like.device:
            raise ValueError(f"{name}: expected a tensor on {like.device}, got {t.device}")
        if t.dtype != like.dtype:
            raise TypeError(f"{name}: expected {like.dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(like.shape):
            raise ValueError(f"{name}: expected shape {tuple(like.shape)}, got {tuple(t.shape)}")
    if t.stride(1) != 1:
        raise ValueError(f"{name}: the elements of a row must be contiguous")
    D = t.shape[1]
    stride = t.stride(0) if t.shape[0] > 1 else D
    return t.data_ptr(), stride


def _weight(w: torch.Tensor, x: torch.Tensor) -> int:
    if not isinstance(w, torch.Tensor) or w.device.type != "cuda":
        raise TypeError("w: expected a GPU tensor")
    D = x.shape[1]
    if w.device != x.device:
        raise ValueError(f"w: expected a tensor on {x.device}, got {w.device}")
    if w.dtype != x.dtype or w.shape != (D,) or not w.is_contiguous():
        raise ValueError(f"w: expected a contiguous {x.dtype} [{D}] tensor")
    return w.data_ptr()


def gated_rmsnorm_workspace_bytes(rows: int, D: int = D_DEFAULT) -> int:
    return int(load_library().gated_rmsnorm_workspace_bytes(rows, D))


def new_workspace(rows: int, device, D: int = D_DEFAULT) -> torch.Tensor:
    """A zero-filled workspace for the backward of `rows` rows of width D.

    Its arrival counters start at zero and every backward leaves them at
    zero, so the workspace can be reused by any later call whose
    gated_rmsnorm_workspace_bytes() it covers."""
    need = max(gated_rmsnorm_workspace_bytes(rows, D), 16)
    return torch.zeros(need, dtype=torch.uint8, device=device)


def gated_rmsnorm_workspace_init(workspace: torch.Tensor) -> None:
    """Zero the arrival counters of a workspace (enqueued on the current stream)."""
    lib = load_library()
    _check(lib.gated_rmsnorm_workspace_init(workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(workspace)))


def _workspace(rows, D, device, workspace):
    if workspace is None:
        # one extra allocation per call; pass a workspace to avoid it
        workspace = new_workspace(rows, device, D)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace: expected a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def gated_rmsnorm_fwd(x, g, w, eps: float = 1e-6, y=None):
    """y = x * rsqrt(mean(x^2) + eps) * w * silu(g) row by row; returns y."""
    lib = load_library()
    (px, sx) = _act("x", x)
    rows, D = x.shape
    (pg, sg), pw = _act("g", g, x), _weight(w, x)
    if y is None:
        y = _new_act(x)
    py, sy = _act("y", y, x)
    dt = _dtype_code(x)
    if sx == sg == sy == D:
        st = lib.gated_rmsnorm_fwd(px, pg, pw, py, rows, D, float(eps), dt, _stream(x))
    else:
        st = lib.gated_rmsnorm_fwd_strided(px, sx, pg, sg, pw, py, sy, rows, D, float(eps),
                                           dt, _stream(x))
    _check(st)
    return y


def gated_rmsnorm_bwd(x, g, w, dy, eps: float = 1e-6, dw_fp32: bool = False,
                      dx=None, dg=None, dw=None, workspace=None, deterministic: bool = True):
    """Gradients of sum(dy * y): returns (dx, dg, dw); dw is FP32 if dw_fp32,
    else of x's dtype.

    deterministic=False sums dw with float atomics (bits may vary per run)."""
    lib = load_library()
    (px, sx) = _act("x", x)
    rows, D = x.shape
    (pg, sg), pw = _act("g", g, x), _weight(w, x)
    pdy, sdy = _act("dy", dy, x)
    dx = _new_act(x) if dx is None else dx
    dg = _new_act(x) if dg is None else dg
    (pdx, sdx), (pdg, sdg) = _act("dx", dx, x), _act("dg", dg, x)
    dw = _dw(dw, dw_fp32, x)
    ws, ws_bytes = _workspace(rows, D, x.device, workspace)
    dt = _dtype_code(x)
    if deterministic and sx == sg == sdy == sdx == sdg == D:
        st = lib.gated_rmsnorm_bwd(px, pg, pw, pdy, pdx, pdg, dw.data_ptr(), ws.data_ptr(),
                                   ws_bytes, rows, D, float(eps), dt, int(bool(dw_fp32)),
                                   _stream(x))
    else:
        st = lib.gated_rmsnorm_bwd_strided(px, sx, pg, sg, pw, pdy, sdy, pdx, sdx, pdg, sdg,
                                           dw.data_ptr(), ws.data_ptr(), ws_bytes, rows, D,
                                           float(eps), dt, int(bool(dw_fp32)),
                                           int(bool(deterministic)), _stream(x))
    _check(st)
    return dx, dg, dw


def gated_rmsnorm_bwd_noalloc(x, g, w, dy, dx, dg, dw, eps: float = 1e-6):
    """gated_rmsnorm_bwd on the library's static scratch (no workspace): for
    callers that cannot allocate.  x, g, dy, dx, dg are packed [rows, D]
    tensors; dw is an FP32 or x-typed [D] tensor (its dtype selects dw_fp32).
    Returns (dx, dg, dw).  Calls that overlap on one GPU share the scratch."""
    lib = load_library()
    (px, sx) = _act("x", x)
    rows, D = x.shape
    (pg, sg), pw = _act("g", g, x), _weight(w, x)
    pdy, sdy = _act("dy", dy, x)
    (pdx, sdx), (pdg, sdg) = _act("dx", dx, x), _act("dg", dg, x)
    if not (sx == sg == sdy == sdx == sdg == D):
        raise ValueError("gated_rmsnorm_bwd_noalloc takes packed rows only")
    dw_fp32 = dw.dtype == torch.float32 and x.dtype != torch.float32
    dw = _dw(dw, dw_fp32, x)
    _check(lib.gated_rmsnorm_bwd_noalloc(px, pg, pw, pdy, pdx, pdg, dw.data_ptr(), rows, D,
                                         float(eps), _dtype_code(x), int(dw_fp32), _stream(x)))
    return dx, dg, dw


def gated_rmsnorm_ckpt_step(x, g, w, dy, eps: float = 1e-6, dw_fp32: bool = False,
                            y=None, dx=None, dg=None, dw=None, workspace=None,
                            deterministic: bool = True):
    """Forward, recomputed forward, backward: returns (y, dx, dg, dw)."""
    lib = load_library()
    (px, sx) = _act("x", x)
    rows, D = x.shape
    (pg, sg), pw = _act("g", g, x), _weight(w, x)
    pdy, sdy = _act("dy", dy, x)
    y = _new_act(x) if y is None else y
    dx = _new_act(x) if dx is None else dx
    dg = _new_act(x) if dg is None else dg
    (py, sy), (pdx, sdx), (pdg, sdg) = (_act("y", y, x), _act("dx", dx, x),
                                        _act("dg", dg, x))
    dw = _dw(dw, dw_fp32, x)
    ws, ws_bytes = _workspace(rows, D, x.device, workspace)
    dt = _dtype_code(x)
    if deterministic and sx == sg == sdy == sy == sdx == sdg == D:
        st = lib.gated_rmsnorm_ckpt_step(px, pg, pw, pdy, py, pdx, pdg, dw.data_ptr(),
                                         ws.data_ptr(), ws_bytes, rows, D, float(eps), dt,
                                         int(bool(dw_fp32)), _stream(x))
    else:
        st = lib.gated_rmsnorm_ckpt_step_strided(px, sx, pg, sg, pw, pdy, sdy, py, sy, pdx,
                                                 sdx, pdg, sdg, dw.data_ptr(), ws.data_ptr(),
                                                 ws_bytes, rows, D, float(eps), dt,
                                                 int(bool(dw_fp32)), int(bool(deterministic)),
                                                 _stream(x))
    _check(st)
    return y, dx, dg, dw


def _new_act(like: torch.Tensor) -> torch.Tensor:
    return torch.empty(like.shape[0], like.shape[1], dtype=like.dtype, device=like.device)


def _dw(dw, dw_fp32, x):
    D = x.shape[1]
    dw_dtype = torch.float32 if dw_fp32 else x.dtype
    if dw is None:
        return torch.empty(D, dtype=dw_dtype, device=x.device)
    if dw.dtype != dw_dtype or dw.shape != (D,) or dw.device != x.device:
        raise ValueError(f"dw: expected a {dw_dtype} [{D}] tensor on the inputs' device")
    return dw
