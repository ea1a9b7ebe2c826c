"""FP64 CPU oracle for the SiLU-gated RMSNorm training forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``silu_gated_rmsnorm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``gated_rmsnorm_oracle.c`` (plain C, double
precision); this module only builds it with gcc, loads it with ctypes and
marshals numpy arrays.  The definition it follows is written out at the top
of the C file (operator named in flashinfer PR #8701,
"perf(cake_rmsnorm_silu_gate_train): L2-prefetching extra-long forward on
SM107", PR description and commit 10c6017 message).

Arrays:
  * BF16 tensors are passed as ``numpy.uint16`` arrays of bit patterns, shape
    ``[rows, D]`` (row-major, rows packed); ``w`` has shape ``[D]``.
  * Double tensors (for finite differences) are ``numpy.float64`` arrays.
  * Results are ``numpy.float64``.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess
import threading

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
_SRC = _HERE / "gated_rmsnorm_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lock = threading.Lock()
_lib = None


def build(verbose: bool = False) -> pathlib.Path:
    """Compile the C oracle with gcc (OpenMP, -O2, strict IEEE: no fast-math)."""
    tmp = _LIB_PATH.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off",
           str(_SRC), "-o", str(tmp), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if (not _LIB_PATH.exists()
                or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime):
            build()
        lib = ctypes.CDLL(str(_LIB_PATH))
        dp = ctypes.POINTER(ctypes.c_double)
        up = ctypes.POINTER(ctypes.c_uint16)
        i64 = ctypes.c_int64
        dbl = ctypes.c_double
        lib.orc_fwd_f64.argtypes = [dp, dp, dp, i64, i64, dbl, dp]
        lib.orc_bwd_f64.argtypes = [dp, dp, dp, dp, i64, i64, dbl, dp, dp, dp]
        lib.orc_fwd_bf16.argtypes = [up, up, up, i64, i64, dbl, dp]
        lib.orc_bwd_bf16.argtypes = [up, up, up, up, i64, i64, dbl, dp, dp, dp]
        lib.orc_round_bf16.argtypes = [dbl]
        lib.orc_round_bf16.restype = ctypes.c_uint16
        lib.orc_round_bf16_array.argtypes = [dp, i64, up]
        lib.orc_num_threads.restype = ctypes.c_int
        for fn in (lib.orc_fwd_f64, lib.orc_bwd_f64, lib.orc_fwd_bf16,
                   lib.orc_bwd_bf16, lib.orc_round_bf16_array):
            fn.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check_2d(name, a, dtype):
    if a.dtype != dtype or a.ndim != 2 or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected a C-contiguous 2-D {dtype} array")


def _check_w(w, D, dtype):
    if w.dtype != dtype or w.shape != (D,) or not w.flags.c_contiguous:
        raise TypeError(f"w: expected a contiguous [{D}] {dtype} array")


def num_threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS or all cores)."""
    return int(_load().orc_num_threads())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns (they are the top half of binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest BF16 (ties to even) of each double, as uint16 bit patterns."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_round_bf16_array(_ptr(a, ctypes.c_double), a.size,
                                 _ptr(out, ctypes.c_uint16))
    return out


def fwd(x: np.ndarray, g: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x * rsqrt(mean(x^2) + eps) * w * silu(g), per row, in FP64.

    x, g are [rows, D] and w is [D]; all uint16 (BF16 bits) or all float64.
    """
    lib = _load()
    if x.dtype == np.uint16:
        _check_2d("x", x, np.uint16)
        _check_2d("g", g, np.uint16)
        rows, D = x.shape
        _check_w(w, D, np.uint16)
        if g.shape != x.shape:
            raise ValueError("g must have the shape of x")
        y = np.empty((rows, D), dtype=np.float64)
        lib.orc_fwd_bf16(_ptr(x, ctypes.c_uint16), _ptr(g, ctypes.c_uint16),
                         _ptr(w, ctypes.c_uint16), rows, D, float(eps),
                         _ptr(y, ctypes.c_double))
        return y
    _check_2d("x", x, np.float64)
    _check_2d("g", g, np.float64)
    rows, D = x.shape
    _check_w(w, D, np.float64)
    if g.shape != x.shape:
        raise ValueError("g must have the shape of x")
    y = np.empty((rows, D), dtype=np.float64)
    lib.orc_fwd_f64(_ptr(x, ctypes.c_double), _ptr(g, ctypes.c_double),
                    _ptr(w, ctypes.c_double), rows, D, float(eps),
                    _ptr(y, ctypes.c_double))
    return y


def bwd(x: np.ndarray, g: np.ndarray, w: np.ndarray, dy: np.ndarray,
        eps: float, want_dw: bool = True):
    """Gradients (dx, dg, dw) of L = sum(dy * y), in FP64.

    dw is the plain row-order sum over all rows given (None if ``want_dw`` is
    False, which is how a sample of rows of a large problem is checked).
    """
    lib = _load()
    bf = x.dtype == np.uint16
    dt = np.uint16 if bf else np.float64
    ct = ctypes.c_uint16 if bf else ctypes.c_double
    for name, a in (("x", x), ("g", g), ("dy", dy)):
        _check_2d(name, a, dt)
        if a.shape != x.shape:
            raise ValueError(f"{name} must have the shape of x")
    rows, D = x.shape
    _check_w(w, D, dt)
    dx = np.empty((rows, D), dtype=np.float64)
    dg = np.empty((rows, D), dtype=np.float64)
    dw = np.empty((D,), dtype=np.float64) if (want_dw or not bf) else None
    dwp = _ptr(dw, ctypes.c_double) if dw is not None else None
    fn = lib.orc_bwd_bf16 if bf else lib.orc_bwd_f64
    fn(_ptr(x, ct), _ptr(g, ct), _ptr(w, ct), _ptr(dy, ct), rows, D,
       float(eps), _ptr(dx, ctypes.c_double), _ptr(dg, ctypes.c_double), dwp)
    return dx, dg, dw
