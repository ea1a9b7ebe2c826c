"""Comparison metrics of GPU results against the FP64 oracle.

The tolerances (max relative error 1e-2 for y, dx and dg; FP32 dw relative
error 1e-4; BF16 dw within 2 BF16 ulp) are the bars this project sets for
itself.  Near zero and under cancellation, "relative" needs a floor; the
floors used are:

* y, dx, dg: per element, err = |gpu - ref| / max(|ref|, tau * rms(ref row))
  with tau = 1e-3.  A row whose reference is identically zero must be zero.
  The floor is per row so rows scaled by 100 (outlier rows) are held to the
  same relative standard as the others.
* FP32 dw: |gpu - ref| / max(|ref_j|, 1e-2 * max_k |ref_k|).
* BF16 dw: distance in units in the last place between the GPU bits and the
  BF16 nearest (ties to even) to the exact value, counted on the monotone
  integer order of BF16 patterns; columns with |ref| < 1e-2 max|ref| are
  held to |gpu - ref| <= 2 ulp(1e-2 max|ref|) instead.  FP16 dw: the same
  with FP16 patterns and ulps.

Other storage types (FP16 and FP32 activations) get bars derived from the
arithmetic.  It is FP32 in every case, with hardware exp2, reciprocal and
reciprocal square root (about 1 ulp each); the worst elements are those where
terms cancel: dx = r (dn - n c) and silu'(g) = sig + s (1 - sig), which is 0
near g = -1.28.  There an error of a few FP32 ulps (~1e-7) of the largest
term, |dy w n| up to ~5 times its row RMS, measured against the floor
tau * rms(row) = 1e-3 * rms, gives up to ~1e-3.  FP32 outputs add nothing,
so their bar is 1e-3; FP16 outputs add one rounding of at most 2^-11
(4.9e-4) relative, so theirs is 2e-3.  (BF16's rounding, 2^-8, dominates its
1e-2 bar.)
"""
from __future__ import annotations

import numpy as np

import oracle

Y_TOL = 1e-2
Y_TOL_F16 = 2e-3
Y_TOL_F32 = 1e-3
DW32_TOL = 1e-4
DW16_ULPS = 2
TAU = 1e-3


def act_err(gpu: np.ndarray, ref: np.ndarray, tau: float = TAU):
    """Return (err, n_floor_binds, unfloored_max) for [rows, D] arrays."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.shape != ref.shape:
        raise ValueError("shape mismatch")
    if gpu.size == 0:
        return 0.0, 0, 0.0
    if not np.all(np.isfinite(gpu)):
        return float("inf"), 0, float("inf")
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    zero_rows = rms[:, 0] == 0.0
    if np.any(gpu[zero_rows] != 0.0):
        return float("inf"), 0, float("inf")
    floor = np.maximum(np.abs(ref), tau * rms)
    diff = np.abs(gpu - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(floor > 0, diff / np.where(floor > 0, floor, 1.0), 0.0)
        unf = np.where(np.abs(ref) > 0, diff / np.where(ref != 0, np.abs(ref), 1.0), 0.0)
    binds = int(np.count_nonzero(np.abs(ref) < tau * rms))
    return float(rel.max()), binds, float(unf.max())


def dw32_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0.0:
        return 0.0 if np.all(gpu == 0.0) else float("inf")
    floor = np.maximum(np.abs(ref), 1e-2 * scale)
    return float(np.max(np.abs(gpu - ref) / floor))


def _bf16_order(bits: np.ndarray) -> np.ndarray:
    """Map BF16 patterns to integers that increase with the value (+0 = -0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bf16_ulp(v: float) -> float:
    a = abs(v)
    if a == 0.0:
        return 2.0 ** -133
    e = int(np.floor(np.log2(a)))
    return 2.0 ** max(e - 7, -133)


def dw16_check(gpu_bits: np.ndarray, ref: np.ndarray):
    """Return (max_ulps, ok) for a BF16 dw against the exact FP64 dw."""
    ref = np.asarray(ref, dtype=np.float64)
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    want = oracle.round_bf16(ref)
    dist = np.abs(_bf16_order(gpu_bits) - _bf16_order(want))
    scale = np.abs(ref).max()
    small = np.abs(ref) < 1e-2 * scale
    ok_big = np.all(dist[~small] <= DW16_ULPS)
    gpu = oracle.bf16_to_f64(gpu_bits)
    bound = DW16_ULPS * _bf16_ulp(1e-2 * scale) if scale > 0 else 0.0
    ok_small = np.all(np.abs(gpu[small] - ref[small]) <= bound)
    worst = int(dist[~small].max()) if np.any(~small) else 0
    return worst, bool(ok_big and ok_small)


def _f16_ulp(v: float) -> float:
    a = abs(v)
    if a < 2.0 ** -14:
        return 2.0 ** -24
    e = int(np.floor(np.log2(a)))
    return 2.0 ** (e - 10)


def dwf16_check(gpu_bits: np.ndarray, ref: np.ndarray):
    """Return (max_ulps, ok) for an FP16 dw against the exact FP64 dw.

    numpy converts float64 to float16 with one rounding, to nearest even."""
    ref = np.asarray(ref, dtype=np.float64)
    gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)
    want = ref.astype(np.float16).view(np.uint16)
    dist = np.abs(_bf16_order(gpu_bits) - _bf16_order(want))
    scale = np.abs(ref).max()
    small = np.abs(ref) < 1e-2 * scale
    ok_big = np.all(dist[~small] <= DW16_ULPS)
    gpu = gpu_bits.view(np.float16).astype(np.float64)
    bound = DW16_ULPS * _f16_ulp(1e-2 * scale) if scale > 0 else 0.0
    ok_small = np.all(np.abs(gpu[small] - ref[small]) <= bound)
    worst = int(dist[~small].max()) if np.any(~small) else 0
    return worst, bool(ok_big and ok_small)
