"""Seeded synthetic inputs for the SiLU-gated RMSNorm workloads.

This module draws random tensors and nothing else: it holds none of the
operator's arithmetic, so both the HIP path and the CPU oracle can consume
its bytes.  flashinfer PR #8701 ("perf(cake_rmsnorm_silu_gate_train):
L2-prefetching extra-long forward on SM107") times the operator on BF16
inputs of T x H rows ("How the tables were measured", Tables 1 and 2); the
distributions below are synthetic stand-ins of those shapes.

Recipe: a ``torch.Generator`` on ``device`` seeded with ``seed`` draws, in
order, x, g, dy (each ``[rows, D]`` standard normal, g scaled by ``g_std``),
then w = 1 + 0.1 * N(0, 1) of shape ``[D]``, then (only when
``outlier_frac > 0``) a permutation of the rows whose first
``int(rows * outlier_frac)`` entries select outlier rows of x, which are
multiplied by ``outlier_scale``.  All draws are float32 and are rounded to
the storage type (BF16 by default; FP16 or FP32 on request; round to
nearest even) once, at the end.  The same seed gives
different numbers on the CPU and on the GPU (different generators); each
test hands the very same bytes to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """One benchmark shape: rows = T * H rows of D values."""
    name: str
    T: int
    H: int
    D: int = 128
    g_std: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0
    eps: float = 1e-6

    @property
    def rows(self) -> int:
        return self.T * self.H


# The shapes the benchmark and the parity tests use (all D = 128,
# eps = 1e-6, seed 0).  1031x48 and 7684x48 appear in Table 2 of PR #8701
# and 16384x32 (the H = 32 head count) in its Tables 1 and 2; the larger
# three T x 48 shapes extend the same family.
WORKLOADS = {
    "1031x48": Workload("1031x48", 1031, 48),
    "7684x48": Workload("7684x48", 7684, 48),
    "32768x48": Workload("32768x48", 32768, 48),
    "65536x48": Workload("65536x48", 65536, 48),
    "262144x48_outliers": Workload("262144x48_outliers", 262144, 48,
                                   g_std=2.0, outlier_frac=0.01),
    "16384x32": Workload("16384x32", 16384, 32),
}


def make_inputs(rows: int, D: int = 128, *, seed: int = 0,
                device="cpu", g_std: float = 1.0,
                outlier_frac: float = 0.0, outlier_scale: float = 100.0,
                dtype=torch.bfloat16):
    """Return ``dict(x, g, dy, w)`` of ``dtype`` tensors on ``device``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(shape):
        return torch.randn(shape, generator=gen, device=device,
                           dtype=torch.float32)

    x = normal((rows, D))
    g = normal((rows, D))
    if g_std != 1.0:
        g.mul_(g_std)
    dy = normal((rows, D))
    w = normal((D,)).mul_(0.1).add_(1.0)
    if outlier_frac > 0.0 and rows > 0:
        perm = torch.randperm(rows, generator=gen, device=device)
        sel = perm[: int(rows * outlier_frac)]
        x[sel] *= outlier_scale
    return {
        "x": x.to(dtype),
        "g": g.to(dtype),
        "dy": dy.to(dtype),
        "w": w.to(dtype),
    }


def make_workload_inputs(wl: Workload, *, seed: int = 0, device="cpu",
                         dtype=torch.bfloat16):
    """``make_inputs`` with the distributions of a named workload."""
    return make_inputs(wl.rows, wl.D, seed=seed, device=device,
                       g_std=wl.g_std, outlier_frac=wl.outlier_frac,
                       outlier_scale=wl.outlier_scale, dtype=dtype)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a BF16 tensor as a numpy uint16 array (copied to host)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray, device="cpu") -> torch.Tensor:
    """BF16 tensor from uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
