"""Pins for the FP64 oracle: facts fixed by the mathematics, not by the oracle.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a wrong index, a transposed operand, an eps in the wrong place)
fails at least one of them:

* hand-derived worked examples (tests/golden/worked_examples.json);
* closed forms: constant rows, the RMS of the normalised row, D = 1;
* special gates: g = 0 (y = 0, s'(0) = 1/2), large positive and very
  negative g;
* invariants: scale invariance at eps = 0, dx orthogonal to x at eps = 0,
  dw = sum_i dy*y / w, row independence, permutation invariance of dw;
* torch autograd in float64 on library primitives (rms_norm, silu);
* central finite differences of L = sum(dy * y) on tiny inputs.

The operator is the SiLU-gated RMSNorm of flashinfer PR #8701
("perf(cake_rmsnorm_silu_gate_train): L2-prefetching extra-long forward on
SM107", PR description); the page prints no formula or values.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
LN3 = math.log(3.0)
_ENV = {"sqrt": math.sqrt, "log": math.log}


def _ev(e):
    return float(eval(str(e), {"__builtins__": {}}, _ENV))


def _rand(rows, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, D)) * scale


# --------------------------------------------------------------------------
# worked examples

def _examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_worked_example(ex):
    x = np.array(ex["x"], dtype=np.float64)
    g = np.array([[_ev(v) for v in ex["g"]]], dtype=np.float64)
    w = np.array(ex["w"], dtype=np.float64)
    dy = np.array(ex["dy"], dtype=np.float64)
    eps = ex["eps"]
    y = oracle.fwd(x, g, w, eps)
    dx, dg, dw = oracle.bwd(x, g, w, dy, eps)
    for name, got in (("y", y), ("dx", dx), ("dg", dg)):
        want = np.array([[_ev(v) for v in row] for row in ex[name]])
        np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15, err_msg=name)
    want_dw = np.array([_ev(v) for v in ex["dw"]])
    np.testing.assert_allclose(dw, want_dw, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# closed forms

@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3])
@pytest.mark.parametrize("D", [1, 4, 128])
def test_constant_row(eps, D):
    """x = c*1 gives n_j = c / sqrt(c^2 + eps) (unit RMS as eps -> 0)."""
    cs = np.array([1.0, -2.5, 100.0, 1e-3])
    x = np.repeat(cs[:, None], D, axis=1)
    g = np.full_like(x, LN3)                 # silu(ln 3) = 3/4 ln 3
    w = np.linspace(0.5, 1.5, D)
    y = oracle.fwd(x, g, w, eps)
    n = cs / np.sqrt(cs * cs + eps)
    want = n[:, None] * w[None, :] * (0.75 * LN3)
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rms_of_normalised_row(eps):
    """RMS_j(n_ij) = sqrt(ms_i / (ms_i + eps)) for every row."""
    x = _rand(7, 128, 1) * np.array([1, 3, 0.01, 100, 1, 2, 0.5])[:, None]
    g = np.full_like(x, LN3)
    w = np.ones(128)
    n = oracle.fwd(x, g, w, eps) / (0.75 * LN3)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)),
                               np.sqrt(ms / (ms + eps)), rtol=1e-14)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_d1(eps):
    """D = 1: n = x / sqrt(x^2 + eps) and dx = r dn eps / (x^2 + eps)."""
    xs = np.array([[0.3], [-2.0], [7.0]])
    g = np.full_like(xs, -LN3)               # sigma = 1/4, silu = -ln3/4
    w = np.array([1.7])
    dy = np.array([[1.0], [-0.5], [2.0]])
    y = oracle.fwd(xs, g, w, eps)
    n = xs / np.sqrt(xs * xs + eps)
    np.testing.assert_allclose(y, n * 1.7 * (-0.25 * LN3), rtol=1e-14)
    dx, _, _ = oracle.bwd(xs, g, w, dy, eps)
    r = 1.0 / np.sqrt(xs * xs + eps)
    dn = dy * 1.7 * (-0.25 * LN3)
    np.testing.assert_allclose(dx, r * dn * eps / (xs * xs + eps),
                               rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# special gates

def test_gate_zero():
    """g = 0: y = 0 exactly, and dg = 1/2 dy w n (silu'(0) = 1/2)."""
    x = _rand(5, 128, 2)
    w = 1.0 + 0.1 * _rand(1, 128, 3)[0]
    dy = _rand(5, 128, 4)
    eps = 1e-6
    y0 = oracle.fwd(x, np.zeros_like(x), w, eps)
    assert np.all(y0 == 0.0)
    # n from the forward with a constant gate ln 3 (silu = 3/4 ln 3)
    n = oracle.fwd(x, np.full_like(x, LN3), np.ones(128), eps) / (0.75 * LN3)
    _, dg, dw = oracle.bwd(x, np.zeros_like(x), w, dy, eps)
    np.testing.assert_allclose(dg, 0.5 * dy * w * n, rtol=1e-13, atol=1e-15)
    assert np.all(dw == 0.0)


def test_gate_large_positive():
    """y / g -> n w as g -> +inf (sigma -> 1); dg -> dy w n."""
    x = _rand(3, 128, 5)
    w = 1.0 + 0.1 * _rand(1, 128, 6)[0]
    dy = _rand(3, 128, 7)
    eps = 1e-6
    G = 40.0                                   # 1 - sigma(40) ~ 4e-18
    n = oracle.fwd(x, np.full_like(x, LN3), np.ones(128), eps) / (0.75 * LN3)
    y = oracle.fwd(x, np.full_like(x, G), w, eps)
    np.testing.assert_allclose(y / G, n * w, rtol=1e-14)
    _, dg, _ = oracle.bwd(x, np.full_like(x, G), w, dy, eps)
    np.testing.assert_allclose(dg, dy * w * n, rtol=1e-13)


def test_gate_very_negative_no_nan():
    """g -> -inf: y, dg, dx, dw -> 0 without NaN or overflow."""
    x = _rand(3, 128, 8)
    w = np.ones(128)
    dy = _rand(3, 128, 9)
    g = np.full_like(x, -1000.0)
    y = oracle.fwd(x, g, w, 1e-6)
    dx, dg, dw = oracle.bwd(x, g, w, dy, 1e-6)
    for a in (y, dx, dg, dw):
        assert np.all(np.isfinite(a))
        assert np.all(a == 0.0)


def test_zero_row():
    """An all-zero row with eps > 0: r = eps^-1/2, y = 0, dx = r dy w silu(g)."""
    eps = 1e-6
    x = np.zeros((2, 128))
    g = _rand(2, 128, 10)
    w = 1.0 + 0.1 * _rand(1, 128, 11)[0]
    dy = _rand(2, 128, 12)
    y = oracle.fwd(x, g, w, eps)
    assert np.all(y == 0.0)
    dx, dg, dw = oracle.bwd(x, g, w, dy, eps)
    silu = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    np.testing.assert_allclose(dx, dy * w * silu / math.sqrt(eps), rtol=1e-13)
    assert np.all(dg == 0.0) and np.all(dw == 0.0)


# --------------------------------------------------------------------------
# invariants

@pytest.mark.parametrize("alpha", [100.0, 1e-3, -7.0])
def test_scale_invariance_eps0(alpha):
    x = _rand(4, 128, 13)
    g = _rand(4, 128, 14)
    w = 1.0 + 0.1 * _rand(1, 128, 15)[0]
    y1 = oracle.fwd(x, g, w, 0.0)
    y2 = oracle.fwd(alpha * x, g, w, 0.0)
    np.testing.assert_allclose(y2, np.sign(alpha) * y1, rtol=1e-13, atol=1e-15)


def test_dx_orthogonal_to_x_eps0():
    """With eps = 0 the function is scale invariant in x, so dx . x = 0."""
    x = _rand(6, 128, 16)
    g = _rand(6, 128, 17)
    w = 1.0 + 0.1 * _rand(1, 128, 18)[0]
    dy = _rand(6, 128, 19)
    dx, _, _ = oracle.bwd(x, g, w, dy, 0.0)
    dots = np.sum(dx * x, axis=1)
    scale = np.linalg.norm(dx, axis=1) * np.linalg.norm(x, axis=1)
    assert np.all(np.abs(dots) <= 1e-13 * scale)
    # with eps > 0 the projection is not zero: dx . x = r eps/(ms+eps) sum(dn x)
    dx_e, _, _ = oracle.bwd(x, g, w, dy, 0.5)
    assert np.all(np.abs(np.sum(dx_e * x, axis=1)) > 1e-6 * scale)


def test_dw_is_sum_dy_y_over_w():
    """Since y = n w s, dw_j = sum_i dy_ij y_ij / w_j."""
    x = _rand(33, 128, 20)
    g = _rand(33, 128, 21)
    w = 1.0 + 0.1 * _rand(1, 128, 22)[0]
    dy = _rand(33, 128, 23)
    y = oracle.fwd(x, g, w, 1e-6)
    _, _, dw = oracle.bwd(x, g, w, dy, 1e-6)
    np.testing.assert_allclose(dw, np.sum(dy * y, axis=0) / w, rtol=1e-12, atol=1e-13)


def test_rows_independent_and_dw_order_free():
    """Each row's outputs depend on that row only (bitwise); dw is a sum."""
    rows = 50
    x = _rand(rows, 128, 24)
    g = _rand(rows, 128, 25)
    w = 1.0 + 0.1 * _rand(1, 128, 26)[0]
    dy = _rand(rows, 128, 27)
    y = oracle.fwd(x, g, w, 1e-6)
    dx, dg, dw = oracle.bwd(x, g, w, dy, 1e-6)
    idx = np.array([49, 3, 17, 0, 25])
    ys = oracle.fwd(x[idx].copy(), g[idx].copy(), w, 1e-6)
    dxs, dgs, _ = oracle.bwd(x[idx].copy(), g[idx].copy(), w, dy[idx].copy(), 1e-6)
    assert np.array_equal(ys, y[idx])
    assert np.array_equal(dxs, dx[idx]) and np.array_equal(dgs, dg[idx])
    perm = np.random.default_rng(0).permutation(rows)
    _, _, dwp = oracle.bwd(x[perm].copy(), g[perm].copy(), w, dy[perm].copy(), 1e-6)
    np.testing.assert_allclose(dwp, dw, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# library routines: torch autograd in float64

@pytest.mark.parametrize("eps", [1e-6, 1e-2])
@pytest.mark.parametrize("D", [1, 8, 64, 128, 256])
def test_against_torch_autograd_fp64(eps, D):
    rows = 9
    x = _rand(rows, D, 30) * np.linspace(0.1, 10, rows)[:, None]
    g = _rand(rows, D, 31) * 3.0
    g[0, 0] = 20.0
    g[-1, -1] = -20.0
    w = 1.0 + 0.1 * _rand(1, D, 32)[0]
    dy = _rand(rows, D, 33)
    tx, tg, tw = (torch.tensor(a, requires_grad=True) for a in (x, g, w))
    ty = torch.nn.functional.rms_norm(tx, (D,), eps=eps) * tw \
        * torch.nn.functional.silu(tg)
    (ty * torch.from_numpy(dy)).sum().backward()
    y = oracle.fwd(x, g, w, eps)
    dx, dg, dw = oracle.bwd(x, g, w, dy, eps)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-14)
    for got, want in ((dx, tx.grad), (dg, tg.grad), (dw, tw.grad)):
        want = want.numpy()
        np.testing.assert_allclose(got, want, rtol=1e-11,
                                   atol=1e-12 * max(1.0, np.abs(want).max()))


# --------------------------------------------------------------------------
# central finite differences of L = sum(dy * y)

def _loss(x, g, w, dy, eps):
    return float(np.sum(dy * oracle.fwd(x, g, w, eps)))


def _fd(arr, f):
    out = np.empty_like(arr)
    flat = arr.reshape(-1)
    o = out.reshape(-1)
    for k in range(flat.size):
        v = flat[k]
        h = 1e-6 * max(1.0, abs(v))
        flat[k] = v + h
        lp = f()
        flat[k] = v - h
        lm = f()
        flat[k] = v
        o[k] = (lp - lm) / (2 * h)
    return out


@pytest.mark.parametrize("rows,D", [(r, d) for r in (1, 3) for d in (1, 2, 8, 16, 128)]
                         + [(1, 64), (1, 256)])
@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_finite_differences(rows, D, eps):
    rng = np.random.default_rng(1000 * rows + D)
    x = rng.standard_normal((rows, D))
    g = rng.standard_normal((rows, D))
    g.reshape(-1)[0] = 20.0
    if g.size > 1:
        g.reshape(-1)[-1] = -20.0
    w = 1.0 + 0.1 * rng.standard_normal(D)
    dy = rng.standard_normal((rows, D))
    dx, dg, dw = oracle.bwd(x, g, w, dy, eps)

    def f():
        return _loss(x, g, w, dy, eps)

    for got, arr in ((dx, x), (dg, g), (dw, w)):
        num = _fd(arr, f)
        tol = 1e-6 * max(1.0, np.abs(num).max())
        assert np.max(np.abs(got - num)) <= tol


# --------------------------------------------------------------------------
# BF16 entry points and rounding helper

def test_bf16_entry_equals_f64_entry():
    rng = np.random.default_rng(40)
    x = torch.from_numpy(rng.standard_normal((20, 128))).to(torch.bfloat16)
    g = torch.from_numpy(rng.standard_normal((20, 128))).to(torch.bfloat16)
    dy = torch.from_numpy(rng.standard_normal((20, 128))).to(torch.bfloat16)
    w = torch.from_numpy(1 + 0.1 * rng.standard_normal(128)).to(torch.bfloat16)
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in (x, g, w, dy)]
    f64 = [t.double().numpy() for t in (x, g, w, dy)]
    for b, d in zip(bits, f64):
        assert np.array_equal(oracle.bf16_to_f64(b), d)
    assert np.array_equal(oracle.fwd(bits[0], bits[1], bits[2], 1e-6),
                          oracle.fwd(f64[0], f64[1], f64[2], 1e-6))
    got = oracle.bwd(*bits, 1e-6)
    want = oracle.bwd(*f64, 1e-6)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


def test_round_bf16_known_values():
    cases = [
        (1.0, 0x3F80), (-1.0, 0xBF80), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie
        (2.0 ** -133, 0x0001),                # smallest subnormal
        (2.0 ** -134, 0x0000),                # half of it: tie -> even zero
        (3.0 * 2.0 ** -135, 0x0001),
        (3.3895313892515355e38, 0x7F7F),      # largest finite BF16
        (3.4e38, 0x7F80),                     # rounds past it -> inf
    ]
    for v, bits in cases:
        assert int(oracle.round_bf16(np.array([v]))[0]) == bits, v


def test_round_bf16_matches_torch_on_binary32():
    """torch's float32 -> bfloat16 cast rounds to nearest even."""
    rng = np.random.default_rng(41)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.float32(rng.standard_normal(1000)) * 1e-39])
    v32 = v.astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(v32.astype(np.float64))
    assert np.array_equal(got, want)
