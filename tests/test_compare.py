"""The comparison metrics themselves (CPU): each bar accepts what it should and
rejects a planted error just beyond it."""
import numpy as np

import oracle
from _compare import act_err, dw16_check, dw32_err, dwf16_check


def test_act_err_floor_and_zero_rows():
    ref = np.array([[1.0, -2.0, 1e-9, 0.5], [0.0, 0.0, 0.0, 0.0]])
    assert act_err(ref.copy(), ref)[0] == 0.0
    got = ref.copy()
    got[0, 1] *= 1 + 5e-3                       # relative 5e-3 on a large element
    assert abs(act_err(got, ref)[0] - 5e-3) < 1e-12
    got = ref.copy()
    rms = np.sqrt(np.mean(ref[0] ** 2))
    got[0, 2] += 1e-3 * rms * 0.5               # half the floor on a tiny element
    assert abs(act_err(got, ref)[0] - 0.5) < 1e-9
    got = ref.copy()
    got[1, 3] = 1e-30                           # a zero row must stay zero
    assert act_err(got, ref)[0] == float("inf")


def test_dw32_err():
    ref = np.array([100.0, -50.0, 1e-6])
    got = ref * (1 + np.array([1e-5, -2e-5, 0.0]))
    assert abs(dw32_err(got, ref) - 2e-5) < 1e-12
    got = ref.copy()
    got[2] += 1e-2 * 100.0 * 3e-5               # small column: floor 1e-2 max|ref|
    assert abs(dw32_err(got, ref) - 3e-5) < 1e-12


def _bits16(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def test_dwf16_ulps():
    ref = np.array([1000.3, -3.14159, 0.25, 1e-7])
    exact = _bits16(ref)
    assert dwf16_check(exact, ref) == (0, True)
    off2 = exact.copy()
    off2[0] += 2                                # 2 ulp away from the nearest
    assert dwf16_check(off2, ref) == (2, True)
    off3 = exact.copy()
    off3[0] += 3
    assert dwf16_check(off3, ref)[1] is False


def test_dw16_ulps():
    ref = np.array([1000.3, -3.14159, 0.25, 1e-7])
    exact = oracle.round_bf16(ref)
    assert dw16_check(exact, ref) == (0, True)
    off3 = exact.copy()
    off3[0] += 3
    assert dw16_check(off3, ref)[1] is False
