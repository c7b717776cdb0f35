"""Pins of the two pieces of the oracle that every parity decision goes
through (CPU only):

* ``within_tolerance``, the acceptance rule of every parity test, the smoke
  check and the benchmark's check: |d - ref| <= 2^-7 |ref| + 1e-3 max|ref|
  per element, with max|ref| taken over the reference of the whole call, and
  a NaN in d failing.  The expected outcomes below are worked out by hand
  from that statement, with the arithmetic written in the comments.
* ``bf16_rne``, the one rounding of an exact FP64 value to BF16 that the
  bit-exact tests compare against: in the subnormal range [2^-133, 2^-126),
  at the boundary to the normal range, and at the overflow edge, against a
  brute force over every finite BF16 value in exact rational arithmetic.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def tol(d, ref):
    return oracle.within_tolerance(np.array(d, np.float64), np.array(ref, np.float64))


# ---- within_tolerance ------------------------------------------------------

def test_tolerance_just_inside_and_just_outside():
    # ref = [100, 1]: max|ref| = 100, so the absolute term is 0.1.  For the
    # element ref = 1 the bound is 1/128 + 0.1 = 0.1078125.
    ok, worst = tol([100.0, 1.1077], [100.0, 1.0])      # err 0.1077 -> ratio 0.998957
    assert ok and worst == pytest.approx(1077000 / 1078125, rel=1e-9)
    ok, worst = tol([100.0, 1.1079], [100.0, 1.0])      # err 0.1079 -> ratio 1.000812
    assert not ok and worst == pytest.approx(1079000 / 1078125, rel=1e-9)
    # the element ref = 100: bound 100/128 + 0.1 = 0.88125
    assert tol([100.8, 1.0], [100.0, 1.0])[0]           # err 0.8 -> ratio 0.9078
    assert not tol([100.9, 1.0], [100.0, 1.0])[0]       # err 0.9 -> ratio 1.0213
    # below the reference as well as above, and negative references
    assert tol([-100.0, -0.8923], [-100.0, -1.0])[0]    # err 0.1077
    assert not tol([-100.0, -0.8921], [-100.0, -1.0])[0]  # err 0.1079


def test_tolerance_ratio_at_the_bound():
    # err exactly equal to the bound passes (<=): ref = [128, 0], abs term
    # 0.128; element 1 has bound 0.128 and err 0.125 = 0.9765625 of it.
    ok, worst = tol([128.0, 0.125], [128.0, 0.0])
    assert ok and worst == pytest.approx(0.125 / 0.128, rel=1e-12)
    # element 0: bound 128/128 + 0.128 = 1.128; d = 129.128 is at it (up to
    # the FP64 rounding of 129.128), d = 129.2 is past it
    assert tol([129.127, 0.0], [128.0, 0.0])[0]
    assert not tol([129.2, 0.0], [128.0, 0.0])[0]


def test_tolerance_nan_and_inf_fail():
    assert not tol([1.0, float("nan")], [1.0, 0.5])[0]
    assert not tol([float("nan")], [0.0])[0]
    assert not tol([1.0, float("inf")], [1.0, 0.5])[0]
    assert not tol([float("-inf")], [1.0])[0]


def test_tolerance_takes_the_maximum_over_the_reference():
    # ref = [0.5, 0]: absolute term 1e-3 * 0.5 = 5e-4 for the zero element.
    # d = [0.503, 5.015e-4]: element 0 passes (err 0.003 <= 0.5/128 + 5e-4 =
    # 0.00440625); element 1 has err 5.015e-4 > 5e-4 and must fail.  Had the
    # maximum been taken over d (0.503, term 5.03e-4) it would pass.
    assert not tol([0.503, 5.015e-4], [0.5, 0.0])[0]
    # d = [0.497, 4.985e-4]: err 4.985e-4 <= 5e-4 passes.  With the maximum
    # over d (0.497, term 4.97e-4) it would fail.
    assert tol([0.497, 4.985e-4], [0.5, 0.0])[0]


def test_tolerance_relative_term_is_per_element():
    # A tiny reference next to a large one gets the absolute term only:
    # ref = [1000, 0.001]: bound of element 1 = 0.001/128 + 1.0.
    assert tol([1000.0, 1.0009], [1000.0, 0.001])[0]     # err 0.9999
    assert not tol([1000.0, 1.0011], [1000.0, 0.001])[0]  # err 1.0001
    # all-zero reference: every bound is 0, so only exact zeros pass
    assert tol([0.0, -0.0], [0.0, 0.0])[0]
    ok, worst = tol([0.0, 1e-300], [0.0, 0.0])
    assert not ok and worst == float("inf")


def test_tolerance_empty():
    assert tol([], []) == (True, 0.0)


def test_tolerance_catches_a_plausible_kernel_mistake():
    # A result that applies one scale block twice: D doubles on one entry.
    rng = np.random.default_rng(5)
    ref = rng.standard_normal(1000)
    d = ref.copy()
    d[17] *= 2.0
    ok, _ = tol(np.float64(np.float32(d)), ref)
    assert not ok or abs(ref[17]) < 1e-3 * np.abs(ref).max()


# ---- bf16_rne ---------------------------------------------------------------

def _all_bf16():
    """(value as Fraction, bit pattern) for every finite non-negative BF16,
    plus +Inf standing for 2^128 (the next value after the largest finite
    one, with an even pattern), sorted by value."""
    out = []
    for u in range(0x0000, 0x7F81):
        f = float(np.array([u << 16], np.uint32).view(np.float32)[0])
        out.append((Fraction(2) ** 128 if u == 0x7F80 else Fraction(f), u))
    return out


_TABLE = None


def _brute_bf16(x):
    """Nearest BF16 to the exact value of the double x, ties to the even
    pattern; magnitudes at or past the midpoint to 2^128 give Inf."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _all_bf16()
        _TABLE.sort()
    vals = [v for v, _ in _TABLE]
    fx = abs(Fraction(x))
    i = bisect.bisect_left(vals, fx)
    cands = [_TABLE[j] for j in (i - 1, i) if 0 <= j < len(_TABLE)]
    best = min(abs(v - fx) for v, _ in cands)
    near = [(v, u) for v, u in cands if abs(v - fx) == best]
    if len(near) > 1:
        near = [(v, u) for v, u in near if u % 2 == 0]
    u = near[0][1]
    return u | (0x8000 if math.copysign(1.0, x) < 0 else 0)


def _check(xs):
    got = oracle.bf16_rne(np.array(xs, np.float64))
    for x, g in zip(xs, got):
        assert int(g) == _brute_bf16(x), (x, hex(int(g)), hex(_brute_bf16(x)))


def test_bf16_rne_subnormal_range():
    t = 2.0 ** -133                       # spacing of BF16 subnormals
    xs = []
    for m in range(0, 128):
        xs += [m * t, (m + 0.5) * t, (m + 0.5) * t + t * 2.0 ** -20, (m + 0.5) * t - t * 2.0 ** -20,
               (m + 0.25) * t, (m + 0.75) * t]
    xs += [2.0 ** -134, 2.0 ** -134 * (1 + 2.0 ** -30), 2.0 ** -135, 2.0 ** -140, 5e-324]
    rng = np.random.default_rng(11)
    xs += list(rng.uniform(2.0 ** -133, 2.0 ** -126, 3000))
    xs += [-x for x in xs[::7]]
    _check(xs)
    # hand-checked values: 2^-134 is the tie between 0 and 2^-133 (even: 0);
    # anything above it rounds up to the smallest subnormal, pattern 0x0001;
    # 1.5 * 2^-133 is a tie between patterns 1 and 2 (even: 2)
    b = oracle.bf16_rne(np.array([2.0 ** -134, 2.0 ** -134 * (1 + 2.0 ** -30), 1.5 * t, 2.5 * t]))
    assert [int(v) for v in b] == [0x0000, 0x0001, 0x0002, 0x0002]


def test_bf16_rne_subnormal_to_normal_boundary():
    t = 2.0 ** -133
    # the largest subnormal is 127 * 2^-133 (pattern 0x007F), the smallest
    # normal 2^-126 = 128 * 2^-133 (0x0080); their midpoint ties to 0x0080
    b = oracle.bf16_rne(np.array([127 * t, 127.5 * t, 127.5 * t - t * 2.0 ** -20, 2.0 ** -126,
                                  2.0 ** -126 * (1 + 2.0 ** -8), 2.0 ** -126 * (1 + 3 * 2.0 ** -8)]))
    assert [int(v) for v in b] == [0x007F, 0x0080, 0x007F, 0x0080, 0x0080, 0x0082]
    _check([127 * t, 127.5 * t, 2.0 ** -126, 2.0 ** -126 * (1 + 2.0 ** -9)])


def test_bf16_rne_overflow_edge():
    big = 2.0 ** 127
    top = (2 - 2.0 ** -7) * big           # largest finite BF16, 0x7F7F
    mid = (2 - 2.0 ** -8) * big           # midpoint to 2^128: ties to even -> Inf
    b = oracle.bf16_rne(np.array([top, mid, mid - 2.0 ** 100, mid + 2.0 ** 100, -mid, -top,
                                  3.4e38, 1e39]))
    assert [int(v) for v in b] == [0x7F7F, 0x7F80, 0x7F7F, 0x7F80, 0xFF80, 0xFF7F, 0x7F80, 0x7F80]
    _check([top, mid, mid - 2.0 ** 100, (2 - 3 * 2.0 ** -8) * big, (2 - 5 * 2.0 ** -9) * big])


def test_bf16_rne_normal_range_sweep():
    rng = np.random.default_rng(12)
    xs = list(rng.standard_normal(2000) * np.exp2(rng.integers(-126, 127, 2000)))
    _check(xs)
