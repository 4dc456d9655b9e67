"""Pins of the oracle's interpolation kernels (CPU only).

The pages fix the cubic kernel as Catmull-Rom with a = -0.5, C^1 and passing
through the control points, and give the tap counts (see
tests/golden/page_facts.json).  Keys' kernel with a = -0.5 is the textbook
kernel that reproduces polynomials up to degree 2; that property and the
closed-form values below would fail for any other a, a wrong branch or a
dropped term.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import CUBIC, LINEAR, kernel, kernel_deriv, tap_offsets

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def facts():
    with open(GOLD) as f:
        return json.load(f)


def test_tap_counts_match_pages():
    taps = facts()["taps_per_sample"]["value"]
    for interp, name in ((LINEAR, "linear"), (CUBIC, "cubic")):
        for ndim in (2, 3):
            n = len(list(itertools.product(tap_offsets(interp), repeat=ndim)))
            assert n == taps[f"{name}_{ndim}d"]


def _keys_exact(t: Fraction, a: Fraction) -> Fraction:
    t = abs(t)
    if t <= 1:
        return (a + 2) * t ** 3 - (a + 3) * t ** 2 + 1
    if t < 2:
        return a * t ** 3 - 5 * a * t ** 2 + 8 * a * t - 4 * a
    return Fraction(0)


def test_cubic_closed_form_values():
    a = Fraction(facts()["catmull_rom_a"]["value"]).limit_denominator(8)
    assert a == Fraction(-1, 2)
    # hand values of Keys' kernel at a = -1/2 (exact dyadic rationals)
    hand = {0: 1, Fraction(1, 4): Fraction(111, 128), Fraction(1, 2): Fraction(9, 16),
            Fraction(3, 4): Fraction(29, 128), 1: 0, Fraction(5, 4): Fraction(-9, 128),
            Fraction(3, 2): Fraction(-1, 16), Fraction(7, 4): Fraction(-3, 128), 2: 0,
            Fraction(5, 2): 0}
    for t, v in hand.items():
        assert _keys_exact(Fraction(t), a) == v
        assert kernel(CUBIC, float(t)) == pytest.approx(float(v), abs=1e-15)
        assert kernel(CUBIC, -float(t)) == pytest.approx(float(v), abs=1e-15)


def test_cubic_interpolates_control_points():
    # passes through the control points: K(0) = 1, K(+-1) = K(+-2) = 0
    assert kernel(CUBIC, 0.0) == 1.0
    for t in (-2.0, -1.0, 1.0, 2.0, 3.0):
        assert kernel(CUBIC, t) == 0.0


@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_partition_of_unity_and_polynomial_reproduction(interp, rng):
    f = rng.uniform(0, 1, 1000)
    offs = np.asarray(tap_offsets(interp), float)
    w = kernel(interp, f[:, None] - offs[None, :])
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)
    deg = 1 if interp == LINEAR else 2
    for m in range(deg + 1):
        np.testing.assert_allclose((w * offs[None, :] ** m).sum(1), f ** m, atol=1e-13)
    # the next degree is NOT reproduced (distinguishes a = -0.5 from others)
    err = np.abs((w * offs[None, :] ** (deg + 1)).sum(1) - f ** (deg + 1))
    assert err.max() > 1e-3


def test_other_a_breaks_quadratic_reproduction():
    # the a = -0.5 choice is what makes quadratics exact (textbook property)
    f = Fraction(1, 3)
    offs = [-1, 0, 1, 2]
    for a in (Fraction(-1, 2), Fraction(-3, 4), Fraction(-1, 4)):
        s = sum(_keys_exact(f - o, a) * o ** 2 for o in offs)
        assert (s == f ** 2) == (a == Fraction(-1, 2))


def test_cubic_derivative_matches_finite_difference(rng):
    u = rng.uniform(-2.5, 2.5, 2000)
    u = u[np.min(np.abs(np.abs(u)[:, None] - np.array([0, 1, 2])[None, :]), axis=1) > 1e-3]
    h = 1e-6
    fd = (kernel(CUBIC, u + h) - kernel(CUBIC, u - h)) / (2 * h)
    np.testing.assert_allclose(kernel_deriv(CUBIC, u), fd, atol=1e-7)


def test_cubic_is_c1():
    eps = 1e-9
    for t in (1.0, -1.0, 2.0, -2.0, 0.0):
        left = kernel_deriv(CUBIC, t - eps)
        right = kernel_deriv(CUBIC, t + eps)
        assert abs(left - right) < 1e-7
    # both branches give -0.5 * sign at |t| = 1
    assert kernel_deriv(CUBIC, 1.0) == pytest.approx(-0.5)
    assert kernel_deriv(CUBIC, -1.0) == pytest.approx(0.5)


def test_linear_derivative_is_right_derivative():
    assert kernel_deriv(LINEAR, 0.0) == -1.0     # right of the peak
    assert kernel_deriv(LINEAR, -1.0) == 1.0     # right of the left foot
    assert kernel_deriv(LINEAR, 1.0) == 0.0      # right of the right foot
    assert kernel_deriv(LINEAR, 0.5) == -1.0
    assert kernel_deriv(LINEAR, -0.5) == 1.0
