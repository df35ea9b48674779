"""Pins for the acceptance predicates in tests/checks.py (CPU only).

Every GPU parity test ends in within_tolerance / assert_close or
assert_bit_exact, so these predicates are checked against cases whose answer
is fixed by their definition (the Lecture 12 final-project page's verify
rule |got - ref| <= atol + rtol * |ref|, project_template.cu section 4, with
NaN and infinities failing): a flipped comparison, a dropped term or a NaN
that slips through fails one of them.
"""
import numpy as np
import pytest

from checks import ATOL, RTOL, assert_bit_exact, assert_close, within_tolerance


def test_defaults_are_the_pages_tolerances():
    assert ATOL == 1e-3 and RTOL == 1e-3


def test_boundary_of_the_absolute_term():
    ref = np.zeros(3)
    at = np.array([ATOL, -ATOL, 0.0])
    assert within_tolerance(at, ref)[0]
    above = np.array([np.nextafter(ATOL, np.inf), 0.0, 0.0])
    ok, worst, idx = within_tolerance(above, ref)
    assert not ok and idx == 0 and worst == above[0]


def test_boundary_of_the_relative_term():
    # powers of two keep every quantity exact: tol = 2^-10 + 2^-10 * 1 = 2^-9
    atol = rtol = 2.0 ** -10
    ref = np.array([1.0, -1.0], np.float32)
    edge = np.array([1.0 + 2.0 ** -9, -1.0 - 2.0 ** -9], np.float32)
    assert within_tolerance(edge, ref, atol, rtol)[0]
    for i in range(2):
        out = edge.copy()
        out[i] = np.nextafter(edge[i], np.float32(np.sign(edge[i]) * np.inf))
        ok, _, idx = within_tolerance(out, ref, atol, rtol)
        assert not ok and idx == i
    # the relative term uses |ref|, not ref: a negative reference widens it too
    assert within_tolerance(np.array([-3.0 - 0.0035]), np.array([-3.0]))[0]
    assert not within_tolerance(np.array([-3.0 - 0.0041]), np.array([-3.0]))[0]


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_results_fail(bad):
    ref = np.array([1.0, 2.0, 3.0], np.float32)
    got = ref.copy()
    got[1] = bad
    ok, _, idx = within_tolerance(got, ref)
    assert not ok and idx == 1
    with pytest.raises(AssertionError):
        assert_close(got, ref)
    # even where the reference itself is the same non-finite value
    ref2 = ref.copy()
    ref2[1] = bad
    assert not within_tolerance(got, ref2)[0]


def test_empty_arrays_pass_and_shapes_must_match():
    assert within_tolerance(np.zeros((0, 5)), np.zeros((0, 5)))[0]
    with pytest.raises(AssertionError):
        within_tolerance(np.zeros(3), np.zeros(4))


def test_bit_exact_compares_patterns():
    a = np.array([1.0, -2.5, 0.0], np.float32)
    assert_bit_exact(a.copy(), a)
    with pytest.raises(AssertionError):
        assert_bit_exact(np.array([1.0, -2.5, -0.0], np.float32), a)      # -0.0 is not +0.0
    with pytest.raises(AssertionError):
        b = a.copy()
        b[1] = np.nextafter(b[1], np.float32(0))                         # one ulp
        assert_bit_exact(b, a)
    nan = np.array([np.nan], np.float32)
    with pytest.raises(AssertionError):
        assert_bit_exact(nan, np.array([0.0], np.float32))
    with pytest.raises(AssertionError):
        assert_bit_exact(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32))
