"""Acceptance predicates shared by the GPU parity tests.

Tolerance (the Lecture 12 project_template.cu ``verify`` rule, with the
tolerances it defaults to): |got - ref| <= 1e-3 + 1e-3 * |ref| per element,
evaluated in binary64.  Unlike the page's check, a NaN or infinite GPU value
fails (the comparison is written so that NaN is never <= tol).
Bit-exact: identical binary32 patterns.
"""
import numpy as np

ATOL = 1e-3
RTOL = 1e-3


def within_tolerance(got, ref, atol=ATOL, rtol=RTOL):
    """(ok, worst_abs, worst_index) for the per-element tolerance rule."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    assert g.shape == r.shape
    if g.size == 0:
        return True, 0.0, -1
    with np.errstate(invalid="ignore"):         # inf - inf is NaN, and fails below
        diff = np.abs(g - r)
        ok = diff <= atol + rtol * np.abs(r)    # NaN -> False
    ok &= np.isfinite(g)
    worst = int(np.argmax(np.where(np.isnan(diff), np.inf, diff)))
    return bool(ok.all()), float(diff[worst]), worst


def assert_close(got, ref, what=""):
    ok, worst, idx = within_tolerance(got, ref)
    assert ok, f"{what}: tolerance exceeded, max |err| {worst:.3e} at flat index {idx}"


def assert_bit_exact(got, ref, what=""):
    g = np.ascontiguousarray(got, dtype=np.float32).view(np.uint32)
    r = np.ascontiguousarray(ref, dtype=np.float32).view(np.uint32)
    assert g.shape == r.shape, what
    bad = np.flatnonzero(g.ravel() != r.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} elements differ; first at flat index {bad[0]}: "
                           f"got {np.float32(got.ravel()[bad[0]])!r} want {np.float32(ref.ravel()[bad[0]])!r}")
