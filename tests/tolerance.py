"""The parity bar used by every floating-point comparison.

The Q4_K page's test plan asks for parity "within 1e-4 relative tolerance"
against the gold reference without defining the term.  A pure elementwise
relative test fails near-zero outputs even for a perfect fp32 kernel (the
absolute error of a K-term fp32 dot is about eps * sqrt(K) * rms, which can
exceed 1e-4 * |y| when |y| is small), so the bar is read as

    |y_i - ref_i| <= 1e-4 * |ref_i| + 1e-4 * rms(ref)

elementwise, rms taken over the outputs of one call (or one token row).
"""
import numpy as np

REL = 1e-4


def rms(a):
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def parity_report(y, ref, rel=REL):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(y - ref)
    bound = rel * np.abs(ref) + rel * rms(ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        relerr = np.where(ref != 0, err / np.abs(ref), np.where(err == 0, 0, np.inf))
    nrm = float(np.linalg.norm(ref))
    return {
        "n": int(y.size),
        "fail": int(np.count_nonzero(~(err <= bound))),
        "max_abs_err": float(err.max()) if y.size else 0.0,
        "max_rel_err": float(relerr.max()) if y.size else 0.0,
        "normwise": float(np.linalg.norm(y - ref) / nrm) if nrm > 0 else float(np.linalg.norm(y - ref)),
        "pure_rel_fail": int(np.count_nonzero(relerr > rel)),
    }


def assert_parity(y, ref, rel=REL, rowwise=False, what=""):
    """Assert the bar above; rowwise applies it per row of a 2-D result."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    rows = [(y, ref)] if not rowwise else list(zip(y, ref))
    for i, (a, b) in enumerate(rows):
        rep = parity_report(a, b, rel)
        assert rep["fail"] == 0, f"{what} row {i}: {rep}"
        assert np.all(np.isfinite(a)), f"{what} row {i}: non-finite output"
