"""Comparison helpers and tolerances for HIP-vs-oracle parity tests.

Tolerances (fixed before any kernel ran, from the accumulation arithmetic):
  fp32 inputs, fp32 accumulation:             O and LSE max-abs <= 1e-4
  bf16 inputs, fp32 accumulation, bf16 P/O:   O max-abs <= 2e-2, mean-abs <= 2e-3,
                                              LSE max-abs <= 1e-3 (finite rows)
  gradients (bf16 outputs, fp32 accumulation): max-abs <= 5e-2
Rows the oracle gives LSE = -inf must be -inf on the device too, with O = 0.

The gradient bound of 5e-2 is for inputs of the pages' N(0, 1) workloads.
Tests that scale inputs far beyond them (large-logit cases) get a bound that
grows with the gradient's magnitude: rounding a gradient of size g to bf16
alone costs up to g * 2^-8, which passes 5e-2 once g > 12.8, so those tests
allow four such half-ulps of the largest reference magnitude.

Relative error ("Modern attention kernels", "Numerical validation": absolute
and relative tolerances tied to the output precision).  Every comparison also
computes max-rel = max |x - y| / |y| over the elements with |y| > 1e-2 and
logs it with the absolute figures (printed, and collected in ``LOG`` for the
session summary that ``conftest.py`` writes when ETA_PARITY_LOG names a
file).  It is logged, not bounded on its own: the error of a bf16 output
element is set by the probabilities' rounding times the magnitudes of the
values summed, not by the element's own size, so near-cancelling elements
carry large relative errors at the same absolute error; the absolute bound
already holds the relative error of an element of size |y| to bound / |y|.
"""

import os

import numpy as np

TOL_F32 = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3
TOL_LSE_BF16 = 1e-3
TOL_GRAD = 5e-2
REL_FLOOR = 1e-2

# One record per comparison: test id, quantity, element count, max-abs,
# mean-abs, max-rel (|ref| > REL_FLOOR) and the bound that was applied.
LOG = []


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _record(what, err, ref, bound):
    big = np.abs(ref) > REL_FLOOR
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    rec = {
        "test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
        "what": what,
        "n": int(err.size),
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "max_rel": max_rel,
        "bound": bound,
    }
    LOG.append(rec)
    print(f"parity {what}: n={rec['n']} max-abs {rec['max_abs']:.3e} "
          f"mean-abs {rec['mean_abs']:.3e} max-rel(|ref|>{REL_FLOOR:g}) {max_rel:.3e}")
    return rec


def check_out(dev, ref, dtype, what="O"):
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert dev.shape == ref.shape, (what, dev.shape, ref.shape)
    assert np.all(np.isfinite(dev)), f"{what}: non-finite values on the device"
    err = np.abs(dev - ref)
    if err.size == 0:
        return 0.0
    if dtype == "f32":
        _record(what, err, ref, TOL_F32)
        assert err.max() <= TOL_F32, f"{what}: max-abs {err.max():.3e} > {TOL_F32}"
    else:
        _record(what, err, ref, TOL_BF16_MAX)
        assert err.max() <= TOL_BF16_MAX, f"{what}: max-abs {err.max():.3e} > {TOL_BF16_MAX}"
        assert err.mean() <= TOL_BF16_MEAN, f"{what}: mean-abs {err.mean():.3e} > {TOL_BF16_MEAN}"
    return float(err.max())


def check_lse(dev, ref, dtype, what="LSE"):
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(dev), ninf), f"{what}: -inf rows differ"
    if (~ninf).any():
        err = np.abs(dev[~ninf] - ref[~ninf])
        tol = TOL_F32 if dtype == "f32" else TOL_LSE_BF16
        _record(what, err, ref[~ninf], tol)
        assert err.max() <= tol, f"{what}: max-abs {err.max():.3e} > {tol}"
        return float(err.max())
    return 0.0


def check_grad(dev, ref, what, magnitude_aware=False):
    dev = np.asarray(dev, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(dev)), f"{what}: non-finite values on the device"
    err = np.abs(dev - ref)
    tol = TOL_GRAD
    if magnitude_aware:
        tol = max(TOL_GRAD, 4.0 * 2.0 ** -8 * float(np.abs(ref).max()))
    _record(what, err, ref, tol)
    assert err.max() <= tol, f"{what}: max-abs {err.max():.3e} > {tol:.3e}"
    return float(err.max())
