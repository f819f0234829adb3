"""Helpers for the GPU parity tests: tolerances, comparisons, progress lines."""

import sys

import numpy as np

# Tolerances against the fp64 oracle for bf16 inputs: max |dO| <= 2e-2, max |dLSE| <= 1e-3
# (natural log).
TOL_O = 2e-2
TOL_LSE = 1e-3
# fp32 inputs (the fp32 path: fp32 products and sums, accurate exp and log). A score
# s = scale * q.k over D <= 128 terms of unit-variance values carries at most about
# D * 2^-24 * |q||k| * scale ~ 1e-4 of rounding in the worst case (|q||k| ~ D), typically
# ~1e-6; the row sums of <= ~1000 terms add a relative ~1e-4 worst case. The bar sits at
# the worst case, two orders of magnitude above the typical error, so a regression of the
# fp32 path that the bf16 bar would hide still fails.
TOL_O_F32 = 1e-4
TOL_LSE_F32 = 1e-4


def tol(dtype, D=128):
    """(output bar, LSE bar) of a step for an input dtype name ("bf16" or "fp32") and head dim.
    bf16 with head_dim 64 runs on the fp32 vector kernel, like fp32 inputs: its bf16 inputs are
    exact in fp32 and no probability is rounded to bf16, so it is held to the fp32 bar."""
    return (TOL_O_F32, TOL_LSE_F32) if dtype == "fp32" or D == 64 else (TOL_O, TOL_LSE)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().double().numpy() if hasattr(t, "detach") else np.asarray(t, dtype=np.float64)


def max_err(got, want):
    """Max abs difference; -inf must match -inf exactly (returns inf otherwise)."""
    got = to_np(got)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    fin = np.isfinite(want)
    if not np.array_equal(np.isfinite(got), fin) or not np.array_equal(got[~fin], want[~fin]):
        return float("inf")
    if not fin.any():
        return 0.0
    return float(np.abs(got[fin] - want[fin]).max())


def check(name, o, lse, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE, quiet=False):
    eo = max_err(o, o_ref)
    el = max_err(lse, lse_ref) if lse is not None else 0.0
    if not quiet:
        say(f"  {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= tol_o, f"{name}: output error {eo} > {tol_o}"
    assert el <= tol_lse, f"{name}: LSE error {el} > {tol_lse}"
    return eo, el
