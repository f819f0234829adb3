"""Helpers for the GPU parity tests: tolerances, comparisons, progress lines."""

import sys

import numpy as np

# Tolerances against the fp64 oracle for bf16 inputs (and used for fp32 too):
# max |dO| <= 2e-2, max |dLSE| <= 1e-3 (natural log).
TOL_O = 2e-2
TOL_LSE = 1e-3


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


def check(name, o, lse, o_ref, lse_ref, tol_o=TOL_O, tol_lse=TOL_LSE):
    eo = max_err(o, o_ref)
    el = max_err(lse, lse_ref) if lse is not None else 0.0
    say(f"  {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= tol_o, f"{name}: output error {eo} > {tol_o}"
    assert el <= tol_lse, f"{name}: LSE error {el} > {tol_lse}"
    return eo, el
