"""Test-side parity helpers: compare the HIP path with the fp64 oracle.

Tolerances (stated once, used by every parity test):
  H      relative Frobenius error on the lower triangle <= 1e-5
  U      relative Frobenius error (upper triangle), oracle fed the device H <= 1e-4
  codes  tie-aware replay of the oracle on the device codes: no hard
         mismatch; ties (neighbouring code, pre-round value within 1e-4 grid
         units of the midpoint) in at most 0.01% of entries
  grid   per-row scales/zeros bit-exact; group grids: the grid formula on the
         device's own (min, max) reproduces its scales/zeros bit-exactly and
         the (min, max) agree with the replay's to 1e-5 of the range
  error  ||W X - What X||^2 within 0.5% of the oracle's own end-to-end value
"""
from __future__ import annotations

import numpy as np

import oracle

H_TOL = 1e-5
U_TOL = 1e-4
TIE_TOL = 1e-4
TIE_FRAC = 1e-4
OUT_TOL = 5e-3


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def lower(a):
    return np.tril(np.asarray(a, np.float64))


def check_h(H_dev: np.ndarray, H_ref: np.ndarray):
    e = rel_fro(lower(H_dev), lower(H_ref))
    assert e <= H_TOL, f"H rel err {e:.3g}"
    return e


def check_u(U_dev: np.ndarray, H_dev: np.ndarray, damp: float):
    """Stage-isolated: the oracle factors the device's own H."""
    Hs = lower(H_dev)
    Hs = Hs + np.tril(Hs, -1).T
    U_ref, dead_ref, lam_ref = oracle.prepare(Hs, damp)
    e = rel_fro(np.triu(U_dev), U_ref)
    assert np.all(np.tril(U_dev, -1) == 0)
    assert e <= U_TOL, f"U rel err {e:.3g}"
    return e, U_ref, dead_ref, lam_ref


def check_u_ref(U_dev: np.ndarray, U_ref: np.ndarray):
    """U against an oracle factor already computed from the device's H."""
    e = rel_fro(np.triu(U_dev), U_ref)
    assert np.all(np.tril(U_dev, -1) == 0)
    assert e <= U_TOL, f"U rel err {e:.3g}"
    return e


def check_codes(W, U_dev, dead, q, bits, group, block, rows=None):
    """Tie-aware replay on (a sample of) rows; returns the replay result."""
    codes = q["codes"]
    if rows is not None:
        W = W[rows]
        codes = codes[rows]
        q = {k: (v[rows] if hasattr(v, "shape") and v.shape[:1] == (q["codes"].shape[0],) else v)
             for k, v in q.items()}
    r = oracle.quantize(W, np.asarray(U_dev, np.float64), bits, group, block, dead=dead, hint=codes,
                        tie_tol=TIE_TOL)
    n = codes.size
    assert r.hard == 0, f"{r.hard} hard code mismatches (ties {r.ties})"
    assert r.ties <= TIE_FRAC * n, f"{r.ties} ties of {n}"
    assert r.max_tie_dist <= TIE_TOL
    if group == 0:
        np.testing.assert_array_equal(q["scales"], r.scales)
        np.testing.assert_array_equal(q["zeros"], r.zeros)
    else:
        mm = q["minmax"]
        s, z = oracle.grid(mm[..., 0], mm[..., 1], bits)
        np.testing.assert_array_equal(q["scales"], s)
        np.testing.assert_array_equal(q["zeros"], z.astype(np.int32))
        rng = np.maximum(r.minmax[..., 1] - r.minmax[..., 0], 1e-30)
        dev = np.abs(mm - r.minmax).max(axis=-1) / rng
        assert dev.max() <= 1e-5, f"group range deviation {dev.max():.3g}"
        zmis = np.mean(q["zeros"] != r.zeros)
        assert zmis <= 1e-4, f"zero-point mismatch fraction {zmis:.3g}"
    err = np.asarray(q["err_row"], np.float64)
    np.testing.assert_allclose(err, r.err_sq, rtol=2e-3, atol=1e-12)
    return r


def output_errors(W, codes, scales, zeros, group, x_chunks, W_hat_ref):
    """(device, oracle) values of ||W X - What X||^2."""
    chunks = list(x_chunks)
    What = oracle.dequantize(codes, scales, zeros, group)
    e_dev = oracle.output_error(W, What, chunks)
    e_ref = oracle.output_error(W, W_hat_ref, chunks)
    return e_dev, e_ref
