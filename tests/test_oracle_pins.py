"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test would fail for a plausible slip in the oracle: a dropped factor 2,
a wrong sign of the compensation, a transposed or lower/upper-swapped U, a
row of U read at the wrong index, the lazy update applied to the wrong
columns, a grid off by one level, a wrong rounding mode.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import gptq as og

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _spd_problem(d_out, d_in, n, seed, dead=()):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((d_in, n)) + 0.5 * rng.standard_normal((d_in, 3)) @ rng.standard_normal((3, n))
    for d in dead:
        X[d] = 0.0
    W = rng.standard_normal((d_out, d_in)) * 0.02
    return W, X


# ---------------------------------------------------------------------------
# P1: the worked two-weight example (aicassindra "A worked two-weight example")
# ---------------------------------------------------------------------------
def test_worked_example_golden():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    H = np.array(g["H"])
    w = np.array([g["w"]])
    U, dead, lam = oracle.prepare(H, lam=0.0)
    assert lam == 0.0 and not dead.any()
    step = g["grid_step"]
    trace = []
    r = oracle.quantize(w, U, bits=8, group_size=0, block_size=128,
                        fixed_grid=(np.array([step]), np.array([0.0])), trace=trace)
    # q1 = 0.5 on a grid of step 0.5
    assert r.w_hat[0, 0] == pytest.approx(g["q1"], abs=0)
    # delta1 = q1 - w1
    assert r.w_hat[0, 0] - w[0, 0] == pytest.approx(g["delta1"], abs=1e-15)
    # compensation moves w2 from 0.30 to 0.38 (delta2 = +0.08)
    assert trace[1][0] == pytest.approx(g["w2_after"], abs=1e-14)
    assert trace[1][0] - w[0, 1] == pytest.approx(g["delta2"], abs=1e-14)
    # output error delta H delta^T: 0.0576 without compensation ...
    d_nocomp = np.array([g["delta1"], 0.0])
    assert d_nocomp @ H @ d_nocomp == pytest.approx(g["error_no_compensation"], abs=1e-14)
    # ... 0.0384 with it; this equals the first scaled error E_1^2 = e_1^2/[H^-1]_11
    d_comp = np.array([g["delta1"], trace[1][0] - w[0, 1]])
    assert d_comp @ H @ d_comp == pytest.approx(g["error_with_compensation"], abs=1e-14)
    assert r.E[0, 0] ** 2 == pytest.approx(g["error_with_compensation"], abs=1e-14)
    red = 1 - g["error_with_compensation"] / g["error_no_compensation"]
    assert red == pytest.approx(g["reduction_fraction"], abs=0.005)


def test_two_by_two_factor_closed_form():
    # Cholesky of H^-1 for H = [[a, b], [b, c]] in closed form
    a, b, c = 4.0, 2.0, 3.0
    det = a * c - b * b
    hinv = np.array([[c, -b], [-b, a]]) / det
    u00 = np.sqrt(hinv[0, 0])
    u01 = hinv[0, 1] / u00
    u11 = np.sqrt(hinv[1, 1] - u01 ** 2)
    U = oracle.hinv_cholesky_upper(np.array([[a, b], [b, c]]))
    np.testing.assert_allclose(U, [[u00, u01], [0.0, u11]], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(U, [[0.6123724356957945, -0.408248290463863], [0, 0.5773502691896258]], rtol=1e-14)


# ---------------------------------------------------------------------------
# Hessian: the Kronecker structure (math4ai "GPTQ Hessian"), factor 2, layout
# ---------------------------------------------------------------------------
def test_kronecker_bruteforce_pins_factor_two_and_layout():
    rng = np.random.default_rng(3)
    d_out, d_in, n = 2, 3, 5
    X = rng.standard_normal((d_in, n))
    W = rng.standard_normal((d_out, d_in))

    def f(v):
        What = v.reshape(d_out, d_in)  # rows stacked one under another
        R = W @ X - What @ X
        return float(np.sum(R * R))

    m = d_out * d_in
    x0 = rng.standard_normal(m)
    h = 0.5
    Hb = np.zeros((m, m))
    for a in range(m):
        for b in range(m):
            ea = np.zeros(m); ea[a] = h
            eb = np.zeros(m); eb[b] = h
            Hb[a, b] = (f(x0 + ea + eb) - f(x0 + ea) - f(x0 + eb) + f(x0)) / (h * h)
    H = oracle.hessian([X])
    np.testing.assert_allclose(Hb, np.kron(np.eye(d_out), H), rtol=1e-9, atol=1e-9)


def test_hessian_chunks_and_one_hot():
    X = np.zeros((3, 4))
    X[1, 2] = 1.0
    H = oracle.hessian([X[:, :1], X[:, 1:]])
    expect = np.zeros((3, 3)); expect[1, 1] = 2.0
    np.testing.assert_array_equal(H, expect)
    assert np.all(oracle.hessian([], d_in=5) == 0)


# ---------------------------------------------------------------------------
# damping and dead channels (aicassindra "The Cholesky trick")
# ---------------------------------------------------------------------------
def test_damp_closed_form():
    H = np.diag([1.0, 2.0, 3.0, 0.0])
    H[0, 1] = H[1, 0] = 0.5
    Hd, dead, lam = oracle.damp(H, 0.01)
    assert lam == pytest.approx(0.01 * 6.0 / 4)
    assert dead.tolist() == [False, False, False, True]
    np.testing.assert_allclose(np.diag(Hd), [1.015, 2.015, 3.015, 1.015])
    assert Hd[0, 1] == 0.5 and Hd[1, 0] == 0.5


def test_non_pd_detection():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((12, 5))  # N < d_in: rank 5
    H = oracle.hessian([X])
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.prepare(H, lam=0.0)
    U, _, _ = oracle.prepare(H, 0.01)  # damping makes it well-posed
    assert np.all(np.isfinite(U))


def test_factor_properties_and_reverse_route():
    W, X = _spd_problem(4, 20, 60, 5)
    Hd, _, _ = oracle.damp(oracle.hessian([X]))
    U = oracle.hinv_cholesky_upper(Hd)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(20), atol=1e-10)
    # the device route: reverse-order Cholesky H = R R^T (R upper), U = R^-1
    J = np.eye(20)[::-1]
    Lt = np.linalg.cholesky(J @ Hd @ J)
    R = J @ Lt @ J
    np.testing.assert_allclose(R @ R.T, Hd, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(np.linalg.inv(R), U, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# grid and rounding (readings; hand-computed values)
# ---------------------------------------------------------------------------
def test_grid_hand_values():
    s, z = oracle.grid(F32(-0.3), F32(0.45), 4)
    assert s == F32(F32(F32(0.45) - F32(-0.3)) / F32(15))
    assert float(s) == pytest.approx(0.05, rel=1e-6)
    assert z == 6.0
    # all-zero range -> [-1, 1]: s = fl32(2/15) = 0.13333334 rounds up, so
    # fl32(1/s) = 7.4999995 and z = 7 (not 8)
    s, z = oracle.grid(F32(0), F32(0), 4)
    assert s == F32(F32(2) / F32(15)) and F32(F32(1) / s) == F32(7.4999995) and z == 7.0
    # positive-only: zero is the lower end
    s, z = oracle.grid(F32(0.2), F32(0.5), 4)
    assert z == 0.0 and s == F32(F32(0.5) / F32(15))
    # negative-only: zero is the upper end
    s, z = oracle.grid(F32(-0.6), F32(-0.1), 3)
    assert z == 7.0 and s == F32(F32(0.6) / F32(7))


def test_grid_covers_range_and_represents_zero():
    rng = np.random.default_rng(9)
    mn = -np.abs(rng.standard_normal(1000)).astype(F32)
    mx = np.abs(rng.standard_normal(1000)).astype(F32)
    for bits in (2, 3, 4, 8):
        s, z = oracle.grid(mn, mx, bits)
        maxq = 2 ** bits - 1
        lo = s.astype(np.float64) * (0 - z)
        hi = s.astype(np.float64) * (maxq - z)
        assert np.all(np.abs(lo - mn) <= s * 0.5 + 1e-7)
        assert np.all(np.abs(hi - mx) <= s * 0.5 + 1e-7)
        q, _ = oracle.quantize_values(np.zeros(1000), s, z, bits)
        assert np.all(q == z)


def test_rounding_half_to_even_and_clamp():
    s = np.array([1.0, 1.0, 1.0, 1.0, 0.5], F32)
    z = np.array([0.0, 0.0, 0.0, 0.0, 3.0], F32)
    q, v = oracle.quantize_values(np.array([2.5, 3.5, -4.0, 99.0, 0.25]), s, z, 4)
    assert q.tolist() == [2.0, 4.0, 0.0, 15.0, 4.0]
    assert v[-1] == F32(3.5)


# ---------------------------------------------------------------------------
# P2: the Cholesky-row update equals the explicit OBS update by re-inversion
# (aicassindra "Greedy quantization..."; mbrenndoerfer Schur complement)
# ---------------------------------------------------------------------------
def test_schur_complement_formula():
    W, X = _spd_problem(1, 9, 30, 2)
    Hd, _, _ = oracle.damp(oracle.hessian([X]))
    Hinv = np.linalg.inv(Hd)
    q = 0
    down = Hinv[1:, 1:] - np.outer(Hinv[1:, q], Hinv[q, 1:]) / Hinv[q, q]
    np.testing.assert_allclose(down, np.linalg.inv(Hd[1:, 1:]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("d_in,block", [(9, 1), (16, 4), (13, 16)])
def test_sweep_matches_explicit_obs_reinversion(d_in, block):
    W, X = _spd_problem(5, d_in, 40, 11 + d_in)
    Hd, _, _ = oracle.damp(oracle.hessian([X]))
    U = oracle.hinv_cholesky_upper(Hd)
    bits = 3
    r = oracle.quantize(W, U, bits, 0, block)
    s = r.scales[:, 0]
    z = r.zeros[:, 0].astype(F32)
    for row in range(W.shape[0]):
        w = W[row].astype(np.float64).copy()
        for q in range(d_in):
            Finv = np.linalg.inv(Hd[q:, q:])
            qv, _ = oracle.quantize_values(w[q:q + 1], s[row:row + 1], z[row:row + 1], bits)
            wq = float(s[row]) * (float(qv[0]) - float(z[row]))
            e = w[q] - wq
            # OBS: delta = -(e / [Hf^-1]_qq) [Hf^-1]_{:,q}
            w[q:] += -(e / Finv[0, 0]) * Finv[:, 0]
            assert w[q] == pytest.approx(wq, abs=1e-13)
            assert r.codes[row, q] == int(qv[0])
            assert r.E[row, q] == pytest.approx(e / np.sqrt(Finv[0, 0]), rel=1e-9, abs=1e-14)
        np.testing.assert_allclose(r.w_hat[row], w, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------
# P3: lazy batches are exact (aicassindra "GPTQ's speedups": same math)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("g", [0, 8, 16, 40])
def test_lazy_batch_invariance(g):
    W, X = _spd_problem(24, 240, 480, 21)
    U, dead, _ = oracle.prepare(oracle.hessian([X]))
    ref = oracle.quantize(W, U, 4, g, 1)
    for B in (3, 16, 24, 32, 48, 128, 200, 1000):
        r = oracle.quantize(W, U, 4, g, B)
        np.testing.assert_array_equal(r.codes, ref.codes)
        np.testing.assert_array_equal(r.scales, ref.scales)
        np.testing.assert_array_equal(r.zeros, ref.zeros)
        np.testing.assert_array_equal(r.minmax, ref.minmax)
        np.testing.assert_allclose(r.w_hat, ref.w_hat, rtol=0, atol=1e-14)
        np.testing.assert_allclose(r.E, ref.E, rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------------------
# P4: rows decouple (aicassindra objective; math4ai row split)
# ---------------------------------------------------------------------------
def test_row_decoupling_and_permutation():
    W, X = _spd_problem(40, 64, 200, 31)
    U, dead, _ = oracle.prepare(oracle.hessian([X]))
    for g in (0, 16):
        full = oracle.quantize(W, U, 4, g, 16)
        perm = np.random.default_rng(0).permutation(40)
        sub = perm[:7]
        r = oracle.quantize(W[sub], U, 4, g, 16)
        np.testing.assert_array_equal(r.codes, full.codes[sub])
        np.testing.assert_array_equal(r.scales, full.scales[sub])
        np.testing.assert_allclose(r.E, full.E[sub], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# P6: diagonal H -> no compensation -> plain round-to-nearest
# ---------------------------------------------------------------------------
def test_diagonal_hessian_reduces_to_rtn():
    rng = np.random.default_rng(4)
    d_in, n = 32, 64
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    X = (np.diag(rng.uniform(0.5, 2.0, d_in)) @ Q[:d_in])  # orthogonal rows
    H = oracle.hessian([X])
    assert np.max(np.abs(H - np.diag(np.diag(H)))) < 1e-12
    U, _, _ = oracle.prepare(H)
    W = rng.standard_normal((10, d_in)) * 0.02
    r = oracle.quantize(W, U, 4, 0, 8)
    # textbook RTN with the same grid: nearest of the 16 levels s (k - z)
    s = r.scales[:, :1].astype(np.float64)
    z = r.zeros[:, :1].astype(np.float64)
    levels = s * (np.arange(16)[None, :] - z)
    nearest = np.argmin(np.abs(W[:, :, None] - levels[:, None, :]), axis=2)
    np.testing.assert_array_equal(r.codes, nearest)


# ---------------------------------------------------------------------------
# P8: sum of squared scaled errors = tr(dW H dW^T), for any code choice
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("g,dead", [(0, ()), (16, ()), (0, (3, 17)), (8, (0, 40))])
def test_loss_identity(g, dead):
    W, X = _spd_problem(12, 48, 150, 41, dead=dead)
    H = oracle.hessian([X])
    Hd, dmask, lam = oracle.damp(H)
    U = oracle.hinv_cholesky_upper(Hd)
    r = oracle.quantize(W, U, 3, g, 16, dead=dmask)
    W0 = W.copy(); W0[:, dmask] = 0.0
    D = W0 - r.w_hat
    np.testing.assert_allclose(r.err_sq, np.einsum("ij,jk,ik->i", D, Hd, D), rtol=1e-9)
    # and in terms of the objective: sum E^2 = 2 ||dW X||^2 + lam ||dW||^2 (live part)
    out = oracle.output_error(W0, r.w_hat, [X])
    assert r.err_sq.sum() == pytest.approx(2 * out + lam * np.sum(D * D), rel=1e-9)
    # any code choice: replay on random neighbouring codes
    rng = np.random.default_rng(7)
    hint = np.clip(r.codes.astype(int) + rng.integers(-1, 2, r.codes.shape), 0, 7)
    r2 = oracle.quantize(W, U, 3, g, 16, dead=dmask, hint=hint)
    D2 = W0 - r2.w_hat
    np.testing.assert_allclose(r2.err_sq, np.einsum("ij,jk,ik->i", D2, Hd, D2), rtol=1e-9)


# ---------------------------------------------------------------------------
# P9: after each step the free weights are the constrained optimum
# ---------------------------------------------------------------------------
def test_per_step_optimality():
    W, X = _spd_problem(3, 20, 80, 51)
    Hd, _, _ = oracle.damp(oracle.hessian([X]))
    U = oracle.hinv_cholesky_upper(Hd)
    for B in (1, 6, 20):
        trace = []
        r = oracle.quantize(W, U, 3, 0, B, trace=trace)
        T = np.stack(trace, axis=1)  # [d_out, d_in] value of column j just before rounding
        for q in range(1, 20):
            Qi = np.arange(q)
            Fi = np.arange(q, 20)
            # argmin over w_F of (w - w0) H (w - w0)^T with w_Q fixed at What_Q
            dQ = r.w_hat[:, Qi] - W[:, Qi]
            wF = W[:, Fi] - np.linalg.solve(Hd[np.ix_(Fi, Fi)], Hd[np.ix_(Fi, Qi)] @ dQ.T).T
            np.testing.assert_allclose(T[:, q], wF[:, 0], rtol=1e-9, atol=1e-13)


# ---------------------------------------------------------------------------
# P10: dead channels are decoupled (aicassindra "simply skipped")
# ---------------------------------------------------------------------------
def test_dead_channel_removal_equivalence():
    dead_idx = (2, 9, 10)
    W, X = _spd_problem(8, 24, 100, 61, dead=dead_idx)
    W[:, list(dead_idx)] = 0.0  # keep the per-row grid identical in both problems
    H = oracle.hessian([X])
    Hd, dmask, lam = oracle.damp(H)
    assert set(np.nonzero(dmask)[0]) == set(dead_idx)
    r = oracle.quantize(W, oracle.hinv_cholesky_upper(Hd), 4, 0, 5, dead=dmask)
    live = np.setdiff1d(np.arange(24), dead_idx)
    Ur, _, _ = oracle.prepare(oracle.hessian([X[live]]), lam=lam)
    rr = oracle.quantize(W[:, live], Ur, 4, 0, 5)
    np.testing.assert_array_equal(r.codes[:, live], rr.codes)
    np.testing.assert_allclose(r.E[:, live], rr.E, rtol=1e-9, atol=1e-14)
    assert np.all(r.E[:, list(dead_idx)] == 0)
    assert np.all(r.codes[:, list(dead_idx)] == r.zeros[:, :1])


# ---------------------------------------------------------------------------
# group grids: rebuilt from the current weights at each group start
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d_in,g,B", [
    (32, 8, 16),    # groups start inside a block (g < B, g | B)
    (32, 8, 8),     # group starts are block starts (g = B)
    (48, 16, 4),    # a group spans several blocks (g > B, B | g)
    (36, 12, 8),    # unaligned: a group reaches past the block it starts in
    (30, 6, 1),     # unblocked
])
def test_group_grids_equal_explicit_obs_state(d_in, g, B):
    """At every group start the grid is built from the weights with every
    earlier column's compensation applied.  The reference state here comes
    from explicit OBS steps with the inverse of H restricted to the free
    columns, re-inverted at every step (no U, no lazy blocks), and the grid
    of that state must equal the oracle's bit for bit."""
    W, X = _spd_problem(5, d_in, 3 * d_in, 100 + d_in + g + B)
    Hd, _, _ = oracle.damp(oracle.hessian([X]))
    U = oracle.hinv_cholesky_upper(Hd)
    bits = 4
    r = oracle.quantize(W, U, bits, g, B)
    for row in range(W.shape[0]):
        w = W[row].astype(np.float64).copy()
        s = z = None
        for q in range(d_in):
            if q % g == 0:
                cols = w[q:q + g]
                mn, mx = F32(cols.min()), F32(cols.max())
                s1, z1 = oracle.grid(np.array([mn]), np.array([mx]), bits)
                s, z = s1[0], z1[0]
                k = q // g
                assert r.minmax[row, k, 0] == min(mn, F32(0)), (row, q)
                assert r.minmax[row, k, 1] == max(mx, F32(0)), (row, q)
                assert r.scales[row, k] == s and r.zeros[row, k] == int(z), (row, q)
            qv, _ = oracle.quantize_values(w[q:q + 1], np.array([s]), np.array([z]), bits)
            wq = float(s) * (float(qv[0]) - float(z))
            Finv = np.linalg.inv(Hd[q:, q:])
            w[q:] += -((w[q] - wq) / Finv[0, 0]) * Finv[:, 0]
            assert r.codes[row, q] == int(qv[0]), (row, q)
        np.testing.assert_allclose(r.w_hat[row], w, rtol=1e-10, atol=1e-13)


def test_group_grid_spanning_the_row_is_the_row_grid():
    W, X = _spd_problem(6, 32, 90, 71)
    U, _, _ = oracle.prepare(oracle.hessian([X]))
    r1 = oracle.quantize(W, U, 4, 32, 16)
    r0 = oracle.quantize(W, U, 4, 0, 16)
    np.testing.assert_array_equal(r1.scales, r0.scales)
    np.testing.assert_array_equal(r1.codes, r0.codes)


def test_dequantize_matches_sweep():
    W, X = _spd_problem(6, 32, 90, 81)
    U, _, _ = oracle.prepare(oracle.hessian([X]))
    for g in (0, 8):
        r = oracle.quantize(W, U, 4, g, 16)
        np.testing.assert_array_equal(oracle.dequantize(r.codes, r.scales, r.zeros, g), r.w_hat)


# ---------------------------------------------------------------------------
# tie-aware replay classifies an injected tie and an injected real flip
# ---------------------------------------------------------------------------
def test_tie_aware_replay():
    W, X = _spd_problem(64, 64, 200, 91)
    U, _, _ = oracle.prepare(oracle.hessian([X]))
    r = oracle.quantize(W, U, 4, 0, 16)
    same = oracle.quantize(W, U, 4, 0, 16, hint=r.codes)
    assert same.ties == 0 and same.hard == 0
    frac = np.abs(r.V - np.floor(r.V) - 0.5)  # distance to the nearest midpoint
    i, j = np.unravel_index(np.argmin(frac), frac.shape)
    hint = r.codes.copy()
    other = np.floor(r.V[i, j]) if r.codes[i, j] == np.floor(r.V[i, j]) + 1 else np.floor(r.V[i, j]) + 1
    hint[i, j] = int(other)
    t = oracle.quantize(W, U, 4, 0, 16, hint=hint, tie_tol=float(frac[i, j]) + 1e-9)
    assert t.ties == 1 and t.hard == 0
    i2, j2 = np.unravel_index(np.argmax(frac > 0.3), frac.shape)  # far from any midpoint
    hint2 = r.codes.copy()
    hint2[i2, j2] = (int(hint2[i2, j2]) + 1) % 16
    h = oracle.quantize(W, U, 4, 0, 16, hint=hint2)
    assert h.hard >= 1


# ---------------------------------------------------------------------------
# S1: few-bit storage.  The row's stream is the integer sum_j c_j 2^(bits j);
# its 32-bit limbs, least significant first, are the words (an independent
# definition through Python integers), and special widths reduce to byte and
# nibble layouts
# ---------------------------------------------------------------------------
def _limbs(row, bits, nw):
    v = 0
    for j, c in enumerate(row):
        v += int(c) << (bits * j)
    return [(v >> (32 * w)) & 0xFFFFFFFF for w in range(nw)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("d_in", [1, 7, 31, 32, 33, 100, 129])
def test_pack_codes_is_the_bit_stream(bits, d_in):
    rng = np.random.default_rng(bits * 1000 + d_in)
    codes = rng.integers(0, 1 << bits, (5, d_in)).astype(np.uint8)
    P = oracle.pack_codes(codes, bits)
    nw = (d_in * bits + 31) // 32
    assert P.shape == (5, nw) and P.dtype == np.uint32
    for r in range(5):
        assert [int(x) for x in P[r]] == _limbs(codes[r], bits, nw)
    np.testing.assert_array_equal(oracle.unpack_codes(P, bits, d_in), codes)


def test_pack_codes_worked_3bit():
    # 11 codes of 3 bits: 33 bits, two words; code 10 (= 0b011) puts its two
    # low bits in bits 30-31 of word 0 and a zero in bit 0 of word 1
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 3]], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.pack_codes(codes, 3), np.array([[0xD11F58D1, 0]], dtype=np.uint32))


def test_pack_codes_byte_and_nibble_layouts():
    rng = np.random.default_rng(5)
    c8 = rng.integers(0, 256, (3, 12)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.pack_codes(c8, 8), c8.view("<u4"))
    c4 = rng.integers(0, 16, (3, 16)).astype(np.uint8)
    nib = (c4[:, 0::2] | (c4[:, 1::2] << 4)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.pack_codes(c4, 4), nib.view("<u4"))


@pytest.mark.parametrize("g,dead", [(0, ()), (16, (3, 17))])
def test_output_error_from_errors(g, dead):
    W, X = _spd_problem(12, 48, 150, 43, dead=dead)
    H = oracle.hessian([X])
    Hd, dmask, lam = oracle.damp(H)
    U = oracle.hinv_cholesky_upper(Hd)
    r = oracle.quantize(W, U, 4, g, 16, dead=dmask)
    W0 = W.copy(); W0[:, dmask] = 0.0
    per_row = oracle.output_error_from_errors(r.err_sq, W0, r.w_hat, lam)
    direct = np.array([oracle.output_error(W0[i:i + 1], r.w_hat[i:i + 1], [X]) for i in range(W.shape[0])])
    np.testing.assert_allclose(per_row, direct, rtol=1e-9)


# ---------------------------------------------------------------------------
# G: the greedy-order variant (aicassindra "Greedy quantization with error
# compensation"; mbrenndoerfer "Mathematical Details of the Update")
# ---------------------------------------------------------------------------
def test_obq_worked_example_first_pick():
    # the page's example quantizes w_1 first; the greedy rule agrees (its
    # score e^2 / [H^-1]_11 is the page's compensated error 0.0384, against
    # 0.08 for w_2), and the compensation moves w_2 to the page's 0.38
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    H = np.array(g["H"])
    w = np.array([g["w"]])
    tr = []
    r = oracle.obq_quantize(w, np.linalg.inv(H), 4, fixed_grid=(np.array([g["grid_step"]]), np.array([0])),
                            trace=tr)
    _, q0, score0, w_after = tr[0]
    assert q0 == 0
    assert score0 == pytest.approx(g["error_with_compensation"], abs=1e-12)
    assert w_after[0] == pytest.approx(g["q1"], abs=1e-12)
    assert w_after[1] == pytest.approx(g["w2_after"], abs=1e-12)
    assert list(r.order[0]) == [0, 1]
    # both weights land on 0.5; the loss is dw H dw^T of the final error
    dw = w[0] - r.w_hat[0]
    assert r.loss[0] == pytest.approx(dw @ H @ dw, rel=1e-12)


def _greedy_by_direct_solves(w0, H, s, z, bits):
    """Greedy order by explicit re-optimization on H (no inverse, no Schur
    downdate): at each step every free weight is tried, the others free
    weights re-optimized by solving H_FF d_F = -H_Fq d_q, and the one with
    the smallest increase of d^T H d (from the current point) is fixed."""
    d_in = w0.size
    w = w0.astype(np.float64).copy()
    free = np.ones(d_in, bool)
    order, codes = [], np.zeros(d_in, np.int64)
    maxq = 2 ** bits - 1
    for _ in range(d_in):
        best = None
        for q in np.nonzero(free)[0]:
            v = np.float32(np.float32(np.float32(w[q]) / s) + z)
            c = float(np.clip(np.rint(v), 0, maxq))
            dq = s * (c - z) - w[q]                      # the move of w_q onto the grid
            F = free.copy()
            F[q] = False
            d = np.zeros(d_in)
            d[q] = dq
            if F.any():
                d[F] = np.linalg.solve(H[np.ix_(F, F)], -H[F, q] * dq)
            inc = d @ H @ d
            if best is None or inc < best[0] - 1e-15 * abs(best[0]):
                best = (inc, q, c, d)
        _, q, c, d = best
        w = w + d
        w[q] = s * (c - z)
        free[q] = False
        order.append(q)
        codes[q] = int(c)
    return np.array(order), codes


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_obq_matches_greedy_by_direct_solves(seed):
    rng = np.random.default_rng(100 + seed)
    d_in = 5
    A = rng.standard_normal((d_in, 3 * d_in))
    H = A @ A.T + 0.1 * np.eye(d_in)
    w = rng.standard_normal((1, d_in)) * 0.3
    s, z = og.grid(w.astype(F32).min(axis=1), w.astype(F32).max(axis=1), 3)
    r = oracle.obq_quantize(w, np.linalg.inv(H), 3)
    order, codes = _greedy_by_direct_solves(w[0], H, float(s[0]), float(z[0]), 3)
    assert list(r.order[0]) == list(order)
    assert list(r.codes[0]) == list(codes)


@pytest.mark.parametrize("dead", [(), (2, 9)])
def test_obq_fixed_order_is_the_sweep(dead):
    # the fixed left-to-right order with the Schur downdate equals the
    # Cholesky-row sweep, and the pick scores sum to its sum of squared
    # scaled errors
    W, X = _spd_problem(6, 24, 200, 7, dead)
    H = oracle.hessian([X])
    U, dm, lam = oracle.prepare(H)
    Hd, dm2, _ = oracle.damp(H)
    r = oracle.obq_quantize(W, np.linalg.inv(Hd), 4, dead=dm, fixed_order=True)
    g = oracle.quantize(W, U, 4, 0, 8, dead=dm)
    assert np.array_equal(r.codes, g.codes)
    np.testing.assert_allclose(r.w_hat, g.w_hat, rtol=0, atol=1e-15)
    np.testing.assert_allclose(r.loss, g.err_sq, rtol=1e-9)


@pytest.mark.parametrize("dead", [(), (1, 5)])
def test_obq_loss_identity(dead):
    W, X = _spd_problem(5, 16, 120, 11, dead)
    H = oracle.hessian([X])
    Hd, dm, lam = oracle.damp(H)
    r = oracle.obq_quantize(W, np.linalg.inv(Hd), 3, dead=dm)
    W0 = W.copy()
    W0[:, dm] = 0.0
    D = W0 - r.w_hat
    np.testing.assert_allclose(r.loss, np.einsum("ri,ij,rj->r", D, Hd, D), rtol=1e-9)
    # every row's order is a permutation, and each code is the rounding of
    # the weight as it stood when it was picked (checked by the grid values)
    for row in r.order:
        assert sorted(row) == list(range(16))
    assert np.all(r.codes <= 7)


def test_obq_diagonal_h_is_round_to_nearest():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((4, 12)) * 0.05
    Hinv = np.diag(1.0 / rng.uniform(0.5, 2.0, 12))
    r = oracle.obq_quantize(W, Hinv, 4)
    s, z = og.grid(W.astype(F32).min(axis=1), W.astype(F32).max(axis=1), 4)
    q, _ = og.quantize_values(W, s[:, None], z[:, None], 4)
    assert np.array_equal(r.codes, q.astype(np.uint8))


def test_obq_replay_counts():
    W, X = _spd_problem(3, 10, 80, 13)
    Hd, dm, lam = oracle.damp(oracle.hessian([X]))
    Hinv = np.linalg.inv(Hd)
    r = oracle.obq_quantize(W, Hinv, 4)
    same = oracle.obq_quantize(W, Hinv, 4, order_hint=r.order, code_hint=r.codes)
    assert same.ties == 0 and same.hard == 0 and np.array_equal(same.codes, r.codes)
    bad = r.order.copy()
    bad[0, [0, -1]] = bad[0, [-1, 0]]  # the last pick first: not a near-tie
    rep = oracle.obq_quantize(W, Hinv, 4, order_hint=bad)
    assert rep.hard >= 1 and list(rep.order[0]) == list(bad[0][:1]) + list(rep.order[0][1:])


# ---------------------------------------------------------------------------
# Propagation to the next layer (Y = act(What X))
# ---------------------------------------------------------------------------
def test_propagate_permutation_selects_rows():
    """A permutation matrix as What picks rows of X exactly (a transposed
    operand would pick by the inverse permutation)."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((7, 11))
    perm = np.array([3, 0, 6, 1, 5, 2, 4])
    P = np.zeros((7, 7))
    P[np.arange(7), perm] = 1.0
    Y = oracle.propagate(P, X)
    np.testing.assert_array_equal(Y, X[perm])
    inv = np.argsort(perm)
    assert not np.array_equal(Y, X[inv])


def test_propagate_relu_signs_and_scaling():
    X = np.array([[1.0, -2.0, 3.0], [0.5, 0.5, -4.0]])
    W = np.array([[1.0, 0.0], [0.0, -1.0], [2.0, 1.0]])
    Y = oracle.propagate(W, X, "relu")
    np.testing.assert_array_equal(Y, [[1.0, 0.0, 3.0], [0.0, 0.0, 4.0], [2.5, 0.0, 2.0]])
    np.testing.assert_array_equal(oracle.propagate(3.0 * W, X, "relu"), 3.0 * Y)  # positive homogeneity
    with pytest.raises(ValueError):
        oracle.propagate(W, X, "tanh")


def test_propagate_chain_with_identity_layers():
    """Two identity layers hand X through unchanged; a layer of ones sums
    the channels token by token."""
    rng = np.random.default_rng(6)
    X = rng.standard_normal((5, 9))
    np.testing.assert_array_equal(oracle.propagate(np.eye(5), oracle.propagate(np.eye(5), X)), X)
    np.testing.assert_allclose(oracle.propagate(np.ones((1, 5)), X)[0], X.sum(axis=0), rtol=1e-15)
