"""Plain fp64 CPU oracle of the GPTQ per-layer path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares no code with the HIP
library and imports nothing from it; the product path never calls it.

Every step follows the pages, in their order and notation:

* objective ``argmin_What ||W X - What X||^2`` with ``W: [d_row, d_col]``,
  ``X: [d_col, N]``; rows decouple and all share one Hessian
  (aicassindra.com "tm_gptq_math", "The reconstruction objective, written
  out"; math4ai "GPTQ Hessian", row-split paragraph);
* ``H = 2 X X^T`` (aicassindra "Why it is second-order: the Hessian");
* damping ``H <- H + lambda I``, lambda = 1% of the mean diagonal, and
  zero-diagonal (dead) channels skipped (aicassindra "The Cholesky trick for
  the inverse Hessian"; math4ai damping sentence);
* ``U`` = upper Cholesky factor of ``H^-1`` (``H^-1 = U^T U``) computed once by
  a stable library routine (math4ai column-sweep paragraph; aicassindra "The
  Cholesky trick"; mbrenndoerfer "Mathematical Details of the Update",
  Cholesky paragraph);
* fixed left-to-right column order shared by all rows, with the OBS
  compensation ``delta = -(e_q / [H^-1]_qq) H^-1[:, q]`` read off row q of U,
  done immediately inside a block of B columns and lazily for the columns
  after the block (aicassindra "Greedy quantization with error compensation"
  and "GPTQ's speedups: fixed order and lazy batches").

Readings of passages the pages leave open (the grid form, rounding, clamping,
the precision of the rounding decision, dead-channel handling) are stated on
the function that applies them.

The greedy-order variant the fixed order replaces (``obq_quantize``: per
row, quantize next the weight with the smallest ``e_q^2 / [H^-1]_qq``,
compensate, and downdate the inverse by the Schur complement; aicassindra
"Greedy quantization with error compensation", mbrenndoerfer "Mathematical
Details of the Update") is here too, as the check of the device's variant.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(worked example, Schur re-inversion, lazy-batch invariance, row decoupling,
Kronecker brute force, diagonal-H reduction to round-to-nearest, the
loss identity, per-step optimality, dead-channel removal, non-PD detection;
for the greedy variant: the worked example's first pick and score, fixed
order equal to the sweep, brute-force re-optimization scores, the loss
identity).
"""
from __future__ import annotations

import dataclasses
from typing import Iterable, Optional, Tuple

import numpy as np
import scipy.linalg

F32 = np.float32


class NotPositiveDefinite(ValueError):
    """Raised when the damped Hessian has no Cholesky factor."""


# ----------------------------------------------------------------------------
# Stage 1: Hessian
# ----------------------------------------------------------------------------
def hessian(x_chunks: Iterable[np.ndarray], d_in: Optional[int] = None) -> np.ndarray:
    """``H = 2 X X^T`` in fp64, summed over token chunks of ``X: [d_in, n]``.

    aicassindra "Why it is second-order: the Hessian" gives H = 2 X X^T with
    H of size d_col x d_col; the sum over tokens is split into chunks only
    because X need not fit in memory (X X^T = sum_c X_c X_c^T).  No 1/N
    normalisation: the pages write none.
    """
    H = None
    for xc in x_chunks:
        xc = np.asarray(xc, dtype=np.float64)
        if H is None:
            H = np.zeros((xc.shape[0], xc.shape[0]))
        H += 2.0 * (xc @ xc.T)
    if H is None:
        if d_in is None:
            raise ValueError("no chunks")
        H = np.zeros((d_in, d_in))
    return H


# ----------------------------------------------------------------------------
# Stage 2: damping and dead channels
# ----------------------------------------------------------------------------
def damp(H: np.ndarray, damp_frac: float = 0.01, lam: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray, float]:
    """Damped copy of H, the dead-channel mask and lambda.

    aicassindra "The Cholesky trick": H <- H + lambda I with lambda around 1%
    of the mean diagonal; columns with a zero diagonal are simply skipped.
    Readings: the mean runs over all d_in diagonal entries of the undamped H
    (dead ones count as 0); a dead channel gets H_dd = 1 before the common
    lambda is added (any positive value decouples it: its row and column of
    H are exactly zero); ``lam`` overrides the computed lambda.
    """
    H = np.array(H, dtype=np.float64, copy=True)
    diag = np.diag(H).copy()
    dead = diag == 0.0
    if lam is None:
        lam = float(damp_frac) * float(np.mean(diag)) if diag.size else 0.0
    idx = np.arange(H.shape[0])
    H[idx[dead], idx[dead]] = 1.0
    H[idx, idx] += lam
    return H, dead, float(lam)


# ----------------------------------------------------------------------------
# Stage 3: U = upper Cholesky factor of H^-1
# ----------------------------------------------------------------------------
def hinv_cholesky_upper(Hd: np.ndarray) -> np.ndarray:
    """``U`` upper triangular with ``H^-1 = U^T U``.

    Literally as math4ai "GPTQ Hessian" (column-sweep paragraph) and
    aicassindra "The Cholesky trick" state it: invert H with a stable library
    routine (LAPACK Cholesky solve) and take the Cholesky factor of the
    inverse.  A non-positive-definite H raises ``NotPositiveDefinite``; there
    is no retry with more damping.
    """
    n = Hd.shape[0]
    if n == 0:
        return np.zeros((0, 0))
    try:
        c = scipy.linalg.cho_factor(Hd, lower=True, check_finite=True)
        Hinv = scipy.linalg.cho_solve(c, np.eye(n))
        Hinv = 0.5 * (Hinv + Hinv.T)
        L = np.linalg.cholesky(Hinv)
    except (np.linalg.LinAlgError, scipy.linalg.LinAlgError) as exc:
        raise NotPositiveDefinite(str(exc)) from exc
    return np.ascontiguousarray(L.T)


def prepare(H: np.ndarray, damp_frac: float = 0.01, lam: Optional[float] = None):
    """Stages 2 and 3 together: returns ``(U, dead, lam)``."""
    Hd, dead, lam = damp(H, damp_frac, lam)
    return hinv_cholesky_upper(Hd), dead, lam


# ----------------------------------------------------------------------------
# Stage 4: quantization grid
# ----------------------------------------------------------------------------
def grid(mn, mx, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Asymmetric min-max grid of ``2^bits`` levels (fp32 op sequence).

    The pages fix only that weights go to a few-bit integer grid (aicassindra
    "Post-training quantization ..." 16-bit floats to 4-bit integers; the
    worked example's grid of step 0.5).  Reading: the grid spans
    [min(0, min w), max(0, max w)]; an all-zero range becomes [-1, 1];
    ``s = fl32(fl32(mx - mn) / maxq)``, ``z = clamp(rint(fl32(-mn / s)), 0,
    maxq)`` with ``maxq = 2^bits - 1``, every operation an IEEE fp32 one, so
    that the per-row scale is a fixed function of the fp32 inputs.
    """
    mn = np.minimum(np.asarray(mn, dtype=F32), F32(0))
    mx = np.maximum(np.asarray(mx, dtype=F32), F32(0))
    both0 = (mn == 0) & (mx == 0)
    mn = np.where(both0, F32(-1), mn).astype(F32)
    mx = np.where(both0, F32(1), mx).astype(F32)
    maxq = F32(2 ** bits - 1)
    s = ((mx - mn).astype(F32) / maxq).astype(F32)
    z = np.rint((-mn / s).astype(F32)).astype(F32)
    z = np.clip(z, F32(0), maxq).astype(F32)
    return s, z


def quantize_values(w: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int) -> Tuple[np.ndarray, np.ndarray]:
    """Round to the nearest grid point: returns ``(q, v)``.

    ``v = fl32(fl32(w / s) + z)`` is the position on the grid in grid units
    and ``q = clamp(rint(v), 0, maxq)``.  Reading: the rounding decision is
    taken in IEEE fp32 (the precision of the device kernel), with
    round-half-to-even; a value outside the grid is clamped to its end code
    and its full error is still compensated.
    """
    w32 = np.asarray(w).astype(F32)
    v = ((w32 / s).astype(F32) + z).astype(F32)
    q = np.clip(np.rint(v), F32(0), F32(2 ** bits - 1)).astype(F32)
    return q, v


# ----------------------------------------------------------------------------
# Stage 4: the column sweep
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class QuantResult:
    codes: np.ndarray       # [d_out, d_in] uint8
    scales: np.ndarray      # [d_out, n_groups] float32
    zeros: np.ndarray       # [d_out, n_groups] int32
    minmax: np.ndarray      # [d_out, n_groups, 2] float32 (the range each grid was built from)
    E: np.ndarray           # [d_out, d_in] fp64 scaled errors e_j / U_jj
    V: np.ndarray           # [d_out, d_in] float32 pre-round grid positions
    w_hat: np.ndarray       # [d_out, d_in] fp64 dequantised weights s (q - z)
    err_sq: np.ndarray      # [d_out] fp64 sum_j E_j^2 per row
    ties: int = 0
    hard: int = 0
    max_tie_dist: float = 0.0
    mismatch_rows: Optional[np.ndarray] = None


def quantize(W: np.ndarray, U: np.ndarray, bits: int, group_size: int = 0, block_size: int = 128,
             dead: Optional[np.ndarray] = None, hint: Optional[np.ndarray] = None, tie_tol: float = 1e-4,
             fixed_grid: Optional[Tuple[np.ndarray, np.ndarray]] = None,
             trace: Optional[list] = None) -> QuantResult:
    """Fixed-order, block-lazy quantize-and-compensate sweep of one layer.

    Steps (math4ai "GPTQ Hessian" column-sweep paragraph, whose per-column
    equations the extraction lost; aicassindra "Greedy quantization with
    error compensation" and "GPTQ's speedups"):

    for each block [b0, b1) of ``block_size`` columns, for each column j in
    order: (at a group start, rebuild the grid from the current weights)
    round ``W[:, j]`` to the grid, take the error ``e = W[:, j] - What[:, j]``
    and its scaled form ``E_j = e / U_jj``; apply the OBS compensation to the
    rest of the block at once, ``W[:, j+1:b1] -= E_j U[j, j+1:b1]``; after the
    block, apply the deferred compensation ``W[:, b1:] -= E[:, b0:b1] U[b0:b1,
    b1:]``.

    Why row j of U: the OBS step moves the free weights by
    ``-(e / [Hf^-1]_jj) [Hf^-1]_{j,k}`` where Hf^-1 is the inverse restricted
    to the not-yet-quantized columns (mbrenndoerfer "Mathematical Details of
    the Update"); row j of the upper factor of H^-1 is that row divided by
    ``sqrt([Hf^-1]_jj) = U_jj``, so the move is ``-(e / U_jj) U_{j,k}``.

    Grid (reading): ``group_size == 0`` builds one grid per row from the
    input W before any change; ``group_size > 0`` rebuilds it at every
    ``j % group_size == 0`` from the current weights ``W[:, j:j+group_size]``,
    i.e. with the compensation of every column before j applied, which is
    what an unblocked sweep (B = 1) holds there.  Lazy batching only delays
    when updates are written ("same math"), so the grid does not depend on
    B: where a group reaches past the current block, its columns there get
    the block's pending compensation before the min/max is taken.  Dead
    columns are zeroed after the per-row grid, so they round to ``z`` with
    zero error and move nothing.

    ``hint`` (tie-aware replay): where the hint code differs from the own
    code, the hint is adopted and the difference is counted as a tie when
    the two codes are neighbours and ``v`` lies within ``tie_tol`` grid units
    of the midpoint between them, else as a hard mismatch.  Adopting keeps
    the replay on the hinted path so later decisions are compared against
    the same history.

    ``fixed_grid`` = (scales, zeros) per row overrides the grid (used for the
    worked example with its grid of step 0.5).  ``trace``, if a list, receives
    a copy of each column ``W[:, j]`` just before it is rounded.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    d_out, d_in = W.shape
    if U.shape != (d_in, d_in):
        raise ValueError("U shape")
    if not (1 <= bits <= 16):
        raise ValueError("bits")
    if block_size <= 0:
        raise ValueError("block_size")
    if group_size < 0 or (group_size > 0 and d_in % group_size):
        raise ValueError("group_size")
    maxq = 2 ** bits - 1
    n_groups = 1 if group_size == 0 else d_in // group_size
    scales = np.zeros((d_out, n_groups), F32)
    zeros = np.zeros((d_out, n_groups), np.int32)
    minmax = np.zeros((d_out, n_groups, 2), F32)
    codes = np.zeros((d_out, d_in), np.uint8)
    E = np.zeros((d_out, d_in))
    V = np.zeros((d_out, d_in), F32)
    w_hat = np.zeros((d_out, d_in))
    res_ties = 0
    res_hard = 0
    max_tie = 0.0
    mismatch_rows = np.zeros(d_out, bool)

    if fixed_grid is not None:
        s = np.asarray(fixed_grid[0], F32).reshape(d_out)
        z = np.asarray(fixed_grid[1], F32).reshape(d_out)
    elif group_size == 0:
        mn = W.astype(F32).min(axis=1) if d_in else np.zeros(d_out, F32)
        mx = W.astype(F32).max(axis=1) if d_in else np.zeros(d_out, F32)
        s, z = grid(mn, mx, bits)
        minmax[:, 0, 0] = np.minimum(mn, 0)
        minmax[:, 0, 1] = np.maximum(mx, 0)
    else:
        s = z = None
    if fixed_grid is not None or group_size == 0:
        scales[:, 0] = s
        zeros[:, 0] = z.astype(np.int32)
    if dead is not None and np.any(dead):
        W[:, np.asarray(dead, bool)] = 0.0

    for b0 in range(0, d_in, block_size):
        b1 = min(b0 + block_size, d_in)
        for j in range(b0, b1):
            if group_size and fixed_grid is None and j % group_size == 0:
                gcols = W[:, j:j + group_size].copy()
                # columns past this block still lack the compensation from
                # columns b0..j-1 (it is deferred to the block's end); the
                # grid sees them with it applied, as an unblocked sweep would
                lo = max(b1, j)
                if j > b0 and j + group_size > lo:
                    gcols[:, lo - j:] -= E[:, b0:j] @ U[b0:j, lo:j + group_size]
                mn = gcols.min(axis=1).astype(F32)
                mx = gcols.max(axis=1).astype(F32)
                s, z = grid(mn, mx, bits)
                g = j // group_size
                scales[:, g] = s
                zeros[:, g] = z.astype(np.int32)
                minmax[:, g, 0] = np.minimum(mn, 0)
                minmax[:, g, 1] = np.maximum(mx, 0)
            if trace is not None:
                trace.append(W[:, j].copy())
            q, v = quantize_values(W[:, j], s, z, bits)
            if hint is not None:
                h = np.asarray(hint[:, j], F32)
                diff = h != q
                if np.any(diff):
                    mid = (h[diff].astype(np.float64) + q[diff]) / 2.0
                    dist = np.abs(v[diff].astype(np.float64) - mid)
                    tie = (np.abs(h[diff].astype(np.float64) - q[diff]) == 1.0) & (dist <= tie_tol)
                    res_ties += int(tie.sum())
                    res_hard += int((~tie).sum())
                    if tie.any():
                        max_tie = max(max_tie, float(dist[tie].max()))
                    mismatch_rows[np.nonzero(diff)[0]] = True
                    q = np.where(diff, np.clip(h, 0, maxq), q).astype(F32)
            wq = s.astype(np.float64) * (q.astype(np.float64) - z.astype(np.float64))
            err = (W[:, j] - wq) / U[j, j]
            codes[:, j] = q.astype(np.uint8)
            V[:, j] = v
            w_hat[:, j] = wq
            E[:, j] = err
            if j + 1 < b1:
                W[:, j + 1:b1] -= np.outer(err, U[j, j + 1:b1])
        if b1 < d_in:
            W[:, b1:] -= E[:, b0:b1] @ U[b0:b1, b1:]
    err_sq = np.sum(E * E, axis=1)
    return QuantResult(codes, scales, zeros, minmax, E, V, w_hat, err_sq, res_ties, res_hard, max_tie,
                       mismatch_rows)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group_size: int = 0) -> np.ndarray:
    """``What = s (q - z)`` per row or per (row, group), in fp64."""
    codes = codes.astype(np.float64)
    d_out, d_in = codes.shape
    if group_size == 0:
        s = scales.reshape(d_out, -1)[:, :1].astype(np.float64)
        z = zeros.reshape(d_out, -1)[:, :1].astype(np.float64)
        return s * (codes - z)
    g = np.arange(d_in) // group_size
    return scales.astype(np.float64)[:, g] * (codes - zeros.astype(np.float64)[:, g])


def output_error(W: np.ndarray, W_hat: np.ndarray, x_chunks: Iterable[np.ndarray]) -> float:
    """``||W X - What X||_F^2`` in fp64 (aicassindra "The reconstruction
    objective, written out"), summed over token chunks; W is the original
    (undamped, not dead-zeroed) weight."""
    D = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    tot = 0.0
    for xc in x_chunks:
        Y = D @ np.asarray(xc, np.float64)
        tot += float(np.sum(Y * Y))
    return tot


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Few-bit storage of the codes: ``[d_out, ceil(d_in bits / 32)]`` uint32.

    The pages keep the quantized weights as low-bit integers (aicassindra
    "Post-training quantization and the per-layer objective": from 16-bit
    floats to 4-bit integers, 4 being the example given) and fix no bit
    layout.  Reading used here: each row's
    codes form one little-endian bit stream, code j in bits
    ``[j bits, (j+1) bits)``, least significant bit first, cut into 32-bit
    words; the last word of a row is zero-padded.  Written bit by bit.
    """
    codes = np.asarray(codes)
    d_out, d_in = codes.shape
    nw = (d_in * bits + 31) // 32
    out = np.zeros((d_out, nw), dtype=np.uint64)
    for j in range(d_in):
        c = codes[:, j].astype(np.uint64)
        for b in range(bits):
            t = j * bits + b
            out[:, t // 32] |= ((c >> np.uint64(b)) & np.uint64(1)) << np.uint64(t % 32)
    return out.astype(np.uint32)


def unpack_codes(packed: np.ndarray, bits: int, d_in: int) -> np.ndarray:
    """Inverse of ``pack_codes``: ``[d_out, d_in]`` uint8, bit by bit."""
    packed = np.asarray(packed).astype(np.uint64)
    d_out = packed.shape[0]
    codes = np.zeros((d_out, d_in), dtype=np.uint64)
    for j in range(d_in):
        for b in range(bits):
            t = j * bits + b
            codes[:, j] |= ((packed[:, t // 32] >> np.uint64(t % 32)) & np.uint64(1)) << np.uint64(b)
    return codes.astype(np.uint8)


def output_error_from_errors(err_sq: np.ndarray, W0: np.ndarray, W_hat: np.ndarray, lam: float) -> np.ndarray:
    """Per-row ``||dw X||^2`` without X, from the loss identity: the sum of
    squared scaled errors of a row is ``dw H_damped dw^T = 2 ||dw X||^2 +
    lambda ||dw||^2`` (aicassindra "The reconstruction objective, written
    out" with the damped Hessian of "The Cholesky trick"; pinned as P8), so
    ``||dw X||^2 = (sum e^2 - lambda ||dw||^2) / 2`` with ``dw = W0 - What``
    and W0 the weights with dead columns zeroed."""
    D = np.asarray(W0, np.float64) - np.asarray(W_hat, np.float64)
    return (np.asarray(err_sq, np.float64) - float(lam) * np.sum(D * D, axis=1)) / 2.0


# ----------------------------------------------------------------------------
# The greedy-order variant (OBQ) that the fixed order replaces
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class ObqResult:
    codes: np.ndarray       # [d_out, d_in] uint8
    scales: np.ndarray      # [d_out] float32
    zeros: np.ndarray       # [d_out] int32
    order: np.ndarray       # [d_out, d_in] int32: the column quantized at each step
    w_hat: np.ndarray       # [d_out, d_in] fp64 s (q - z)
    loss: np.ndarray        # [d_out] fp64 sum over the steps of e_q^2 / [Hf^-1]_qq
    ties: int = 0           # replay: picks or codes adopted from the hint at a near-tie
    hard: int = 0           # replay: adopted where the hint was not near a tie


def obq_quantize(W: np.ndarray, Hinv: np.ndarray, bits: int, dead: Optional[np.ndarray] = None,
                 fixed_order: bool = False, order_hint: Optional[np.ndarray] = None,
                 code_hint: Optional[np.ndarray] = None, pick_tol: float = 1e-9,
                 tie_tol: float = 1e-4, fixed_grid: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                 trace: Optional[list] = None) -> ObqResult:
    """Greedy-order quantization of each row with error compensation (OBQ).

    Per row, with ``Hf^-1`` the inverse Hessian restricted to the free
    (not yet quantized) weights, starting from ``Hinv`` = the inverse of the
    damped Hessian (aicassindra "Greedy quantization with error
    compensation"; mbrenndoerfer "Mathematical Details of the Update"):

    repeat until no weight is free:
      round every free weight to the grid, ``e_q = w_q - quant(w_q)``;
      pick the free q with the smallest ``e_q^2 / [Hf^-1]_qq`` (the lowest
      index among equal scores; with ``fixed_order`` simply the next column);
      move the free weights by ``delta = -(e_q / [Hf^-1]_qq) Hf^-1[:, q]``,
      which leaves ``w_q`` at its grid value;
      remove q: ``[Hf^-1]_ij -= [Hf^-1]_iq [Hf^-1]_qj / [Hf^-1]_qq``
      (the Schur complement; row and column q become zero).

    Grid, rounding and dead channels as in ``quantize`` with
    ``group_size == 0``: one grid per row from the input W, the rounding
    decision in fp32, dead columns zeroed after the grid.  ``loss`` sums the
    pick scores; it equals ``dw H_damped dw^T`` with ``dw = W0 - What``
    (every step's compensation is the constrained optimum).

    Replay (parity with a device run): with ``order_hint``, where the
    hinted pick differs from the own pick it is adopted and counted as a tie
    when its score is within ``pick_tol`` (relative) of the smallest,
    else as a hard mismatch; with ``code_hint`` the picked weight's code is
    compared as in ``quantize`` (tie within ``tie_tol`` grid units of the
    midpoint).  Adopting keeps the replay on the device's path.

    ``fixed_grid`` = (scales, zeros) per row overrides the grid (the worked
    example's grid of step 0.5); ``trace``, if a list, receives
    ``(row, q, score_q, w)`` after every step, ``w`` the row's weights then.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    Hinv = np.asarray(Hinv, dtype=np.float64)
    d_out, d_in = W.shape
    if Hinv.shape != (d_in, d_in):
        raise ValueError("Hinv shape")
    if not (1 <= bits <= 16):
        raise ValueError("bits")
    maxq = 2 ** bits - 1
    if fixed_grid is not None:
        s = np.asarray(fixed_grid[0], F32).reshape(d_out)
        z = np.asarray(fixed_grid[1], F32).reshape(d_out)
    else:
        mn = W.astype(F32).min(axis=1) if d_in else np.zeros(d_out, F32)
        mx = W.astype(F32).max(axis=1) if d_in else np.zeros(d_out, F32)
        s, z = grid(mn, mx, bits)
    if dead is not None and np.any(dead):
        W[:, np.asarray(dead, bool)] = 0.0
    codes = np.zeros((d_out, d_in), np.uint8)
    order = np.zeros((d_out, d_in), np.int32)
    w_hat = np.zeros((d_out, d_in))
    loss = np.zeros(d_out)
    ties = hard = 0
    for r in range(d_out):
        w = W[r].copy()
        Hf = Hinv.copy()
        free = np.ones(d_in, bool)
        sr = np.full(d_in, s[r], F32)
        zr = np.full(d_in, z[r], F32)
        for t in range(d_in):
            q_all, v_all = quantize_values(w, sr, zr, bits)
            wq_all = float(s[r]) * (q_all.astype(np.float64) - float(z[r]))
            e_all = w - wq_all
            score = np.full(d_in, np.inf)
            diag = np.diag(Hf)
            score[free] = e_all[free] ** 2 / diag[free]
            q = t if fixed_order else int(np.argmin(score))
            if order_hint is not None and int(order_hint[r, t]) != q:
                h = int(order_hint[r, t])
                if free[h] and score[h] <= score[q] * (1.0 + pick_tol):
                    ties += 1
                else:
                    hard += 1
                q = h
            code = q_all[q]
            if code_hint is not None and int(code_hint[r, q]) != int(code):
                hc = float(code_hint[r, q])
                if abs(hc - code) == 1.0 and abs(float(v_all[q]) - (hc + code) / 2.0) <= tie_tol:
                    ties += 1
                else:
                    hard += 1
                code = np.float32(min(max(hc, 0.0), maxq))
            wq = float(s[r]) * (float(code) - float(z[r]))
            e = w[q] - wq
            d = Hf[q, q]
            loss[r] += e * e / d
            col = Hf[:, q].copy()
            w[free] -= (e / d) * col[free]
            w[q] = wq
            Hf -= np.outer(col, Hf[q, :]) / d
            free[q] = False
            codes[r, q] = np.uint8(code)
            order[r, t] = q
            w_hat[r, q] = wq
            if trace is not None:
                trace.append((r, q, e * e / d, w.copy()))
    return ObqResult(codes, s.astype(F32), z.astype(np.int32), order, w_hat, loss, ties, hard)


def propagate(W_hat: np.ndarray, X: np.ndarray, activation: str = "none") -> np.ndarray:
    """The next layer's input from a quantized layer: ``Y = act(What X)`` in
    fp64, ``What: [d_out, d_in]``, ``X: [d_in, N]``.

    The pages quantize a network one linear layer at a time, each layer
    against its own input activations (math4ai "GPTQ Hessian", opening
    paragraph; aicassindra "Post-training quantization and the per-layer
    objective", X the layer's calibration inputs).  Reading for a chain of
    layers: the next layer's X is the already-quantized layer's output.  The
    pages name no nonlinearity; ``activation`` is "none" or "relu"
    (``max(0, .)``), the plainest stand-in.
    """
    Y = np.asarray(W_hat, dtype=np.float64) @ np.asarray(X, dtype=np.float64)
    if activation == "relu":
        Y = np.maximum(Y, 0.0)
    elif activation != "none":
        raise ValueError(f"activation {activation!r}")
    return Y


def layer(W: np.ndarray, x_chunks: Iterable[np.ndarray], bits: int, group_size: int, block_size: int,
          damp_frac: float = 0.01):
    """The whole path on one layer: returns ``(H, U, dead, lam, QuantResult)``."""
    xs = list(x_chunks)
    H = hessian(xs, d_in=W.shape[1])
    U, dead, lam = prepare(H, damp_frac)
    res = quantize(W, U, bits, group_size, block_size, dead=dead)
    return H, U, dead, lam, res
