"""Host check of the factorization's launch schedule (no GPU).

The device builds L^-1 for G = L L^T (G = J H_damped J, the reversed
Hessian) in 64-wide steps, one launch per step: the diagonal-block
workgroups of step k+1 apply step k's update to the blocks they read, in
registers, then factor the diagonal block and form step k+1's panel; one
workgroup copies M_kk into G_kk; the others apply step k's update to every
other block.  On wide layers the steps are paired: an even step's update of
those other blocks is deferred and applied in the next launch together with
the odd step's, and the odd launch's diagonal-block workgroups apply both
steps.  Step s's panel lives in buffer s % 3.

Who does what in each launch comes from the schedule code the kernels and
the launcher use (csrc/sched.hpp, built for the host by tests/sched_lib.py):
the launch geometry and the tile of each rest workgroup.  This replays that
schedule block by block in numpy (every launch reads the
state as it was when the launch started, as the device's workgroups do) with
small blocks, and checks the result against the inverse of numpy's Cholesky
factor: a block missed, applied twice, read from the wrong panel buffer or
read after it was overwritten shows up as a wrong L^-1.  The inverse
Cholesky factor is the Cholesky trick of aicassindra.com "tm_gptq_math"
("The Cholesky trick for the inverse Hessian"), with H^-1 = U^T U and
U = J L^-1 J.
"""
import numpy as np
import pytest

import sched_lib


def _inv_chol(D):
    return np.linalg.inv(np.linalg.cholesky(D))


def replay(Gfull, nb, paired):
    n = Gfull.shape[0]
    T = n // nb
    G = {(i, j): Gfull[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb].copy() for i in range(T) for j in range(i + 1)}
    P = [dict(), dict(), dict()]
    # step 0: diagonal block and panel
    M = _inv_chol(G[0, 0])
    P[0][0] = M
    for i in range(1, T):
        P[0][i] = G[i, 0] @ M.T
    for k in range(T):
        old = {key: v.copy() for key, v in G.items()}
        Pk, Pkm, Pk1 = P[k % 3], P[(k + 2) % 3], P[(k + 1) % 3]
        odd = k % 2 == 1
        pair = paired and odd
        writes = {}
        k1 = k + 1
        if k1 < T:
            pd = Pk[k1]
            D = old[k1, k1] - pd @ pd.T
            c2 = {}
            for t in range(T - 1):
                if t >= k1:
                    c2[t] = old[t + 1, k1] - Pk[t + 1] @ pd.T
                elif t == k:
                    c2[t] = -(pd @ Pk[0])
                elif pair and t == k - 1:
                    c2[t] = -(pd @ old[k, t])
                else:
                    c2[t] = old[k1, t] - pd @ old[k, t]
            if pair:
                pm = Pkm[k1]
                D = D - pm @ pm.T
                for t in range(T - 1):
                    if t >= k1:
                        c2[t] = c2[t] - Pkm[t + 1] @ pm.T
                    elif t == k:
                        pass
                    elif t == k - 1:
                        c2[t] = c2[t] - pm @ Pkm[0]
                    else:
                        c2[t] = c2[t] - pm @ old[k - 1, t]
            Mk1 = _inv_chol(D)
            Pk1.clear()
            Pk1[0] = Mk1
            for t in range(T - 1):
                if t < k1:
                    writes[k1, t] = Mk1 @ c2[t]
                else:
                    Pk1[t + 1] = c2[t] @ Mk1.T
        writes[k, k] = Pk[0].copy()
        g = sched_lib.chol_geom(k, T, paired)
        assert g["nchain"] == (max(T - 1, 1) if k1 < T else 0)
        assert g["grid"] == g["nchain"] + 1 + g["n_rest"]
        assert g["n_rest"] == (0 if (paired and not odd) else sched_lib.chol_rest_tiles(k, T))
        rest = [sched_lib.chol_rest_tile(k, b) for b in range(g["n_rest"])]
        assert len(set(rest)) == len(rest)
        for i, j in rest:
            assert k + 2 <= i < T and 0 <= j <= i and j != k1
            if True:
                if True:
                    if not pair:
                        if j < k:
                            writes[i, j] = old[i, j] - Pk[i] @ old[k, j]
                        elif j == k:
                            writes[i, j] = -(Pk[i] @ Pk[0])
                        else:
                            writes[i, j] = old[i, j] - Pk[i] @ Pk[j].T
                    else:
                        if j < k - 1:
                            writes[i, j] = old[i, j] - Pkm[i] @ old[k - 1, j] - Pk[i] @ old[k, j]
                        elif j == k - 1:
                            writes[i, j] = -(Pkm[i] @ Pkm[0]) - Pk[i] @ old[k, j]
                        elif j == k:
                            writes[i, j] = -(Pk[i] @ Pk[0])
                        else:
                            writes[i, j] = old[i, j] - Pkm[i] @ Pkm[j].T - Pk[i] @ Pk[j].T
        G.update(writes)
    Minv = np.zeros_like(Gfull)
    for (i, j), v in G.items():
        Minv[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb] = v
    return np.tril(Minv)


@pytest.mark.parametrize("paired", [False, True])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8, 9, 13])
def test_schedule_builds_inverse_cholesky_factor(T, paired):
    nb = 3
    n = T * nb
    rng = np.random.default_rng(100 + T)
    A = rng.standard_normal((n, 2 * n))
    Gfull = A @ A.T + 0.5 * np.eye(n)
    got = replay(Gfull, nb, paired)
    want = _inv_chol(Gfull)
    assert np.allclose(got, want, rtol=1e-9, atol=1e-9 * np.abs(want).max())


def test_schedule_gives_u_of_the_inverse():
    """U = J L^-1 J is the upper Cholesky factor of H^-1 (H^-1 = U^T U)."""
    nb, T = 2, 5
    n = nb * T
    rng = np.random.default_rng(7)
    A = rng.standard_normal((n, 3 * n))
    H = A @ A.T + np.eye(n)
    J = np.eye(n)[::-1]
    Minv = replay(J @ H @ J, nb, paired=True)
    U = J @ Minv @ J
    assert np.allclose(np.tril(U, -1), 0.0)
    assert np.allclose(U.T @ U, np.linalg.inv(H), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("T", [64, 172, 129, 2048])
def test_launch_geometry_at_layer_widths(T):
    """Every launch at the widths the layers use: the rest items of step k
    are exactly the lower tiles below row k+1 outside column and row block
    k+1 (or none, for a deferred even step), in the row-major order."""
    paired = bool(sched_lib.load().chol_paired_default(T))
    assert paired == (T >= 128)
    for k in range(T):
        g = sched_lib.chol_geom(k, T, paired)
        n = g["n_rest"]
        if paired and k % 2 == 0:
            assert n == 0
            continue
        # row i >= k+2 holds i items (columns 0..i without k+1)
        assert n == sum(range(k + 2, T))
        for b in {0, n // 3, n // 2, n - 1} if n else ():
            i, j = sched_lib.chol_rest_tile(k, b)
            assert k + 2 <= i < T and 0 <= j <= i and j != k + 1
            assert b == sum(range(k + 2, i)) + (j if j < k + 1 else j - 1)


def test_rest_tile_enumeration_is_row_major():
    for T in (5, 17, 64):
        for k in range(T):
            want = [(i, j) for i in range(k + 2, T) for j in range(i + 1) if j != k + 1]
            got = [sched_lib.chol_rest_tile(k, b) for b in range(sched_lib.chol_rest_tiles(k, T))]
            assert got == want
