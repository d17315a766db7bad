"""Host check of the quantize stage's far-update partition (no GPU).

Each launch of the quantize stage sweeps one lazy block and, in the same
launch, applies the previous block's scaled errors to every column after
the block (the lazy trailing update of aicassindra.com "tm_gptq_math",
"GPTQ's speedups: fixed order and lazy batches").  That update is cut into
units of 128 rows x 64 columns and dealt out as contiguous ranges: each
sweeping workgroup takes `per_sweep` units after its sweep, the far-only
workgroups share the rest evenly, and every workgroup walks its range in
sub-tiles of at most four strips.

This mirrors `far_split` and the range arithmetic of `step_kernel` /
`far_range` (csrc/quant.hip) and checks that every (row tile, strip) of
the update is applied exactly once, for a spread of layer shapes, block
widths and CU counts.
"""
import math

import pytest

ROWS_PER_WG = 64      # rows of one sweeping workgroup
REST_ROWS = 128       # rows of a far-update unit
STRIP = 64            # columns of a far-update unit
REST_COLS = 256       # columns of a far-update sub-tile
SWEEP_UNITS = 3.0     # a sweep's duration in units


def far_split(n_units, n_sweep, n_cu):
    """(n_far, per_sweep, q, r) as the launcher computes them."""
    if n_units <= 0:
        return 0, 0, 0, 0
    n_far = max(0, n_cu - n_sweep)
    if n_far == 0:
        return 0, (n_units + n_sweep - 1) // n_sweep, 0, 0
    t = (n_units + n_sweep * SWEEP_UNITS) / (n_sweep + n_far)
    per_sweep = int(max(0.0, math.floor(t - SWEEP_UNITS)))
    rest = n_units - n_sweep * per_sweep
    nf = min(n_far, rest)
    q = r = 0
    if nf > 0:
        q, r = rest // nf, rest % nf
    return nf, per_sweep, q, r


def ranges(n_units, n_sweep, n_cu):
    nf, per_sweep, q, r = far_split(n_units, n_sweep, n_cu)
    out = []
    for b in range(n_sweep + nf):
        if b < n_sweep:
            u0 = min(b * per_sweep, n_units)
            u1 = min(u0 + per_sweep, n_units)
        else:
            f = b - n_sweep
            u0 = n_sweep * per_sweep + f * q + min(f, r)
            u1 = u0 + q + (1 if f < r else 0)
        out.append((u0, u1))
    return out


def sub_tiles(u0, u1, nstrip):
    """(row tile, first strip, strips) of each sub-tile a range walks."""
    u = u0
    while u < u1:
        rt, st = divmod(u, nstrip)
        ns = min(REST_COLS // STRIP, nstrip - st, u1 - u)
        yield rt, st, ns
        u += ns


@pytest.mark.parametrize("d_out", [1, 64, 100, 4096, 11008])
@pytest.mark.parametrize("d_in,block", [(128, 32), (300, 128), (4096, 128), (11008, 128), (1000, 96)])
@pytest.mark.parametrize("n_cu", [8, 32, 100, 256])
def test_every_unit_once(d_out, d_in, block, n_cu):
    n_sweep = (d_out + ROWS_PER_WG - 1) // ROWS_PER_WG
    rest_rows = (d_out + REST_ROWS - 1) // REST_ROWS
    for b0 in range(block, d_in, block):  # blocks after the first carry the previous block's update
        b1 = min(b0 + block, d_in)
        nstrip = (d_in - b1 + STRIP - 1) // STRIP
        n_units = rest_rows * nstrip if b1 < d_in else 0
        seen = {}
        for u0, u1 in ranges(n_units, n_sweep, n_cu):
            assert 0 <= u0 <= u1 <= n_units
            for rt, st, ns in sub_tiles(u0, u1, nstrip):
                assert rt < rest_rows and 0 < ns <= REST_COLS // STRIP and st + ns <= nstrip
                for k in range(ns):
                    key = (rt, st + k)
                    assert key not in seen, f"unit {key} applied twice (block {b0})"
                    seen[key] = True
        assert len(seen) == n_units, f"block {b0}: {n_units - len(seen)} units never applied"
        # the launch never holds more workgroups than the sweep plus one per free CU
        nf, _, _, _ = far_split(n_units, n_sweep, n_cu)
        assert nf <= max(0, n_cu - n_sweep)


def test_sweepers_take_less_when_the_update_is_small():
    """Late blocks: the sweeping workgroups do no far work at all."""
    n_sweep, n_cu = 64, 256
    nf, per_sweep, q, r = far_split(448, n_sweep, n_cu)
    assert per_sweep == 0 and nf * q + r == 448
    nf, per_sweep, q, r = far_split(1920, n_sweep, n_cu)
    assert per_sweep > 0 and per_sweep < q + 1
