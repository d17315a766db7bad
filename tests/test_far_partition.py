"""Host check of the quantize stage's far-update partition (no GPU).

Each launch of the quantize stage sweeps one lazy block and, in the same
launch, applies the previous block's scaled errors to every column after
the block (the lazy trailing update of aicassindra.com "tm_gptq_math",
"GPTQ's speedups: fixed order and lazy batches").  That update is cut into
units of 128 rows x 64 columns and dealt out as contiguous ranges: each
sweeping workgroup takes `per_sweep` units after its sweep, the far-only
workgroups share the rest evenly, and every workgroup walks its range in
sub-tiles of at most four strips.

The split, each workgroup's range and the sub-tile walk come from the code
the kernel and the launcher use (csrc/sched.hpp, built for the host by
tests/sched_lib.py).  The test checks that every (row tile, strip) of the
update is applied exactly once, for a spread of layer shapes, block widths
and CU counts.
"""
import pytest

import sched_lib

ROWS_PER_WG = 64      # rows of one sweeping workgroup (the sweep's lane = row)


def test_unit_shape():
    assert sched_lib.far_constants() == (128, 256, 64)


def walk(n_units, n_sweep, n_cu, c_begin, nstrip, d_in):
    """Every sub-tile of every workgroup's range, as the kernel walks them."""
    nf, _ = sched_lib.far_split(n_units, n_sweep, n_cu, c_begin, nstrip)
    for b in range(n_sweep + nf):
        u0, u1 = sched_lib.far_units(n_units, n_sweep, n_cu, c_begin, nstrip, b)
        assert 0 <= u0 <= u1 <= n_units, (b, u0, u1)
        u = u0
        while u < u1:
            t = sched_lib.far_sub(n_units, n_sweep, n_cu, c_begin, nstrip, u, u1, d_in)
            yield b, u, t
            assert t["ns"] > 0
            u += t["ns"]


@pytest.mark.parametrize("d_out", [1, 64, 100, 4096, 11008])
@pytest.mark.parametrize("d_in,block", [(128, 32), (300, 128), (4096, 128), (11008, 128), (1000, 96)])
@pytest.mark.parametrize("n_cu", [8, 32, 100, 256])
def test_every_unit_once(d_out, d_in, block, n_cu):
    rows, cols, strip = sched_lib.far_constants()
    n_sweep = (d_out + ROWS_PER_WG - 1) // ROWS_PER_WG
    rest_rows = (d_out + rows - 1) // rows
    for b0 in range(block, d_in, block):  # blocks after the first carry the previous block's update
        b1 = min(b0 + block, d_in)
        nstrip = (d_in - b1 + strip - 1) // strip
        n_units = rest_rows * nstrip if b1 < d_in else 0
        seen = set()
        for b, u, t in walk(n_units, n_sweep, n_cu, b1, nstrip, d_in):
            rt, st = divmod(u, nstrip)
            assert t["rt"] == rt < rest_rows
            assert 0 < t["ns"] <= cols // strip and st + t["ns"] <= nstrip
            # columns of the sub-tile: its strips, cut at the layer's edge
            assert t["c0"] == b1 + st * strip
            assert t["c_end"] == min(d_in, t["c0"] + t["ns"] * strip) and t["c_end"] > t["c0"]
            for k in range(t["ns"]):
                key = (rt, st + k)
                assert key not in seen, f"unit {key} applied twice (block {b0})"
                seen.add(key)
        assert len(seen) == n_units, f"block {b0}: {n_units - len(seen)} units never applied"
        # the launch never holds more workgroups than the sweep plus one per free CU
        nf, _ = sched_lib.far_split(n_units, n_sweep, n_cu, b1, nstrip)
        assert nf <= max(0, n_cu - n_sweep)


def test_sweepers_take_less_when_the_update_is_small():
    """Late blocks: the sweeping workgroups do no far work at all."""
    n_sweep, n_cu = 64, 256
    nf, fs = sched_lib.far_split(448, n_sweep, n_cu, 0, 7)
    assert fs["per_sweep"] == 0 and nf * fs["q"] + fs["r"] == 448
    nf, fs = sched_lib.far_split(1920, n_sweep, n_cu, 0, 60)
    assert 0 < fs["per_sweep"] < fs["q"] + 1


def test_more_sweepers_than_cus_do_it_all():
    nf, fs = sched_lib.far_split(1000, 300, 256, 0, 10)
    assert nf == 0 and fs["per_sweep"] * 300 >= 1000
