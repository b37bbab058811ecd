"""Pins of the Morton (Z-order) reorder oracle.

The "Piecewise-Taylor-Attention" README names the curve (Wan2.1 results
paragraph; changelog item on the Morton tile reorder and its fused gather
kernel) but prints no order. The pins are the curve's definition worked by
hand on small grids (tests/golden/z_order_2d.txt), the inverse map (decoding
codes instead of sorting them), the locality that defines the curve's use
(aligned runs of 8^m cells of a power-of-two cube are cubes), and brute-force
loops for the gather / scatter.
"""

import os

import numpy as np
import pytest

from oracle import reorder_oracle as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "z_order_2d.txt")


def golden_2d():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split(":")
        rows, cols = (int(x) for x in lhs.split())
        out.append(((rows, cols), [int(x) for x in rhs.split()]))
    return out


@pytest.mark.parametrize("case", golden_2d(), ids=lambda c: f"{c[0][0]}x{c[0][1]}")
def test_z_order_matches_hand_worked_2d(case):
    grid, want = case
    assert R.z_order(grid).tolist() == want


def test_z_order_2x2x2_is_raster_order():
    # with the fastest axis on the lowest bit, the 2x2x2 codes equal the raster indices
    assert R.z_order((2, 2, 2)).tolist() == list(range(8))


@pytest.mark.parametrize("grid", [(3, 5, 6), (21, 30, 52)[:1] + (5, 7), (5, 9), (1, 7, 3), (2, 3, 4)])
def test_z_order_equals_cube_walk_by_decoding(grid):
    """Z2 by another route: walk every code of the enclosing cube, decode it, keep cells inside."""
    ndim = len(grid)
    nb = max(int(np.ceil(np.log2(max(g, 2)))) for g in grid)
    want = []
    for code in range(1 << (ndim * nb)):
        c = R.z_decode(code, ndim, nb)
        if all(ci < gi for ci, gi in zip(c, grid)):
            want.append(int(np.ravel_multi_index(c, grid)))
    assert R.z_order(grid).tolist() == want


def test_z_order_is_a_permutation_with_prefix():
    grid, prefix = (4, 6, 5), 17
    p = R.z_order(grid, prefix)
    n = prefix + 4 * 6 * 5
    assert p.dtype == np.int32 and p.shape == (n,)
    assert p[:prefix].tolist() == list(range(prefix))
    assert sorted(p.tolist()) == list(range(n))
    assert (p[prefix:] - prefix).tolist() == R.z_order(grid).tolist()


@pytest.mark.parametrize("m", [1, 2])
def test_aligned_runs_of_a_cube_are_cubes(m):
    """Runs of 8^m consecutive cells of an 8x8x8 Z-order are (2^m)^3 sub-cubes."""
    grid = (8, 8, 8)
    p = R.z_order(grid)
    run = 8 ** m
    side = 2 ** m
    for s in range(0, p.size, run):
        c = np.stack(np.unravel_index(p[s:s + run], grid), axis=1)
        lo = c.min(axis=0)
        assert (c.max(axis=0) - lo == side - 1).all()
        assert (lo % side == 0).all()
        assert len({tuple(x) for x in c}) == run


def test_gather_and_scatter_by_loops():
    r = np.random.default_rng(3)
    B, T, H, D = 2, 13, 3, 4
    x = r.standard_normal((B, T, H, D))
    perm = r.permutation(T).astype(np.int32)
    g = R.gather_head_major(x, perm)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                assert np.array_equal(g[b, h, i], x[b, perm[i], h])
    y = R.scatter_token_major(g, perm)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                assert np.array_equal(y[b, perm[i], h], g[b, h, i])
    assert np.array_equal(y, x)          # the scatter inverts the gather
