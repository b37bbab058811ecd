"""Plain CPU oracle for the Morton (Z-order) token reorder around the operator.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP library and imports nothing from it.

Source: the "Piecewise-Taylor-Attention" README (GitHub HaoyiZhu), the
Wan2.1 results paragraph (64-token blocks over a Morton / Z-order tile
reordering of the 480x832x81 latent grid) and the changelog item on the
Morton tile reorder with its fused gather kernel (one kernel that gathers the
tokens into the new order while transposing [B,T,H,D] into [B,H,T,D], and
the inverse on the output).

The pages name the curve but do not spell out its bit order. The Z-order
(Morton) curve is the textbook one: a cell's code interleaves the bits of its
coordinates, bit b of every coordinate forming bit group b, groups ascending.
Readings adopted (both this oracle and the HIP library's host helper follow
them):

Z1  grid axes are listed slowest first (frames, rows, columns for video;
    rows, columns for images); inside a bit group the fastest axis supplies
    the lowest bit. Cells are visited in ascending code; codes are distinct.
Z2  a grid that is not a power of two per axis is visited in the order of the
    enclosing power-of-two cube with the missing cells skipped (coordinates
    padded with zero high bits).
Z3  tokens are numbered raster-order (row-major over the grid, fastest axis
    last); ``prefix`` leading tokens (e.g. text tokens before image tokens)
    keep their places and the grid's cells follow them.
Z4  perm[i] is the raster index of the token placed at position i; the
    gather is out[b, h, i] = x[b, perm[i], h], the inverse scatters
    y[b, perm[i], h] = o[b, h, i].
"""

from __future__ import annotations

import numpy as np

__all__ = ["z_order", "z_decode", "gather_head_major", "scatter_token_major"]


def _bits(n: int) -> int:
    """Bits needed for coordinates 0 .. n-1."""
    b = 0
    while (1 << b) < n:
        b += 1
    return max(b, 1)


def z_order(grid, prefix: int = 0) -> np.ndarray:
    """perm for a grid (slowest axis first) after ``prefix`` fixed tokens (Z1-Z4)."""
    grid = tuple(int(g) for g in grid)
    ndim = len(grid)
    nb = max(_bits(g) for g in grid)
    cells = int(np.prod(grid))
    coords = np.indices(grid).reshape(ndim, cells).astype(np.int64)
    code = np.zeros(cells, dtype=np.int64)
    for b in range(nb):                       # bit group b
        for slot in range(ndim):              # slot 0 = fastest axis
            axis = ndim - 1 - slot
            code |= ((coords[axis] >> b) & 1) << (ndim * b + slot)
    order = np.argsort(code)                  # codes are distinct
    return np.concatenate([np.arange(prefix, dtype=np.int64), prefix + order]).astype(np.int32)


def z_decode(code: int, ndim: int, nb: int):
    """Coordinates (slowest axis first) of a Z-order code: the inverse map."""
    c = [0] * ndim
    for b in range(nb):
        for slot in range(ndim):
            c[ndim - 1 - slot] |= ((code >> (ndim * b + slot)) & 1) << b
    return tuple(c)


def gather_head_major(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """[B,T,H,D] -> [B,H,T,D] with out[b, h, i] = x[b, perm[i], h]  (Z4)."""
    return np.ascontiguousarray(x[:, perm].transpose(0, 2, 1, 3))


def scatter_token_major(o: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """[B,H,T,D] -> [B,T,H,D] with y[b, perm[i], h] = o[b, h, i]  (Z4)."""
    y = np.empty((o.shape[0], o.shape[2], o.shape[1], o.shape[3]), dtype=o.dtype)
    y[:, perm] = o.transpose(0, 2, 1, 3)
    return y
