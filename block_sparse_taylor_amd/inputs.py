"""Seeded synthetic inputs shaped like the DiT attention workloads.

This module only draws numbers: it holds none of the attention method's
arithmetic and is shared by the tests, the benchmark and the smoke check.

Workloads (shapes as the PISA paper, §4.1, and the Piecewise-Taylor-Attention
README describe them; the real activations are not available, so these
stand in for them):

* ``tiny``    batch 1, 2 heads, T=1024, D=64, fp32, q,k,v i.i.d. N(0,1).
* ``wan13``   Wan2.1-1.3B 480p: 12 heads, D=128, 21x30x52 latent grid
              (T=32760) in 3D Morton order, bf16.
* ``wan14``   Wan2.1-14B: as wan13 with 40 heads and two outlier key
              dimensions (k[..., 0:2] scaled by 8).
* ``hunyuan`` Hunyuan-Video 720p: 24 heads, 33x45x80 grid (T=118800).
* ``flux``    FLUX 1024^2: 24 heads, 512 text tokens (i.i.d. N(0,1)) then
              64x64 image tokens in 2D Morton order, T=4608.
* ``wan14_kv`` a test case, not a benchmark: the Wan2.1-14B shape (8 heads)
              with v built from the key noise (v[:, d] = eps_k[:, (d + 1) % D]),
              so values follow the in-block key deviations and the global
              first-order matrix sum_j (K_j - kbar_j)^T V_j grows like T
              instead of averaging out.

Spatially correlated q/k: per head a smooth field
f_d(p) = sum_{m<8} a_{d,m} cos(2 pi w_m . p + phi_{d,m}) with integer
frequencies w_m in {0..3}^dims, a ~ N(0, 1/4) (so Var f_d = 1) and
phi ~ U[0, 2 pi); q = f + 0.3 eps_q, k = f + 0.3 eps_k, v ~ N(0, 1).
Every (batch, head) draws from its own counter-addressed stream
``SeedSequence(seed, spawn_key=(b, h, tensor))``, so any head can be
regenerated alone. bf16 tensors are rounded to nearest-even from fp32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_head", "make_inputs", "bf16_bits", "bf16_to_f64",
           "morton_order"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    density: float
    band: int
    second_order: bool
    seed: int
    kind: str                  # "iid", "video", "image"
    grid: tuple = ()
    text_tokens: int = 0
    outlier_key_dims: tuple = ()
    v_from_key_noise: bool = False
    block: int = 64
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1024, 64, "f32", 0.25, 1, False, 0, "iid",
                     note="q,k,v i.i.d. N(0,1); softmax scale 1/sqrt(64)"),
    "wan13": Workload("wan13", 1, 12, 32760, 128, "bf16", 0.125, 1, False, 1, "video",
                      grid=(21, 30, 52)),
    "wan14": Workload("wan14", 1, 40, 32760, 128, "bf16", 0.125, 1, False, 2, "video",
                      grid=(21, 30, 52), outlier_key_dims=(0, 1)),
    "hunyuan": Workload("hunyuan", 1, 24, 118800, 128, "bf16", 0.125, 1, True, 3, "video",
                        grid=(33, 45, 80)),
    "flux": Workload("flux", 1, 24, 4608, 128, "bf16", 0.15, 1, False, 4, "image",
                     grid=(64, 64), text_tokens=512),
    # one GPU's share of the Wan2.1-14B shape with its 40 heads sharded over 8
    # GPUs: heads 0..4 of the same inputs (the streams are per (seed, batch, head))
    "wan14_shard8": Workload("wan14_shard8", 1, 5, 32760, 128, "bf16", 0.125, 1, False, 2, "video",
                             grid=(21, 30, 52), outlier_key_dims=(0, 1)),
    "wan14_kv": Workload("wan14_kv", 1, 8, 32760, 128, "bf16", 0.125, 1, False, 5, "video",
                         grid=(21, 30, 52), outlier_key_dims=(0, 1), v_from_key_noise=True),
}


def _bits_needed(n: int) -> int:
    return max(1, int(n - 1).bit_length())


def morton_order(grid: tuple) -> np.ndarray:
    """Cells of ``grid`` (slowest axis first) sorted by their Z-order code.

    Code bit (dims*b + a) holds bit b of the coordinate on axis (dims-1-a),
    so the fastest axis supplies the lowest bit of every bit group. Returns
    the flat cell index of each token in emission order.
    """
    dims = len(grid)
    coords = np.indices(grid).reshape(dims, -1)        # [dims, cells]
    nbits = max(_bits_needed(g) for g in grid)
    code = np.zeros(coords.shape[1], dtype=np.int64)
    for b in range(nbits):
        for a in range(dims):
            axis = dims - 1 - a
            code |= ((coords[axis] >> b) & 1).astype(np.int64) << (dims * b + a)
    return np.argsort(code, kind="stable")


def _positions(grid: tuple) -> np.ndarray:
    """Cell-centre positions in [0,1]^dims of the Morton-ordered tokens."""
    order = morton_order(grid)
    coords = np.stack(np.unravel_index(order, grid), axis=1).astype(np.float64)
    return (coords + 0.5) / np.asarray(grid, dtype=np.float64)


def _rng(seed: int, b: int, h: int, t: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(b, h, t))))


def _field(rng: np.random.Generator, pos: np.ndarray, D: int, n_terms: int = 8) -> np.ndarray:
    dims = pos.shape[1]
    omega = rng.integers(0, 4, size=(n_terms, dims)).astype(np.float64)
    amp = rng.normal(0.0, 0.5, size=(n_terms, D))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(n_terms, D))
    theta = 2.0 * np.pi * (pos @ omega.T)                        # [T, m]
    return np.cos(theta) @ (amp * np.cos(phi)) - np.sin(theta) @ (amp * np.sin(phi))


def make_head(w: Workload, b: int, h: int):
    """float64 q, k, v [T, D] of one (batch, head), before dtype rounding."""
    T, D = w.seq_len, w.head_dim
    if w.kind == "iid":
        q = _rng(w.seed, b, h, 1).standard_normal((T, D))
        k = _rng(w.seed, b, h, 2).standard_normal((T, D))
        v = _rng(w.seed, b, h, 3).standard_normal((T, D))
        return q, k, v
    n_text = w.text_tokens
    pos = _positions(w.grid)
    assert n_text + pos.shape[0] == T, (w.name, n_text, pos.shape, T)
    f = _field(_rng(w.seed, b, h, 0), pos, D)
    eq = _rng(w.seed, b, h, 1).standard_normal((T, D))
    ek = _rng(w.seed, b, h, 2).standard_normal((T, D))
    v = _rng(w.seed, b, h, 3).standard_normal((T, D))
    q = eq.copy()
    k = ek.copy()
    q[n_text:] = f + 0.3 * eq[n_text:]
    k[n_text:] = f + 0.3 * ek[n_text:]
    if w.v_from_key_noise:
        v = np.roll(ek, -1, axis=1)
    for d in w.outlier_key_dims:
        k[:, d] *= 8.0
    return q, k, v


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to fp32 (nearest-even), then to bf16 (nearest-even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def make_inputs(w: Workload, heads=None, batches=None):
    """q, k, v as [Bt, H', T, D] arrays in the workload's storage type.

    bf16 workloads return uint16 bit patterns (view them as bfloat16); fp32
    workloads return float32. ``heads``/``batches`` select a subset.
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    T, D = w.seq_len, w.head_dim
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    out = [np.empty((len(batches), len(heads), T, D), dtype=dt) for _ in range(3)]
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            for arr, x in zip(out, make_head(w, b, h)):
                arr[bi, hi] = bf16_bits(x) if w.dtype == "bf16" else x.astype(np.float32)
    return tuple(out)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 upcast of stored inputs."""
    return bf16_to_f64(x) if dtype == "bf16" else x.astype(np.float64)
