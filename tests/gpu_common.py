"""Helpers shared by the GPU parity tests (inputs to device, oracle per head)."""

import functools
import sys

import numpy as np
import torch

from block_sparse_taylor_amd import inputs as I

BLOCK = 64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


@functools.lru_cache(maxsize=2)
def workload_inputs(name: str):
    """Host arrays (storage type) of a whole workload."""
    w = I.WORKLOADS[name]
    return w, I.make_inputs(w)


def head_f64(arrs, dtype, b, h):
    return [I.as_f64(a[b, h], dtype) for a in arrs]


def n_blocks(T):
    return -(-T // BLOCK)


def oracle_topk(density, N):
    # the routed count the tests expect: floor(density * N), band excluded
    return int(np.floor(density * N + 1e-9))


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (nearest) -> bf16 (nearest-even), as float64."""
    return I.bf16_to_f64(I.bf16_bits(x))
