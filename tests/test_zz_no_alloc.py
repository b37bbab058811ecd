"""pisa_block_stats_noalloc, the statistics pass for callers that cannot
allocate (its partial H sums live in the library's static device scratch
instead of a caller workspace), against pisa_block_stats: the same kernels
and launch shapes, so every statistic and every byte of the operand buffer
must agree exactly (the statistics' own bar is bit-exact means, one fp32
rounding of V-hat and a derived bound on H, all met with equality). Two calls
in a row, the second smaller than the first, so the second runs on what the
first left in the scratch."""

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from block_sparse_taylor_amd import inputs as I
from oracle import pisa_oracle as O

from gpu_common import head_f64, say, to_device

pytestmark = pytest.mark.gpu


def one_call(name, heads, so):
    w = I.WORKLOADS[name]
    arrs = I.make_inputs(w, heads=heads)
    q, k, v = (to_device(a, w.dtype) for a in arrs)
    say(f"[gpu] noalloc stats {name}: {tuple(q.shape)} second_order={so}")
    a = P.alloc_stats(k, so, operands=False)
    a.operands = torch.zeros(P.operands_bytes(k), dtype=torch.uint8, device=k.device)
    P.pisa_block_stats(q, k, v, second_order=so, out=a)
    b = P.alloc_stats(k, so, operands=False)
    b.operands = torch.zeros(P.operands_bytes(k), dtype=torch.uint8, device=k.device)
    P.pisa_block_stats_noalloc(q, k, v, b, second_order=so)
    torch.cuda.synchronize()
    for x, y in zip(a.__dict__.values(), b.__dict__.values()):
        if x is not None:
            assert torch.equal(x, y)
    # and the shared result against the oracle's H for one head
    qh, kh, vh = head_f64(arrs, w.dtype, 0, 0)
    ref = O.kv_block_stats(kh, vh, 64)
    mag = np.abs(kh).T @ np.abs(vh)
    err = np.abs(b.hsum[0, 0].double().cpu().numpy() - ref.H)
    assert (err <= 64 * 2.0 ** -24 * mag + 1e-30).all()


def test_noalloc_stats_twice_second_smaller():
    # first: the Wan2.1-14B shape, 40 heads (31.5 MiB of the 32 MiB scratch)
    one_call("wan14", None, False)
    # second: a FLUX-shaped call with 4 heads and the second-order statistics
    one_call("flux", [0, 1, 2, 3], True)
