"""GPU parity of the Morton token reorder (pisa_reorder_gather / _scatter and
the library's host Z-order) against the reorder oracle, bit for bit, plus the
operator run on token-major raster-order inputs with reorder="morton"."""

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from oracle import pisa_oracle as O
from oracle import reorder_oracle as R

from gpu_common import say

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a device tensor on the host (exact comparison)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


def make_x(B, T, H, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, H, D, generator=g)
    return x.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


CASES = [
    # name, B, T, H, D, dtype, perm source
    ("wan14_raster", 1, 32760, 40, 128, "bf16", ("z", (21, 30, 52), 0)),
    ("flux_text_prefix", 1, 4608, 24, 128, "bf16", ("z", (64, 64), 512)),
    ("fp32_random_perm", 2, 1000, 3, 64, "f32", ("rand", 1000)),
    ("ragged_fp32_d128", 3, 77, 5, 128, "f32", ("rand", 77)),
    ("one_token", 1, 1, 1, 64, "bf16", ("rand", 1)),
    ("many_heads_bf16_d64", 1, 300, 130, 64, "bf16", ("z", (3, 10, 10), 0)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gather_scatter_match_oracle(case):
    name, B, T, H, D, dtype, src = case
    say(f"[gpu] reorder {name}: B={B} T={T} H={H} D={D} {dtype}")
    if src[0] == "z":
        perm_h = P.z_order(src[1], src[2]).numpy()
        assert np.array_equal(perm_h, R.z_order(src[1], src[2]))
    else:
        perm_h = np.random.default_rng(T).permutation(src[1]).astype(np.int32)
    perm = torch.from_numpy(perm_h).cuda()
    x = make_x(B, T, H, D, dtype, seed=T + H)
    g = P.reorder_gather(x, perm)
    torch.cuda.synchronize()
    xb = bits(x)
    assert np.array_equal(bits(g), R.gather_head_major(xb, perm_h))
    y = P.reorder_scatter(g, perm)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), R.scatter_token_major(bits(g), perm_h))
    assert np.array_equal(bits(y), xb)          # the scatter inverts the gather


def test_out_of_range_perm_entries():
    """Gather writes zeros where perm is outside [0, T); scatter skips those positions."""
    B, T, H, D = 1, 200, 3, 64
    say("[gpu] reorder out-of-range perm entries")
    perm_h = np.random.default_rng(5).permutation(T).astype(np.int32)
    bad = np.array([0, 17, 199])
    perm_h[bad] = [-1, T, 1 << 30]
    perm = torch.from_numpy(perm_h).cuda()
    x = make_x(B, T, H, D, "f32", seed=9)
    g = P.reorder_gather(x, perm)
    y = torch.full_like(x, 7.0)
    P.reorder_scatter(g, perm, out=y)
    torch.cuda.synchronize()
    gh, xh, yh = g.cpu().numpy(), x.cpu().numpy(), y.cpu().numpy()
    ok = np.setdiff1d(np.arange(T), bad)
    assert (gh[:, :, bad] == 0).all()
    assert np.array_equal(gh[:, :, ok], xh[:, perm_h[ok]].transpose(0, 2, 1, 3))
    hit = np.zeros(T, bool)
    hit[perm_h[ok]] = True
    assert np.array_equal(yh[:, hit], xh[:, hit])
    assert (yh[:, ~hit] == 7.0).all()


def test_operator_with_morton_reorder_matches_oracle():
    """Token-major raster input, reorder="morton": the oracle gathers, runs PISA
    per head and scatters back; fp32 so routing and outputs are comparable
    at the fp32 tolerance."""
    grid = (4, 8, 16)
    B, H, D = 1, 2, 64
    T = 4 * 8 * 16
    say(f"[gpu] operator with Morton reorder: grid {grid}")
    x = [make_x(B, T, H, D, "f32", seed=s) for s in (1, 2, 3)]
    o = P.piecewise_sparse_attention(*x, density=0.25, reorder="morton", grid=grid)
    torch.cuda.synchronize()
    perm = R.z_order(grid)
    qh, kh, vh = (R.gather_head_major(t.double().cpu().numpy(), perm) for t in x)
    N = -(-T // 64)
    topk = int(np.floor(0.25 * N))
    ref = np.stack([np.stack([O.pisa_forward_head(qh[b, h], kh[b, h], vh[b, h], B=64, topk=topk, band=1)
                              for h in range(H)]) for b in range(B)])
    ref_tm = R.scatter_token_major(ref, perm)
    got = o.double().cpu().numpy()
    for h in range(H):
        err = np.abs(got[:, :, h] - ref_tm[:, :, h]).max() / np.abs(ref_tm[:, :, h]).max()
        assert err <= 1e-5, (h, err)
