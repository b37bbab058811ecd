"""fp32 inputs: pisa_attn_fwd runs the fp32 matrix-core kernel (every
product on v_mfma_f32_16x16x4_f32, P and the virtual tokens' k-bar, V-hat in
fp32). Checked element by element against the fp64 oracle fed the GPU's
routing, to the fp32 bar max|o - o_ref| / max|o_ref| <= 1e-5 per head, on
shapes that span several query blocks, virtual-token groups and a ragged last
block; and against the fp32 vector kernel (pisa_attn_fwd_valu)."""

import math

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from oracle import pisa_oracle as O

from gpu_common import say

pytestmark = pytest.mark.gpu

F32_KERNEL = 3   # PISA_KERNEL_MFMA_F32


def make(B, H, T, D, seed, kscale=1.0):
    r = np.random.default_rng(seed)
    x = [r.standard_normal((B, H, T, D)) for _ in range(3)]
    x[1] *= kscale
    dev = [torch.from_numpy(a).to(torch.float32).cuda().contiguous() for a in x]
    host = [t.double().cpu().numpy() for t in dev]   # the exact values the GPU sees
    return dev, host


CASES = [   # B, H, T, D, topk, band, n_sink, second_order, kscale
    (1, 2, 1024, 64, 4, 1, 0, False, 1.0),      # the Tiny configuration's shape
    (1, 2, 4100, 128, 6, 1, 0, False, 1.0),     # 65 blocks: two virtual groups, 4-row tail
    (2, 3, 2500, 64, 5, 2, 0, True, 1.0),       # batch > 1, second order, ragged
    (1, 2, 3000, 128, 3, 1, 2, True, 1.0),      # sinks with the second order
    (1, 1, 640, 128, 10, 1, 0, False, 1.0),     # every block exact (density 1)
    (1, 2, 2048, 128, 4, 0, 0, False, 3.0),     # no band, wide logit range (rescaling)
    (1, 2, 1000, 64, 0, 1, 0, True, 2.0),       # no routed ids: band plus virtual tokens only
]


@pytest.mark.parametrize("B,H,T,D,topk,band,n_sink,so,kscale", CASES)
def test_f32_matrix_core_kernel_matches_oracle(B, H, T, D, topk, band, n_sink, so, kscale):
    say(f"[gpu] f32 kernel B={B} H={H} T={T} D={D} topk={topk} band={band} sinks={n_sink} so={so} k*{kscale}")
    assert P.attn_fwd_plan(B, H, T, D, "f32", topk, band, so, n_sink) == F32_KERNEL
    (q, k, v), (qh, kh, vh) = make(B, H, T, D, T + 7 * D + topk, kscale)
    st = P.pisa_block_stats(q, k, v, second_order=so)
    idx, wg = P.pisa_route_topk(q, st, topk, band=band, second_order=so, n_sink=n_sink)
    rs = P.alloc_row_stats(q)
    o = P.pisa_attn_fwd(q, k, v, st, idx if topk else None, wg, band=band, second_order=so,
                        n_sink=n_sink, row_stats=rs)
    o_valu = P.pisa_attn_fwd_valu(q, k, v, st, idx if topk else None, wg, band=band, second_order=so,
                                  n_sink=n_sink)
    torch.cuda.synchronize()
    N = -(-T // 64)
    idx_h = idx.cpu().numpy() if topk else np.zeros((B, H, N, 0), np.int32)
    got, gv, rsh = o.double().cpu().numpy(), o_valu.double().cpu().numpy(), rs.double().cpu().numpy()
    worst, worst_v, worst_lse = 0.0, 0.0, 0.0
    for b in range(B):
        for h in range(H):
            ref, parts = O.pisa_forward_head(qh[b, h], kh[b, h], vh[b, h], topk=topk, band=band,
                                             second_order=so, n_sink=n_sink, routing=idx_h[b, h],
                                             return_parts=True)
            scale = np.abs(ref).max()
            e = np.abs(got[b, h] - ref).max() / scale
            ev = np.abs(gv[b, h] - ref).max() / scale
            worst, worst_v = max(worst, e), max(worst_v, ev)
            assert e <= 1e-5, (b, h, e)
            # the row statistics: lse = ln(den), c = l_tail / (T den); fp32 logits of
            # up to ~|q||k|/sqrt(D) carry ~1e-6 relative rounding each
            lse = parts["m"] + np.log(parts["den"])
            c = parts["l_tail"] / (T * parts["den"])
            el = np.abs(rsh[b, h, :, 0] - lse).max()
            worst_lse = max(worst_lse, el)
            assert el <= 2.5e-4, (b, h, el)
            assert np.abs(rsh[b, h, :, 1] - c).max() <= 5e-4 * max(1.0, np.abs(c).max())
    say(f"[gpu]   worst relative error: matrix-core {worst:.2e}, vector {worst_v:.2e}; lse {worst_lse:.2e}")
    assert np.abs(got - gv).max() / np.abs(gv).max() <= 2e-5


@pytest.mark.parametrize("D", [64, 128])
def test_f32_first_order_off_and_exact_phase(D):
    """first_order off ("-0th") and phase_mask 1 (exact blocks only, i.e.
    keep-or-drop block-sparse attention) on the fp32 kernel."""
    T = 1500
    say(f"[gpu] f32 kernel phases D={D}")
    (q, k, v), (qh, kh, vh) = make(1, 2, T, D, 11 + D)
    st = P.pisa_block_stats(q, k, v)
    idx, _ = P.pisa_route_topk(q, st, 3, band=1)
    o0 = P.pisa_attn_fwd(q, k, v, st, idx, None, band=1, first_order=False)
    o1 = P.pisa_attn_fwd(q, k, v, st, idx, None, band=1, phase_mask=1)
    torch.cuda.synchronize()
    ih = idx.cpu().numpy()
    for h in range(2):
        ref0 = O.pisa_forward_head(qh[0, h], kh[0, h], vh[0, h], topk=3, band=1, first_order="none",
                                   routing=ih[0, h])
        ref1 = O.pisa_forward_head(qh[0, h], kh[0, h], vh[0, h], topk=3, band=1, sparse_only=True,
                                   routing=ih[0, h])
        for out, ref in ((o0, ref0), (o1, ref1)):
            e = np.abs(out[0, h].double().cpu().numpy() - ref).max() / np.abs(ref).max()
            assert e <= 1e-5, e


def test_f32_kernel_deterministic():
    (q, k, v), _ = make(1, 2, 3333, 128, 5)
    st = P.pisa_block_stats(q, k, v, second_order=True)
    idx, wg = P.pisa_route_topk(q, st, 5, band=1, second_order=True)
    a = P.pisa_attn_fwd(q, k, v, st, idx, wg, band=1, second_order=True)
    b = P.pisa_attn_fwd(q, k, v, st, idx, wg, band=1, second_order=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert math.isfinite(float(a.abs().max()))
