"""GPU parity of pisa_attn_bwd (through the C ABI) against the float64
gradient oracle (oracle/backward_oracle.py), fed the GPU's routing.

Tolerances, per head and per gradient, on e = max|g - g_ref| / max|g_ref|:
* fp32 inputs: e <= 2e-5. Every gradient element is an fp32 sum of at most
  a few thousand products whose terms are bounded by max|g_ref| times the
  attention weight of their pair; the weights of a row sum to 1, so a sum's
  rounding stays within about sqrt(n) u ~ 4e-6 of max|g_ref| (u = 2^-24,
  n <= T), and the forward's o (itself within 1e-5 relative) enters only
  through delta = dout . o.
* bf16 inputs: e <= 2e-2. The gradients are rounded once to bf16 (relative
  2^-9), and delta uses the bf16 output of the MFMA forward, whose P is
  rounded to bf16 (the forward's own bar is 2e-2 absolute on o).
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from block_sparse_taylor_amd import inputs as I
from oracle import backward_oracle as BO

from gpu_common import say, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 2e-2}


def device_case(w, seed):
    qa, ka, va = I.make_inputs(w)
    r = np.random.default_rng(seed)
    da = r.standard_normal(qa.shape).astype(np.float32)
    if w.dtype == "bf16":
        da = I.bf16_bits(da)
    host = [I.as_f64(a, w.dtype) for a in (qa, ka, va, da)]
    return [to_device(a, w.dtype) for a in (qa, ka, va, da)], host


def check(w, seed, topk, band=1, n_sink=0, so=False, fo=True, idx_fn=None, valu_fwd=False):
    say(f"[gpu] bwd case: {w.name} T={w.seq_len} D={w.head_dim} {w.dtype} heads={w.heads} topk={topk} "
        f"band={band} sinks={n_sink} so={so} fo={fo} seed={seed}")
    (q, k, v, do), host = device_case(w, seed)
    s = 1.0 / math.sqrt(w.head_dim)
    st = P.pisa_block_stats(q, k, v, second_order=so)
    idx, wg = P.pisa_route_topk(q, st, topk, band=band, second_order=so, n_sink=n_sink)
    if idx_fn is not None:
        idx = idx_fn(idx)
    fwd = P.pisa_attn_fwd_valu if valu_fwd else P.pisa_attn_fwd
    o = fwd(q, k, v, st, idx, wg, band=band, second_order=so, first_order=fo, n_sink=n_sink)
    dq, dk, dv = P.pisa_attn_bwd(q, k, v, o, do, st, idx, wg, band=band, second_order=so, first_order=fo,
                                 n_sink=n_sink)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in (dq, dk, dv)]
    ih = None if idx is None else idx.cpu().numpy()
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            qh, kh, vh, dh = (x[b, h] for x in host)
            N = -(-w.seq_len // 64)
            table = ih[b, h] if ih is not None else np.full((N, 1), -1, np.int32)
            ref = BO.grads(qh, kh, vh, dh, table, B=64, scale=s, band=band, n_sink=n_sink,
                           second_order=so, first_order=fo)
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                e = np.abs(g[b, h] - r).max() / np.abs(r).max()
                worst = max(worst, e)
                assert e <= TOL[w.dtype], (name, b, h, e)
    say(f"[gpu]   worst normalised error {worst:.2e}")
    return worst


def wl(base, **kw):
    return dataclasses.replace(I.WORKLOADS[base], **kw)


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_first_order(D):
    check(wl("tiny", seq_len=1000, head_dim=D, heads=2), seed=1, topk=3)


def test_fp32_second_order_sinks_band0():
    check(wl("tiny", seq_len=777, head_dim=128, heads=2), seed=2, topk=2, band=0, n_sink=1, so=True)


def test_fp32_zeroth_order_second_order():
    check(wl("tiny", seq_len=1100, head_dim=64, heads=1, batch=2), seed=3, topk=4, so=True, fo=False)


@pytest.mark.parametrize("so", [False, True])
def test_bf16_video(so):
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023, outlier_key_dims=(0, 1))
    check(w, seed=4, topk=2, so=so)


def test_bf16_d64_zeroth_order_vs_valu_forward():
    w = wl("flux", heads=2, grid=(30, 32), seq_len=1472, text_tokens=512, head_dim=64)
    check(w, seed=5, topk=3, n_sink=2, fo=False, valu_fwd=True)


def test_single_partial_block():
    check(wl("tiny", seq_len=50, head_dim=64, heads=2), seed=6, topk=0)


def test_no_routing_all_virtual_but_band():
    check(wl("tiny", seq_len=700, head_dim=64, heads=1), seed=7, topk=0, band=0, so=True)


def test_routing_with_invalid_ids_and_padding():
    def mangle(idx):
        x = idx.clone()
        x[..., 0] = -7           # invalid: ignored like -1
        x[..., -1] = 10 ** 6     # out of range: ignored
        return x
    check(wl("tiny", seq_len=900, head_dim=64, heads=2), seed=8, topk=4, idx_fn=mangle)


def test_every_block_exact():
    w = wl("tiny", seq_len=640, head_dim=128, heads=1)
    check(w, seed=9, topk=8, band=1)   # N = 10: every candidate routed


def test_deterministic():
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023)
    (q, k, v, do), _ = device_case(w, 10)
    st = P.pisa_block_stats(q, k, v, second_order=True)
    idx, wg = P.pisa_route_topk(q, st, 3, band=1, second_order=True)
    o = P.pisa_attn_fwd(q, k, v, st, idx, wg, second_order=True)
    a = P.pisa_attn_bwd(q, k, v, o, do, st, idx, wg, second_order=True)
    b = P.pisa_attn_bwd(q, k, v, o, do, st, idx, wg, second_order=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
