"""GPU parity of pisa_attn_bwd (through the C ABI) against the float64
gradient oracle (oracle/backward_oracle.py), fed the GPU's routing.

Two kinds of case. End to end: the backward gets the GPU forward's o, and the
oracle returns the exact gradient. Contract: the backward gets the oracle's
own forward output rounded to the input dtype (o'), and the oracle returns
the gradient a backward computes when delta = dout . o' (grads(o_used=o')),
so only the backward's own arithmetic is measured.

Tolerances, per head and per gradient, on e = max|g - g_ref| / max|g_ref|:
* fp32 inputs: e <= 5e-5. Every gradient element is an fp32 sum of at most
  a few thousand products; the rounding of such a sum stays within about
  sqrt(n) u (u = 2^-24, n <= T: ~4e-6) of the sum of its terms' magnitudes.
  Those terms can exceed the result itself: dq_t = sum P (dP - delta) k is a
  covariance under P, while each term carries the full key, so |terms| /
  |dq| grows with |mean attended key| / |dq|. On the video-like inputs (keys
  sharing a smooth field, two key dims scaled by 8) that ratio reaches ~10,
  hence the bound; the i.i.d. cases stay near 1e-6.
* bf16, contract: e <= 4e-3: each gradient is rounded once to bf16 (at most
  2^-8 of its magnitude: bf16 keeps 8 significant bits), on top of the fp32
  arithmetic above.
* bf16, end to end: e <= 2e-2. delta = dout . o uses o stored in bf16, and a
  delta error c_t moves dq_t by -c_t s E_P[k] (dk likewise; dv not at all),
  which the mean key of an attended set can make larger than dq_t itself
  (the oracle module's pins give this closed form).
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from block_sparse_taylor_amd import inputs as I
from oracle import backward_oracle as BO
from oracle import pisa_oracle as O

from gpu_common import say, to_device

pytestmark = pytest.mark.gpu

TOL = {("f32", False): 5e-5, ("bf16", False): 2e-2, ("f32", True): 5e-5, ("bf16", True): 4e-3}


def device_case(w, seed):
    qa, ka, va = I.make_inputs(w)
    r = np.random.default_rng(seed)
    da = r.standard_normal(qa.shape).astype(np.float32)
    if w.dtype == "bf16":
        da = I.bf16_bits(da)
    host = [I.as_f64(a, w.dtype) for a in (qa, ka, va, da)]
    return [to_device(a, w.dtype) for a in (qa, ka, va, da)], host


def oracle_output(w, host, ih, s, band, n_sink, so, fo):
    """The oracle's forward [B,H,T,D] for the GPU's routing, rounded to the input dtype."""
    o = np.empty(host[0].shape)
    N = -(-w.seq_len // 64)
    for b in range(w.batch):
        for h in range(w.heads):
            qh, kh, vh = (x[b, h] for x in host[:3])
            table = ih[b, h] if ih is not None else np.full((N, 1), -1, np.int32)
            o[b, h] = O.pisa_forward_head(qh, kh, vh, B=64, scale=s, topk=table.shape[1], band=band,
                                          n_sink=n_sink, second_order=so,
                                          first_order="global" if fo else "none", routing=table)
    if w.dtype == "bf16":
        bits = I.bf16_bits(o.astype(np.float32))
        return to_device(bits, "bf16"), I.as_f64(bits, "bf16")
    o32 = o.astype(np.float32)
    return to_device(o32, "f32"), o32.astype(np.float64)


def check(w, seed, topk, band=1, n_sink=0, so=False, fo=True, idx_fn=None, valu_fwd=False, contract=False,
          row_stats=False):
    say(f"[gpu] bwd case: {w.name} T={w.seq_len} D={w.head_dim} {w.dtype} heads={w.heads} topk={topk} "
        f"band={band} sinks={n_sink} so={so} fo={fo} seed={seed} contract={contract} row_stats={row_stats}")
    assert not (row_stats and contract), "the row statistics come from the GPU forward"
    (q, k, v, do), host = device_case(w, seed)
    s = 1.0 / math.sqrt(w.head_dim)
    st = P.pisa_block_stats(q, k, v, second_order=so)
    idx, wg = P.pisa_route_topk(q, st, topk, band=band, second_order=so, n_sink=n_sink)
    if idx_fn is not None:
        idx = idx_fn(idx)
    ih = None if idx is None else idx.cpu().numpy()
    o_used = None
    if contract:
        o, o_used = oracle_output(w, host, ih, s, band, n_sink, so, fo)
    rs = P.alloc_row_stats(q) if row_stats else None
    if not contract:
        fwd = P.pisa_attn_fwd_valu if valu_fwd else P.pisa_attn_fwd
        o = fwd(q, k, v, st, idx, wg, band=band, second_order=so, first_order=fo, n_sink=n_sink, row_stats=rs)
    dq, dk, dv = P.pisa_attn_bwd(q, k, v, o, do, st, idx, wg, band=band, second_order=so, first_order=fo,
                                 n_sink=n_sink, row_stats=rs)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in (dq, dk, dv)]
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.heads):
            qh, kh, vh, dh = (x[b, h] for x in host)
            N = -(-w.seq_len // 64)
            table = ih[b, h] if ih is not None else np.full((N, 1), -1, np.int32)
            ref = BO.grads(qh, kh, vh, dh, table, B=64, scale=s, band=band, n_sink=n_sink,
                           second_order=so, first_order=fo,
                           o_used=None if o_used is None else o_used[b, h])
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                e = np.abs(g[b, h] - r).max() / np.abs(r).max()
                worst = max(worst, e)
                assert e <= TOL[(w.dtype, contract)], (name, b, h, e)
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


@pytest.mark.parametrize("contract", [False, True])
@pytest.mark.parametrize("so", [False, True])
def test_bf16_video(so, contract):
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023, outlier_key_dims=(0, 1))
    check(w, seed=4, topk=2, so=so, contract=contract)


@pytest.mark.parametrize("so", [False, True])
def test_bf16_video_with_forward_row_stats(so):
    """End to end, the backward taking each row's lse and c from the forward
    (pisa_attn_fwd's row_stats) instead of re-scoring the row's pairs."""
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023, outlier_key_dims=(0, 1))
    check(w, seed=4, topk=2, so=so, row_stats=True)


def test_bf16_image_sinks_with_forward_row_stats():
    w = wl("flux", heads=2, grid=(30, 32), seq_len=1472, text_tokens=512)
    check(w, seed=12, topk=3, n_sink=8, so=True, row_stats=True)


def test_fp32_with_forward_row_stats():
    """fp32 inputs recompute the row statistics whether or not the forward's are passed."""
    check(wl("tiny", seq_len=777, head_dim=128, heads=2), seed=2, topk=2, band=0, n_sink=1, so=True,
          row_stats=True)


@pytest.mark.parametrize("kernel", ["asm", "mfma_d64", "valu_bf16", "f32"])
def test_forward_row_stats_match_oracle(kernel):
    """pisa_attn_fwd's row_stats against the oracle's per-row sums: lse_t =
    m_t + ln den_t and c_t = l_tail_t / (T den_t), on each forward kernel (the
    persistent and the non-persistent matrix-core kernel, the vector kernel
    on bf16 and on fp32 inputs), with sinks and the second order. The bf16
    matrix-core kernels sum bf16-rounded weights (each within 2^-8 of the
    exact one: bf16 keeps 8 significant bits), so den is within 2^-8
    relative: lse within ln(1 + 2^-8) = 3.9e-3, 4.5e-3 with the fp32 sums.
    They take l_tail as the row sum minus its value after the last exact
    item, so the fraction l_tail / den (= T c) is within 2^-7 of itself plus
    the fp32 rounding of the running sum, at most ~10^3 additions of 2^-24
    each: 1e-4 absolute. The vector kernels sum in fp32 without a difference;
    there the logits' own fp32 rounding decides: a 128-term dot product
    within 128 * 2^-24 of its terms' magnitude (logits up to ~30 on these
    inputs, two key dims scaled by 8), 2.5e-4 in lse and twice that,
    relative, in the ratio l_tail / den."""
    D = 64 if kernel == "mfma_d64" else 128
    dtype = "f32" if kernel == "f32" else "bf16"
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023, head_dim=D, dtype=dtype)
    (q, k, v, do), host = device_case(w, 20)
    st = P.pisa_block_stats(q, k, v, second_order=True)
    idx, wg = P.pisa_route_topk(q, st, 3, band=1, second_order=True, n_sink=1)
    want_kernel = {"asm": 1, "mfma_d64": 2, "valu_bf16": None, "f32": 3}[kernel]
    if want_kernel is not None:
        assert P.attn_fwd_plan(1, 2, w.seq_len, D, dtype, 3, 1, True, 1) == want_kernel
    rs = P.alloc_row_stats(q)
    fwd = P.pisa_attn_fwd_valu if kernel == "valu_bf16" else P.pisa_attn_fwd
    o = fwd(q, k, v, st, idx, wg, band=1, second_order=True, n_sink=1, row_stats=rs)
    o_plain = fwd(q, k, v, st, idx, wg, band=1, second_order=True, n_sink=1)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)   # the extra output changes nothing else
    got = rs.double().cpu().numpy()
    ih = idx.cpu().numpy()
    exact = kernel in ("asm", "mfma_d64")
    tl, tc = (4.5e-3, 2.0 ** -7) if exact else (2.5e-4, 5e-4)
    worst = [0.0, 0.0]
    for h in range(2):
        qh, kh, vh = (x[0, h] for x in host[:3])
        _, parts = O.pisa_forward_head(qh, kh, vh, B=64, scale=1 / math.sqrt(D), topk=3, band=1, n_sink=1,
                                       second_order=True, routing=ih[0, h], return_parts=True)
        lse = parts["m"] + np.log(parts["den"])
        c = parts["l_tail"] / (w.seq_len * parts["den"])
        el = np.abs(got[0, h, :, 0] - lse).max()
        frac_got, frac = w.seq_len * got[0, h, :, 1], w.seq_len * c   # l_tail / den
        ec = np.abs(frac_got - frac)
        worst = [max(worst[0], el), max(worst[1], float(ec.max()))]
        assert el <= tl, (h, el)
        assert bool(np.all(ec <= tc * frac + (1e-4 if exact else 0.0))), (h, float((ec - tc * frac).max()))
    say(f"[gpu]   {kernel}: lse worst abs error {worst[0]:.2e}, l_tail/den worst abs error {worst[1]:.2e}")


def test_fp32_video_contract():
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023, dtype="f32")
    check(w, seed=11, topk=3, so=True, n_sink=1, contract=True)


def test_bf16_image_sinks_contract():
    w = wl("flux", heads=2, grid=(30, 32), seq_len=1472, text_tokens=512)
    check(w, seed=12, topk=3, n_sink=8, so=True, contract=True)


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


def test_bf16_query_blocks_beyond_one_chunk():
    """N = 301: the dk/dv kernel gathers the query blocks that hold a KV block
    exactly 256 at a time (one mask word per thread, a ballot per wave), so a
    column spans two chunks. Every query block is also routed to block 5
    (where that is not already so), so block 5's column has every bit set,
    bit 31 of each 32-block word included (a word taken as signed would set
    the upper half of its 64-bit pair)."""
    w = wl("wan14", heads=1, grid=(7, 41, 67), seq_len=19229)

    def force5(idx):
        x = idx.cpu().clone()
        for i in range(x.shape[2]):
            row = x[0, 0, i]
            if abs(i - 5) > 1 and not bool((row == 5).any()):
                row[0] = 5
        return x.to(idx.device)
    check(w, seed=14, topk=6, idx_fn=force5)


def test_bf16_bit31_of_mask_words_routed_contract():
    """N = 100: every query block is routed to blocks 31 and 95, bit 31 of
    the first mask word of virtual-token groups 0 and 1 (the virtual-token
    kernel joins a group's two 32-bit words into one 64-bit selection; a
    word taken as signed would mark the group's upper 32 blocks exact and
    drop their virtual-token gradients)."""
    w = wl("tiny", seq_len=64 * 100, head_dim=128, heads=1, dtype="bf16")

    def force(idx):
        x = idx.cpu().clone()
        for i in range(x.shape[2]):
            row = x[0, 0, i]
            for slot, j in enumerate((31, 95)):
                if abs(i - j) > 1 and not bool((row == j).any()):
                    row[slot] = j
        return x.to(idx.device)
    check(w, seed=21, topk=4, idx_fn=force, contract=True)


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


@pytest.mark.parametrize("name,heads,dkdv_head", [("wan14", (3, 29), 3), ("hunyuan", (5, 17), None)])
def test_full_size(name, heads, dkdv_head):
    """A workload of the bench in its launch configuration (every head, one
    call: the Wan2.1-14B shape, T = 32760; the Hunyuan shape, T = 118800 with
    the second order). Checked: dq of sampled query blocks of two heads
    against the oracle one block at a time (end-to-end bf16 bar), and two
    invariances that hold at any size: shifting every key by one vector
    shifts all logits of a row equally (H, the key variance and the pooled q^2
    do not change), so sum_k dk = 0; shifting every value by one vector shifts
    every output by it (H does not change since sum (k - kbar) = 0 per
    block), so sum_k dv = sum_t dout_t. Both sums are compared within 2^-7 of
    sum |.| (bf16 rounding of each term, 2^-8, with fp32 accumulation).
    At the Wan2.1-14B shape one head's dk and dv are also compared element
    by element on sampled KV blocks with the oracle's full-head gradient for
    the o the backward was handed (the contract bar): a KV block's gradient
    collects every query block that attends to it exactly and, through the
    block mean, V-hat and H, every query block, so it needs the whole head
    (about half a minute of float64 autograd on the host)."""
    from gpu_common import head_f64, oracle_topk, workload_inputs
    say(f"[gpu] bwd full size {name}: inputs")
    w, arrs = workload_inputs(name)
    so = w.second_order
    say(f"[gpu] bwd full size {name}: {w.batch}x{w.heads}x{w.seq_len}x{w.head_dim} {w.dtype} second_order={so}")
    q, k, v = (to_device(a, w.dtype) for a in arrs)
    r = np.random.default_rng(13)
    dbits = I.bf16_bits(r.standard_normal(arrs[0].shape, dtype=np.float32))
    do = to_device(dbits, "bf16")
    s = 1.0 / math.sqrt(w.head_dim)
    N = -(-w.seq_len // 64)
    topk = oracle_topk(w.density, N)
    st = P.pisa_block_stats(q, k, v, second_order=so)
    idx, wg = P.pisa_route_topk(q, st, topk, band=w.band, second_order=so)
    o = P.pisa_attn_fwd(q, k, v, st, idx, wg, band=w.band, second_order=so)
    dq, dk, dv = P.pisa_attn_bwd(q, k, v, o, do, st, idx, wg, band=w.band, second_order=so)
    torch.cuda.synchronize()
    say("[gpu]   backward done")
    # with the forward's row statistics: the same o, and gradients within
    # the bf16 weights' 2^-8 (uniformly scaling a row's weights by 1 + e
    # scales its terms of every gradient by 1 + e) plus the two gradients'
    # own bf16 rounding (2^-8 each) of the recomputed ones: 3 * 2^-8
    rs = P.alloc_row_stats(q)
    o_rs = P.pisa_attn_fwd(q, k, v, st, idx, wg, band=w.band, second_order=so, row_stats=rs)
    g_rs = P.pisa_attn_bwd(q, k, v, o_rs, do, st, idx, wg, band=w.band, second_order=so, row_stats=rs)
    torch.cuda.synchronize()
    assert torch.equal(o_rs, o)
    for nm, a, b in zip(("dq", "dk", "dv"), g_rs, (dq, dk, dv)):
        e = float((a.float() - b.float()).abs().max() / b.float().abs().max())
        say(f"[gpu]   {nm} with the forward's row statistics vs recomputed: {e:.2e} of max")
        assert e <= 3 * 2.0 ** -8, (nm, e)
    del o_rs, g_rs, rs
    dkf, dvf, dof = dk.float(), dv.float(), do.float()
    for nm, lhs, ref, mag in (("dk", dkf.sum(2), torch.zeros_like(dkf[:, :, 0]), dkf.abs().sum(2)),
                              ("dv", dvf.sum(2), dof.sum(2), dvf.abs().sum(2))):
        err = (lhs - ref).abs()
        assert bool(torch.all(err <= 2.0 ** -7 * mag)), (nm, float((err / mag).max()))
    del dkf, dvf, dof
    ih = idx.cpu().numpy()
    for h in heads:
        qh, kh, vh = head_f64(arrs, w.dtype, 0, h)
        doh = I.as_f64(dbits[0, h], "bf16")
        blocks = [0, int(r.integers(1, N - 1)), int(r.integers(1, N - 1)), N - 1]
        ref = BO.grads_q_blocks(qh, kh, vh, doh, ih[0, h], blocks, B=64, scale=s, band=w.band, second_order=so)
        rows = np.concatenate([np.arange(64 * i, min(w.seq_len, 64 * i + 64)) for i in blocks])
        got = dq[0, h].double().cpu().numpy()[rows]
        e = np.abs(got - ref).max() / np.abs(ref).max()
        say(f"[gpu]   head {h} blocks {blocks}: dq normalised error {e:.2e}")
        assert e <= TOL[("bf16", False)], (h, blocks, e)
    if dkdv_head is not None:
        h = dkdv_head
        qh, kh, vh = head_f64(arrs, w.dtype, 0, h)
        doh = I.as_f64(dbits[0, h], "bf16")
        oh = o[0, h].double().cpu().numpy()
        say(f"[gpu]   head {h}: full-head gradient oracle for dk, dv")
        _, rdk, rdv = BO.grads(qh, kh, vh, doh, ih[0, h], o_used=oh, B=64, scale=s, band=w.band, second_order=so)
        kvb = [0, 1, int(r.integers(2, N - 2)), int(r.integers(2, N - 2)), N - 2, N - 1]
        rows = np.concatenate([np.arange(64 * j, min(w.seq_len, 64 * j + 64)) for j in kvb])
        for nm, got_t, ref in (("dk", dk, rdk), ("dv", dv, rdv)):
            got = got_t[0, h].double().cpu().numpy()[rows]
            e = np.abs(got - ref[rows]).max() / np.abs(ref[rows]).max()
            say(f"[gpu]   head {h} KV blocks {kvb}: {nm} normalised error {e:.2e}")
            assert e <= TOL[("bf16", True)], (nm, h, kvb, e)


def test_bf16_single_block_of_twenty_rows_contract():
    """One partial block of 20 rows: the exact keys all sit in the first
    32-key half of the tile (the other half of the kernels' waves sees none)."""
    check(wl("tiny", seq_len=20, head_dim=128, heads=2, dtype="bf16"), seed=14, topk=0, contract=True)


def test_bf16_last_block_partial_band0_contract():
    """band 0, no routing: the last query block (25 rows) has only its own
    partial block exact; every other block is a virtual token."""
    check(wl("tiny", seq_len=64 * 6 + 25, head_dim=64, heads=2, dtype="bf16"), seed=15, topk=0, band=0,
          so=True, contract=True)


def test_bf16_d64_second_order_sinks_contract():
    w = wl("flux", heads=2, grid=(30, 32), seq_len=1472, text_tokens=512, head_dim=64)
    check(w, seed=16, topk=2, n_sink=3, so=True, contract=True)


def test_bf16_many_groups_contract():
    """N = 131 blocks: three groups of 64 virtual tokens, the last holding 3."""
    check(wl("tiny", seq_len=64 * 130 + 7, head_dim=128, heads=1, dtype="bf16"), seed=17, topk=5, so=True,
          n_sink=1, contract=True)


def test_bf16_two_batches_contract():
    """batch 2 x 3 heads: the kernels index (batch, head) pairs as one axis."""
    w = wl("wan14", batch=2, heads=3, grid=(3, 11, 31), seq_len=1023)
    check(w, seed=18, topk=3, so=True, n_sink=1, contract=True)


@pytest.mark.parametrize("reorder", ["none", "morton"])
def test_autograd_through_the_wrapper(reorder):
    """piecewise_sparse_attention is differentiable: its gradients equal
    pisa_attn_bwd's on the same routing, given the forward's row statistics,
    bit for bit (through the Morton reorder, whose adjoint is the inverse
    reorder)."""
    w = wl("wan14", heads=2, grid=(3, 11, 31), seq_len=1023)
    (q, k, v, do), _ = device_case(w, 19)
    say(f"[gpu] autograd through piecewise_sparse_attention, reorder={reorder}")
    if reorder == "morton":
        perm = P.z_order(w.grid).cuda()
        q, k, v, do = (P.reorder_scatter(t, perm) for t in (q, k, v, do))   # token-major raster inputs
    leaves = [t.detach().clone().requires_grad_(True) for t in (q, k, v)]
    kw = dict(density=0.25, variant="pwt", n_sink_blocks=1, reorder=reorder)
    if reorder == "morton":
        kw["grid"] = w.grid
    o = P.piecewise_sparse_attention(*leaves, **kw)
    o.backward(do)
    # the same computation through the entry points
    qq, kk, vv, dd = q, k, v, do
    if reorder == "morton":
        qq, kk, vv, dd = (P.reorder_gather(t, perm) for t in (q, k, v, do))
    N = P.num_blocks(w.seq_len)
    topk = P.topk_for_density(0.25, N)
    st = P.pisa_block_stats(qq, kk, vv, second_order=True)
    idx, wg = P.pisa_route_topk(qq, st, topk, band=1, second_order=True, n_sink=1)
    rs = P.alloc_row_stats(qq)
    oo = P.pisa_attn_fwd(qq, kk, vv, st, idx, wg, second_order=True, n_sink=1, row_stats=rs)
    grads = P.pisa_attn_bwd(qq, kk, vv, oo, dd, st, idx, wg, second_order=True, n_sink=1, row_stats=rs)
    if reorder == "morton":
        grads = [P.reorder_scatter(g, perm) for g in grads]
    torch.cuda.synchronize()
    for leaf, g in zip(leaves, grads):
        assert torch.equal(leaf.grad, g)
