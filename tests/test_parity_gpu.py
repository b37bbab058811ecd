"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (from the operator's specification and the arithmetic):
* routing: block-id sets identical; a difference is accepted only where the
  oracle's score gap to the k-th candidate is below 1e-6, and is reported.
* fp32 inputs: per head max|o - o_ref| / max|o_ref| <= 1e-5.
* bf16 inputs: max|o - o_ref| <= 2e-2, the oracle fed the GPU's routing.
* gated second-order table: the gate decision equals float64's; kept values
  within the fp32 dot-product bound 2 (D + 4) u w.
* statistics: qbar/kbar bit-exact (exact fp64 sums), ksig2 to 1e-12; the
  packed copy of K bit-exact (a re-ordering); packed H the exact bf16 hi/lo
  split of the returned hsum; V-hat is the fp64 sum
  rounded once to fp32; the bf16 copies are bit-exact roundings; H within
  64 u sum_t |k_ta||v_tb| elementwise (u = 2^-24; fp32 accumulation of
  bf16 products over block-range partials of at most 5.7K rows, 16 products
  per MFMA step, so about 360 rounded additions per partial: a sqrt(n) u
  growth of ~19 u, and the partials are summed in fp64).
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_taylor_amd as P
from block_sparse_taylor_amd import inputs as I
from oracle import pisa_oracle as O

from gpu_common import bf16_round_f32, head_f64, n_blocks, oracle_topk, say, to_device, workload_inputs

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24

# heads checked in full per workload, and extra (head, query-block) samples
SAMPLES = {
    "tiny": dict(heads=None, extra=0),
    "flux": dict(heads=None, extra=0),
    "wan13": dict(heads=[0, 7], extra=24),
    "wan14": dict(heads=[3], extra=32),
    "hunyuan": dict(heads=[], extra=48),
}
WORKLOAD_ORDER = ["tiny", "flux", "wan13", "wan14", "hunyuan"]


class Run:
    """One full-size run of the three calls on a workload, kept for the tests."""

    def __init__(self, name):
        w, arrs = workload_inputs(name)
        self.w, self.arrs = w, arrs
        say(f"[gpu] workload {name}: {w.batch}x{w.heads}x{w.seq_len}x{w.head_dim} {w.dtype}")
        self.q, self.k, self.v = (to_device(a, w.dtype) for a in arrs)
        self.N = n_blocks(w.seq_len)
        self.topk = oracle_topk(w.density, self.N)
        self.st = P.pisa_block_stats(self.q, self.k, self.v, second_order=w.second_order)
        self.idx, self.wg = P.pisa_route_topk(self.q, self.st, self.topk, band=w.band,
                                              second_order=w.second_order)
        self.o = P.pisa_attn_fwd(self.q, self.k, self.v, self.st, self.idx, self.wg, band=w.band,
                                 second_order=w.second_order)
        torch.cuda.synchronize()
        say(f"[gpu] workload {name}: done")

    def host(self, t):
        return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


_runs = {}


def get_run(name):
    if name not in _runs:
        _runs.clear()
        _runs[name] = Run(name)
    return _runs[name]


def sample_plan(name, w, N):
    s = SAMPLES[name]
    full = list(range(w.heads)) if s["heads"] is None else s["heads"]
    r = np.random.default_rng(1234)
    extra = [(int(r.integers(w.heads)), int(r.integers(N))) for _ in range(s["extra"])]
    extra.append((w.heads - 1, N - 1))      # the ragged last block of the last head
    extra = [(h, i) for h, i in extra if h not in full]
    return full, extra


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_block_stats(name):
    run = get_run(name)
    w = run.w
    full, extra = sample_plan(name, w, run.N)
    heads = sorted(set(full) | {h for h, _ in extra})
    say(f"[gpu] stats parity {name} heads {heads[:8]}...")
    kbar = run.st.kbar.cpu().numpy()
    qbar = run.st.qbar.cpu().numpy()
    q2bar = run.st.q2bar.cpu().numpy() if w.second_order else None
    vsum = run.st.vsum.cpu().numpy()
    hsum = run.st.hsum.cpu().numpy()
    ks2 = run.st.ksig2.cpu().numpy() if w.second_order else None
    # the kernels' arrangements inside the operand buffer
    B, H, D, N = w.batch, w.heads, w.head_dim, run.N
    ops = P.operand_views(run.st, run.k)
    view = lambda name, *shape: ops[name][:math.prod(shape)].reshape(shape)
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    kbc = run.host(view("kbar_c", B, H, N, D))
    vbc = run.host(view("vbar_c", B, H, N, D))
    kp = bits(view("kpack", B, H, N, 64 * D)) if w.dtype == "bf16" else None
    hp = run.host(view("hpack", B, H, 2 * D * D)) if w.dtype == "bf16" else None
    kbp = bits(view("kbpack", B, H, -(-N // 64), 64 * D)) if w.dtype == "bf16" else None
    kbb = bits(view("kbar_c", B, H, N, D)) if w.dtype == "bf16" else None
    NC = -(-N // 16)
    kbr = bits(view("kbar_r", B, H, NC * 16 * D * 2))
    ksr = bits(view("ksig2_r", B, H, NC * 16 * D * 2)) if w.second_order else None
    knr = view("knorm", B, H, NC * 16).cpu().numpy()
    def router_order(x):
        # split into bf16 hi = rn(x), lo = rn(x - hi); per 16-key chunk c,
        # k-step s < D/32 and part p, 64 lanes (g = dim quarter, n = key) of 8
        # dims (D/4) g + 8 s + e
        xp = np.zeros((NC * 16, D))
        xp[:N] = x
        hi = I.bf16_bits(xp)
        lo = I.bf16_bits(xp - I.bf16_to_f64(hi))
        arr = np.stack([hi, lo]).reshape(2, NC, 16, 4, D // 32, 8)      # p, c, n, g, s, e
        return arr.transpose(1, 4, 0, 3, 2, 5)                          # c, s, p, g, n, e
    valid = (np.arange(NC * 16) < N).reshape(NC, 16)[:, None, None, None, :, None]
    for h in heads:
        want_r = router_order(kbar[0, h])
        got_r = kbr[0, h].reshape(want_r.shape)
        assert np.array_equal(np.where(valid, got_r, 0), np.where(valid, want_r, 0)), h
        if ksr is not None:
            want_s = router_order(ks2[0, h])
            assert np.array_equal(np.where(valid, ksr[0, h].reshape(want_s.shape), 0), np.where(valid, want_s, 0)), h
        # the key norms bound ||kbar_j|| from above, within 2e-6
        nrm = np.sqrt((kbar[0, h] ** 2).sum(axis=1))
        kn = knr[0, h][:N].astype(np.float64)
        assert (kn >= nrm).all() and (kn <= nrm * (1 + 2e-6) + 1e-30).all(), h
        if kp is not None:
            # packed K is a pure re-ordering of k's bits: per block and 32-row
            # half, 16-byte chunks chunk-major, then row; zero rows past T
            kb = np.zeros((run.N * 64, w.head_dim), np.uint16)
            kb[:w.seq_len] = run.arrs[1][0, h]
            want = kb.reshape(run.N, 2, 32, w.head_dim // 8, 8).transpose(0, 1, 3, 2, 4).reshape(run.N, -1)
            assert np.array_equal(kp[0, h], want), h
            # packed H: hsum split into bf16 hi + lo (exact roundings), operand order
            D = w.head_dim
            hf = hsum[0, h].astype(np.float32)
            hi = bf16_round_f32(hf)
            lo = bf16_round_f32(hf - hi)
            parts = np.stack([hi, lo])                                  # [p, a, b]
            a = 16 * np.arange(D // 16)[:, None, None] + 8 * (np.arange(64) // 32)[None, :, None] + np.arange(8)[None, None, :]
            want_h = np.empty((D // 32, D // 16, 2, 64, 8), np.float32)
            for dt in range(D // 32):
                bcol = 32 * dt + np.arange(64) % 32
                for p in range(2):
                    want_h[dt, :, p] = parts[p][a, bcol[None, :, None]]
            assert np.array_equal(hp[0, h].reshape(want_h.shape), want_h), h
            # packed virtual keys: kbar_c rows per group of 64 blocks, kpack's order, zero past N
            GV = -(-run.N // 64)
            kc = np.zeros((GV * 64, D), np.uint16)
            kc[:run.N] = kbb[0, h]
            want_kb = kc.reshape(GV, 2, 32, D // 8, 8).transpose(0, 1, 3, 2, 4).reshape(GV, -1)
            assert np.array_equal(kbp[0, h], want_kb), h
        q, k, v = head_f64(run.arrs, w.dtype, 0, h)
        ref = O.kv_block_stats(k, v, 64)
        rq, rq2 = O.pool_queries(q, 64, 1 / math.sqrt(w.head_dim))
        # exact fp64 sums of exact inputs: the means agree bit for bit
        assert np.array_equal(kbar[0, h], ref.kbar)
        assert np.array_equal(qbar[0, h], rq)
        if q2bar is not None:
            np.testing.assert_allclose(q2bar[0, h], rq2, rtol=1e-14, atol=0)
        np.testing.assert_allclose(vsum[0, h], ref.vsum.astype(np.float32), rtol=2 * U32, atol=1e-30)
        if ks2 is not None:
            np.testing.assert_allclose(ks2[0, h], ref.sig2, rtol=1e-12, atol=1e-13)
        # the virtual tokens' values: the stored fp32 V-hat over n, rounded to fp32, then the dtype
        vbar_ref = (vsum[0, h].astype(np.float64) / ref.n[:, None]).astype(np.float32).astype(np.float64)
        if w.dtype == "bf16":
            assert np.array_equal(kbc[0, h], bf16_round_f32(ref.kbar))
            assert np.array_equal(vbc[0, h], bf16_round_f32(vbar_ref))
        else:
            np.testing.assert_allclose(kbc[0, h], ref.kbar.astype(np.float32), rtol=U32, atol=0)
            assert np.array_equal(vbc[0, h], vbar_ref)
        mag = np.abs(k).T @ np.abs(v)
        err = np.abs(hsum[0, h] - ref.H)
        assert (err <= 64 * U32 * mag + 1e-30).all(), (h, float((err / mag).max()))


@pytest.mark.parametrize("second_order", [False, True])
def test_block_stats_bf16_d64_ragged(second_order):
    """The bf16 statistics kernel at D = 64 (the bench workloads are D = 128),
    2 heads, T = 64 * 45 + 23 (a 23-row last block), keys and values with
    per-dimension offsets so that H and the variances are far from zero:
    block means bit-identical to float64, V-hat to fp32 rounding, H within
    64 fp32 ulps of sum |k| |v|, q'^2 and sigma^2 to 1e-14 / 1e-12, and the
    key norms bounding ||kbar_j|| from above within 2e-6."""
    T, D, H = 64 * 45 + 23, 64, 2
    N = -(-T // 64)
    say(f"[gpu] stats parity bf16 D=64 T={T} so={second_order}")
    r = np.random.default_rng(64 + second_order)
    off = r.standard_normal(D)
    q = r.standard_normal((1, H, T, D))
    k = r.standard_normal((1, H, T, D)) + off
    v = 0.5 * r.standard_normal((1, H, T, D)) - off
    dev = [torch.from_numpy(a).to(torch.bfloat16).cuda().contiguous() for a in (q, k, v)]
    host = [t.double().cpu().numpy() for t in dev]   # the exact values the GPU sees
    st = P.pisa_block_stats(*dev, second_order=second_order)
    torch.cuda.synchronize()
    ops = P.operand_views(st, dev[1])
    NC = -(-N // 16)
    knr = ops["knorm"][:H * NC * 16].reshape(1, H, NC * 16).cpu().numpy()
    s = 1 / math.sqrt(D)
    for h in range(H):
        qh, kh, vh = (x[0, h] for x in host)
        ref = O.kv_block_stats(kh, vh, 64)
        rq, rq2 = O.pool_queries(qh, 64, s)
        assert np.array_equal(st.kbar[0, h].cpu().numpy(), ref.kbar), h
        assert np.array_equal(st.qbar[0, h].cpu().numpy(), rq), h
        np.testing.assert_allclose(st.vsum[0, h].cpu().numpy(), ref.vsum.astype(np.float32), rtol=2 * U32, atol=1e-30)
        mag = np.abs(kh).T @ np.abs(vh)
        err = np.abs(st.hsum[0, h].cpu().numpy() - ref.H)
        assert (err <= 64 * U32 * mag + 1e-30).all(), (h, float((err / mag).max()))
        if second_order:
            np.testing.assert_allclose(st.q2bar[0, h].cpu().numpy(), rq2, rtol=1e-14, atol=0)
            np.testing.assert_allclose(st.ksig2[0, h].cpu().numpy(), ref.sig2, rtol=1e-12, atol=1e-13)
        nrm = np.sqrt((ref.kbar ** 2).sum(axis=1))
        kn = knr[0, h][:N].astype(np.float64)
        assert (kn >= nrm).all() and (kn <= nrm * (1 + 2e-6) + 1e-30).all(), h


def check_routing(name, run, heads):
    w = run.w
    idx = run.idx.cpu().numpy()
    scale = 1 / math.sqrt(w.head_dim)
    diffs = 0
    for h in heads:
        q, k, v = head_f64(run.arrs, w.dtype, 0, h)
        st = O.kv_block_stats(k, v, 64)
        qbar, q2bar = O.pool_queries(q, 64, scale)
        wr = O.second_order_w(q2bar, st.sig2, 64)[2] if w.second_order else None
        ref, r = O.route_topk(qbar, st.kbar, scale, run.topk, w.band, wr)
        got = idx[0, h]
        for i in range(run.N):
            if np.array_equal(got[i], ref[i]):
                continue
            gs = set(got[i][got[i] >= 0].tolist())
            rs = set(ref[i][ref[i] >= 0].tolist())
            assert len(gs) == len(rs) and sorted(gs) == got[i][got[i] >= 0].tolist(), (h, i)
            kth = min(r[i, j] for j in rs)
            for j in gs ^ rs:
                assert abs(r[i, j] - kth) < 1e-6, (h, i, j, r[i, j], kth)
            diffs += len(gs - rs)
    return diffs


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_route_topk(name):
    run = get_run(name)
    w = run.w
    heads = list(range(w.heads))      # every head of every workload
    say(f"[gpu] routing parity {name}: all {len(heads)} heads")
    diffs = check_routing(name, run, heads)
    say(f"[gpu] routing {name}: {diffs} near-tie differences over {len(heads)} heads x {run.N} rows")
    if w.second_order:
        wg = run.wg.cpu().numpy()
        lnB = math.log(64)
        scale = 1 / math.sqrt(w.head_dim)
        for h in heads[:2]:
            q, k, v = head_f64(run.arrs, w.dtype, 0, h)
            st = O.kv_block_stats(k, v, 64)
            _, q2bar = O.pool_queries(q, 64, scale)
            wraw, wgr, _ = O.second_order_w(q2bar, st.sig2, 64)
            # the gate decision equals the float64 one (the kernel re-decides in
            # fp64 within its fp32 error bound of ln B); kept values carry the
            # fp32 dot-product error 2 (D + 4) u w
            near = np.abs(wraw - lnB) < 1e-9
            gated = wraw > lnB
            assert ((wg[0, h] == 0) | ~gated | near).all()
            tol = 2 * (w.head_dim + 4) * U32 * wraw + 1e-30
            assert ((np.abs(wg[0, h] - wgr) <= tol) | gated | near).all()
            say(f"[gpu] head {h}: gated fraction {float((wraw > lnB).mean()):.4f}")


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_attn_fwd(name):
    run = get_run(name)
    w = run.w
    full, extra = sample_plan(name, w, run.N)
    idx = run.idx.cpu().numpy()
    o = run.host(run.o)
    worst = 0.0
    kw = dict(B=64, topk=run.topk, band=w.band, second_order=w.second_order)
    plan = [(h, None) for h in full]
    by_head = {}
    for h, i in extra:
        by_head.setdefault(h, []).append(i)
    plan += sorted(by_head.items())
    for h, blocks in plan:
        say(f"[gpu] attn parity {name} head {h} blocks {'all' if blocks is None else len(blocks)}")
        q, k, v = head_f64(run.arrs, w.dtype, 0, h)
        ref = O.pisa_forward_head(q, k, v, routing=idx[0, h], query_blocks=blocks, **kw)
        rows = np.isfinite(ref[:, 0])
        err = np.abs(o[0, h][rows] - ref[rows]).max()
        if w.dtype == "f32":
            rel = err / np.abs(ref[rows]).max()
            assert rel <= 1e-5, (h, rel)
            worst = max(worst, rel)
        else:
            assert err <= 2e-2, (h, err)
            worst = max(worst, err)
    say(f"[gpu] attn {name}: worst {'rel' if w.dtype == 'f32' else 'abs'} error {worst:.3e}")


def _zero_operands(x):
    return torch.zeros(P.operands_bytes(x), dtype=torch.uint8, device=x.device)


@pytest.mark.parametrize("name", ["tiny", "flux", "hunyuan"])
def test_prepare_operands_equals_the_fused_pass(name):
    """pisa_prepare_operands rebuilds the operand buffer from the statistics
    alone (and k): equal, byte for byte, to what pisa_block_stats wrote."""
    w, arrs = workload_inputs(name)
    say(f"[gpu] prepare operands {name}")
    q, k, v = (to_device(a, w.dtype) for a in arrs)
    st = P.alloc_stats(k, w.second_order, operands=False)
    st.operands = _zero_operands(k)
    P.pisa_block_stats(q, k, v, second_order=w.second_order, out=st)
    st2 = P.PisaStats(st.qbar, st.q2bar, st.kbar, st.vsum, st.ksig2, st.hsum, _zero_operands(k))
    P.pisa_prepare_operands(k, st2, second_order=w.second_order)
    torch.cuda.synchronize()
    assert torch.equal(st.operands, st2.operands)


@pytest.mark.parametrize("name,heads,so", [("tiny", None, False), ("flux", None, False), ("wan14", [0, 7], True)])
def test_oracle_statistics_drive_the_kernels(name, heads, so):
    """Statistics from another source: the oracle's (float64 on the host,
    rounded to the ABI's storage types) go through pisa_prepare_operands into
    the router and the fused kernel. Routing equals the oracle's (near-tie
    rule) and the output the oracle's for that routing, to the dtype's bar."""
    w = I.WORKLOADS[name]
    arrs = I.make_inputs(w, heads=heads)
    Bn, H, T, D = arrs[0].shape
    N = n_blocks(T)
    topk = oracle_topk(w.density, N)
    s = 1 / math.sqrt(D)
    say(f"[gpu] oracle statistics -> kernels: {name} heads {H} second_order={so}")
    q, k, v = (to_device(a, w.dtype) for a in arrs)
    qb, q2, kb, vs, sg, hs = ([] for _ in range(6))
    hosts = []
    for h in range(H):
        qh, kh, vh = head_f64(arrs, w.dtype, 0, h)
        hosts.append((qh, kh, vh))
        ks = O.kv_block_stats(kh, vh, 64)
        rq, rq2 = O.pool_queries(qh, 64, s)
        qb.append(rq); q2.append(rq2); kb.append(ks.kbar); vs.append(ks.vsum); sg.append(ks.sig2); hs.append(ks.H)
    dev = lambda xs, dt: torch.from_numpy(np.stack(xs)[None].astype(dt)).cuda()
    st = P.PisaStats(dev(qb, np.float64), dev(q2, np.float64) if so else None, dev(kb, np.float64),
                     dev(vs, np.float32), dev(sg, np.float64) if so else None, dev(hs, np.float32))
    P.pisa_prepare_operands(k, st, second_order=so)
    idx, wg = P.pisa_route_topk(q, st, topk, band=w.band, second_order=so)
    o = P.pisa_attn_fwd(q, k, v, st, idx, wg, band=w.band, second_order=so)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    worst = 0.0
    for h, (qh, kh, vh) in enumerate(hosts):
        wr = O.second_order_w(q2[h], sg[h], 64)[2] if so else None
        ref_idx, r = O.route_topk(qb[h], kb[h], s, topk, w.band, wr)
        for i in range(N):
            got = idx_h[0, h, i]
            if not np.array_equal(got, ref_idx[i]):
                gs, rs = set(got[got >= 0].tolist()), set(ref_idx[i][ref_idx[i] >= 0].tolist())
                kth = min(r[i, j] for j in rs)
                assert all(abs(r[i, j] - kth) < 1e-6 for j in gs ^ rs), (h, i)
        blocks = None if N <= 128 else sorted({0, 1, N // 3, N // 2, N - 2, N - 1})
        ref = O.pisa_forward_head(qh, kh, vh, topk=topk, band=w.band, second_order=so, routing=idx_h[0, h],
                                  query_blocks=blocks)
        rows = np.isfinite(ref[:, 0])
        got = o[0, h].double().cpu().numpy()[rows]
        err = float(np.abs(got - ref[rows]).max())
        if w.dtype == "f32":
            err /= float(np.abs(ref[rows]).max())
            assert err <= 1e-5, (h, err)
        else:
            assert err <= 2e-2, (h, err)
        worst = max(worst, err)
    say(f"[gpu] oracle statistics -> kernels {name}: worst {'rel' if w.dtype == 'f32' else 'abs'} error {worst:.3e}")
