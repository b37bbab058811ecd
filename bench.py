"""Benchmark of the PISA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan14]

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: pisa_block_stats -> pisa_route_topk ->
pisa_attn_fwd. Prints ONE JSON line. ``value`` is the dense-equivalent
throughput of the whole step, 4 B H T^2 D / t_step (the convention that
credits a sparse method with the full attention's work); the fused kernel's
own milliseconds and dense-equivalent TFLOP/s are reported beside it.

``roofline`` refers to the dominant kernel (pisa_attn_fwd, bf16 MFMA): its
algorithmic flops per launch (4 D per (query row, exact key) and per
(query row, virtual token) pair, plus 2 D^2 per query row for the global
first order) over its mean launch time measured with HIP events on the
stream it is launched on. ``cpu_baseline`` times the fp64 oracle (as it
stands) on a bounded sample of the same workload on the host cores.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, datasheet
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 peak (matrix cores; the packed vector peak is the same)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, datasheet

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SRCS = [os.path.join(ROOT, "block_sparse_taylor_amd", "csrc", f)
             for f in ("attn_mfma.hip", "attn_loop_d128.inc")]
ATTN_KERNEL = "attn_asm_kernel"        # the fused forward's kernel at head_dim 128
COPY_KERNEL = "elementwise"            # torch's elementwise kernel used as the calibration copy
COPY_BYTES = 1 << 30                   # bytes read (and written) per calibration copy


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"attn_mfma_{workload}_traffic.json")


def kernel_stats_file(workload):
    return os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.txt")


def profile_avg_ns(workload, kernel=ATTN_KERNEL):
    """Average duration (ns) of `kernel` in the committed rocprofv3 --stats
    summary of this workload, if that summary was taken on the current kernel
    source (its header names the source's sha256), else None."""
    import csv
    try:
        with open(kernel_stats_file(workload)) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    if not any(ln.startswith("#") and source_digest() in ln for ln in lines):
        return None
    rows = [ln for ln in lines if not ln.startswith("#") and ln.strip()]
    for row in csv.DictReader(rows):
        if kernel in row.get("Name", ""):
            return float(row["AverageNs"])
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for path in ATTN_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per launch of the fused kernel recorded from counters, if they
    were taken on the current kernel source (else None)."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_means(path, counter):
    """Mean counter value per dispatch for the fused kernel and the calibration copy."""
    import csv
    vals = {"attn": [], "copy": []}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            name = row.get("Kernel_Name", "")
            key = "attn" if ATTN_KERNEL in name else ("copy" if COPY_KERNEL in name else None)
            if key:
                vals[key].append(float(row["Counter_Value"]))
    if not vals["attn"] or not vals["copy"]:
        raise SystemExit(f"{path}: no {counter} rows for {ATTN_KERNEL} and the calibration copy")
    return float(np.mean(vals["attn"])), float(np.mean(vals["copy"])), len(vals["attn"])


def record_traffic(fetch_csv, write_csv, workload):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    into HBM bytes per launch of the fused kernel, each counter scaled by what it
    reads for a plain copy of COPY_BYTES."""
    fa, fc, nf = _pmc_means(fetch_csv, "FETCH_SIZE")
    wa, wc, nw = _pmc_means(write_csv, "WRITE_SIZE")
    kf = fc * 1024.0 / COPY_BYTES      # counter bytes per true byte read
    kw = wc * 1024.0 / COPY_BYTES
    rec = {
        "workload": workload,
        "kernel": ATTN_KERNEL,
        "source_sha256": source_digest(),
        "fetch_kib_per_launch": fa, "write_kib_per_launch": wa, "dispatches": [nf, nw],
        "copy_fetch_kib": fc, "copy_write_kib": wc, "copy_bytes": COPY_BYTES,
        "fetch_scale": kf, "write_scale": kw,
        "hbm_read_bytes_per_launch": fa * 1024.0 / kf,
        "hbm_write_bytes_per_launch": wa * 1024.0 / kw,
        "hbm_bytes_per_launch": fa * 1024.0 / kf + wa * 1024.0 / kw,
    }
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="heads the oracle evaluates for the CPU baseline")
    ap.add_argument("--no-phase1", action="store_true",
                    help="skip the extra launches after the timed steps (Phase 1 alone, the Morton "
                         "reorder), so that a kernel trace or counter run sees only the steps")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the pisa_attn_bwd leg (timed after the forward steps)")
    ap.add_argument("--bwd-steps", type=int, default=3)
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step captured into a HIP graph (after the timed steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain copy of COPY_BYTES three times "
                         "(the reference kernel for the HBM byte counters)")
    ap.add_argument("--routing-locality", action="store_true",
                    help="after the timed steps, time the fused kernel again under routings of the same "
                         "size but other locality (a sliding window, one fixed set per head, uniform "
                         "random) to bound what re-fetched K/V blocks cost")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: derive the fused kernel's HBM bytes per launch from two "
                         "rocprofv3 --pmc counter_collection.csv files and record them")
    return ap.parse_args()


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.record_traffic[0], args.record_traffic[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the operator shards by (batch, head) with no exchange, see the design notes",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_taylor_amd as P
    from block_sparse_taylor_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    plan_kernel = P.attn_fwd_plan(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype,
                                  P.topk_for_density(w.density, P.num_blocks(w.seq_len)), w.band,
                                  w.second_order)
    attn_kernel_name = {0: "attn_valu_kernel", 1: ATTN_KERNEL, 2: "attn_mfma_kernel", 3: "attn_f32_kernel"}[plan_kernel]
    torch.cuda.set_device(dev)
    t0 = time.time()
    qa, ka, va = I.make_inputs(w)
    gen_s = time.time() - t0

    def to_dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v = to_dev(qa), to_dev(ka), to_dev(va)
    B, H, T, D = q.shape
    N = P.num_blocks(T)
    topk = P.topk_for_density(w.density, N)
    so = w.second_order
    st = P.alloc_stats(k, so)
    ws = P.stats_workspace(k)
    idx = torch.empty(B, H, N, max(topk, 1), dtype=torch.int32, device=dev)[..., :topk].contiguous()
    wg = torch.empty(B, H, N, N, dtype=torch.float32, device=dev) if so else None
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(record=None):
        if record:
            record[0].record(stream)
        P.pisa_block_stats(q, k, v, second_order=so, out=st, workspace=ws)
        if record:
            record[1].record(stream)
        P.pisa_route_topk(q, st, topk, band=w.band, second_order=so, idx=idx, wgate=wg)
        if record:
            record[2].record(stream)
        P.pisa_attn_fwd(q, k, v, st, idx if topk else None, wg, band=w.band, second_order=so, out=o)
        if record:
            record[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    recs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for r in recs:
        step(r)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    per_kernel = [[r[a].elapsed_time(r[a + 1]) for r in recs] for a in range(3)]
    stats_ms, route_ms, attn_ms = (float(np.mean(x)) for x in per_kernel)
    spread = lambda x: {"median_ms": round(float(np.median(x)), 4), "min_ms": round(float(np.min(x)), 4)}

    # inputs that fit the 256 MB Infinity Cache are also timed cold: a 512 MB
    # scratch buffer is written before each step (outside its timed span)
    cold_ms = None
    if 3 * q.numel() * q.element_size() < (256 << 20):
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(args.steps):
            scratch.fill_(1)
            c0, c1 = ev(), ev()
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        cold_ms = round(float(np.mean(cold)), 4)
        del scratch

    # the same step captured once into a HIP graph (no entry point allocates,
    # clears memory or synchronises with the host) and replayed: the launch
    # overhead a graph removes, after the timed steps and outside them
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = ev(), ev()
        g0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph

    # Phase 1 alone (exact tiles only, phase_mask bit 0), after the timed steps
    # and outside them, on the same inputs and routing table
    phase1_ms = None
    if not args.no_phase1:
        o1 = torch.empty_like(q)
        p1 = [ev() for _ in range(args.steps + 1)]
        for _ in range(2):
            P.pisa_attn_fwd(q, k, v, st, idx if topk else None, wg, band=w.band, second_order=so,
                            phase_mask=1, out=o1)
        torch.cuda.synchronize()
        p1[0].record(stream)
        for e_ in p1[1:]:
            P.pisa_attn_fwd(q, k, v, st, idx if topk else None, wg, band=w.band, second_order=so,
                            phase_mask=1, out=o1)
            e_.record(stream)
        torch.cuda.synchronize()
        phase1_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(p1[:-1], p1[1:])]))
        del o1

    # The fused kernel under routings with the router's list sizes but other
    # locality: "window" routes query block i to blocks i+2 .. i+1+topk (mod N),
    # so neighbouring query blocks share all but one; "fixed" routes every
    # query block of a head to the same blocks; "random" draws distinct
    # non-band blocks uniformly. Outside the timed steps.
    locality = None
    if args.routing_locality and topk and not so and w.band == 1 and N > topk + 3:
        ii = torch.arange(N, device=dev).view(N, 1)
        jj = torch.arange(topk, device=dev).view(1, topk)
        routings = {"router": idx,
                    "window": ((ii + 2 + jj) % N).to(torch.int32).expand(B, H, N, topk).contiguous(),
                    "fixed": ((N // 2 + 2 + jj) % N).to(torch.int32).expand(B, H, N, topk).contiguous()}
        gen = torch.Generator(device="cpu").manual_seed(0)
        rnd = torch.empty(B, H, N, topk, dtype=torch.int32)
        band_rows = torch.arange(N).repeat_interleave(3)
        band_cols = (torch.arange(N).view(N, 1) + torch.tensor([-1, 0, 1])).clamp(0, N - 1).reshape(-1)
        for bh in range(B * H):
            sc = torch.rand(N, N, generator=gen)
            sc[band_rows, band_cols] = -1.0
            rnd.view(B * H, N, topk)[bh] = sc.topk(topk, dim=1).indices.to(torch.int32)
        routings["random"] = rnd.to(dev)
        locality = {}
        o_l = torch.empty_like(q)
        for name, ix in routings.items():
            for _ in range(2):
                P.pisa_attn_fwd(q, k, v, st, ix, None, band=1, out=o_l)
            evs = [ev() for _ in range(args.steps + 1)]
            torch.cuda.synchronize()
            evs[0].record(stream)
            for e_ in evs[1:]:
                P.pisa_attn_fwd(q, k, v, st, ix, None, band=1, out=o_l)
                e_.record(stream)
            torch.cuda.synchronize()
            locality[name] = round(float(np.mean([a_.elapsed_time(b_) for a_, b_ in zip(evs[:-1], evs[1:])])), 4)
        locality = {"ms": locality, "note": "pisa_attn_fwd mean ms under each routing (same list sizes)"}
        del o_l, routings

    # Morton token reorder around the operator (raster-order token-major
    # [B,T,H,D] activations -> Z-order [B,H,T,D] for q, k, v, and the output
    # back), timed on its own after the steps; reported beside them
    reorder = None
    if not args.no_phase1 and w.grid:
        perm = P.z_order(w.grid, w.text_tokens).to(dev)
        if perm.numel() == T:
            xt = [torch.empty(B, T, H, D, dtype=q.dtype, device=dev).normal_() for _ in range(3)]
            ht = [torch.empty(B, H, T, D, dtype=q.dtype, device=dev) for _ in range(3)]
            ot = torch.empty(B, T, H, D, dtype=q.dtype, device=dev)

            def reorder_pass():
                for a, b in zip(xt, ht):
                    P.reorder_gather(a, perm, out=b)
                P.reorder_scatter(o, perm, out=ot)

            for _ in range(2):
                reorder_pass()
            torch.cuda.synchronize()
            r0, r1 = ev(), ev()
            r0.record(stream)
            for _ in range(args.steps):
                reorder_pass()
            r1.record(stream)
            torch.cuda.synchronize()
            rms = r0.elapsed_time(r1) / args.steps
            rbytes = 4 * 2 * B * T * H * D * q.element_size()
            reorder = {"ms": round(rms, 4), "tensors": "gather q, k, v + scatter o",
                       "algorithmic_bytes": rbytes, "gbs": round(rbytes / (rms * 1e-3) / 1e9, 1),
                       "frac_hbm": round(rbytes / (rms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del xt, ht, ot

    # Backward (pisa_attn_bwd) of the last step's forward, on seeded dout,
    # timed on its own after the steps: one call runs all its kernels. The
    # forward is run once more (untimed) writing its row statistics, which
    # the backward takes as training does; the backward that recomputes them
    # is timed beside it.
    bwd_ms = bwd_re_ms = None
    if not args.no_backward:
        gen = torch.Generator(device=dev).manual_seed(1234)
        dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
        grads = tuple(torch.empty_like(q) for _ in range(3))
        bws = P.attn_bwd_workspace(q)
        rs = P.alloc_row_stats(q)
        P.pisa_attn_fwd(q, k, v, st, idx if topk else None, wg, band=w.band, second_order=so, out=o,
                        row_stats=rs)

        def time_bwd(row_stats):
            bwd = lambda: P.pisa_attn_bwd(q, k, v, o, dout, st, idx if topk else None, wg, band=w.band,
                                          second_order=so, workspace=bws, out=grads, row_stats=row_stats)
            bwd()
            torch.cuda.synchronize()
            b0, b1 = ev(), ev()
            b0.record(stream)
            for _ in range(args.bwd_steps):
                bwd()
            b1.record(stream)
            torch.cuda.synchronize()
            return b0.elapsed_time(b1) / args.bwd_steps

        bwd_ms = time_bwd(rs)
        bwd_re_ms = time_bwd(None)
        del grads, bws, dout, rs

    # ---- algorithmic work of the fused kernel (from the routing table actually used)
    idx_h = idx.cpu().numpy().reshape(B * H, N, topk)
    nrow = np.array([min(64, T - 64 * j) for j in range(N)], dtype=np.int64)
    exact_pairs = 0
    virt_pairs = 0
    for bh in range(B * H):
        for i in range(N):
            sel = set(range(max(0, i - w.band), min(N, i + w.band + 1)))
            sel.update(int(j) for j in idx_h[bh, i] if j >= 0)
            keys = int(nrow[list(sel)].sum())
            exact_pairs += int(nrow[i]) * keys
            virt_pairs += int(nrow[i]) * (N - len(sel))
    attn_flops = 4 * D * (exact_pairs + virt_pairs) + 2 * D * D * B * H * T
    phase1_tflops = 4 * D * exact_pairs / (phase1_ms * 1e-3) / 1e12 if phase1_ms else None
    dense_flops = 4.0 * B * H * T * T * D
    attn_tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    apeak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS   # the fused kernel's own matrix-core peak
    prof_ns = profile_avg_ns(w.name) if attn_kernel_name == ATTN_KERNEL else None
    traffic = load_traffic(w.name) if attn_kernel_name == ATTN_KERNEL else None
    unique_bytes = 4 * B * H * T * D * (2 if w.dtype == "bf16" else 4)   # Q, K, V read and O written once

    e = 2 if w.dtype == "bf16" else 4
    groups = min(max(1, 512 // (B * H)), -(-N // 4))      # the statistics pass's block ranges per head
    G = -(-N // -(-N // groups))
    BHND = B * H * N * D
    NC16 = -(-N // 16) * 16
    # statistics pass, algorithmic: read Q, K, V once; write the paper's
    # statistics in their storage types (qbar, kbar fp64; V-hat fp32; q2bar,
    # key variance fp64 with the second order; H fp32)
    stats_bytes = (3 * B * H * T * D * e
                   + BHND * (8 + 8 + 4) + (BHND * 16 if so else 0)
                   + B * H * D * D * 4)
    # beyond that it writes the kernels' operand layouts and round-trips the
    # partial H sums through memory: reported, not rated
    stats_layout_bytes = (2 * BHND * e                                   # kbar, vbar in the input dtype
                          + B * H * NC16 * D * 4 * (2 if so else 1)       # router-order kbar (, variance)
                          + (B * H * N * 64 * D * 2 + B * H * -(-N // 64) * 64 * D * 2
                             + B * H * 2 * D * D * 2 if w.dtype == "bf16" else 0)   # packed K, kbar, H
                          + 2 * B * H * G * D * D * 4)                    # partial H write + read
    # routing, algorithmic: read the pooled statistics it ranks (qbar fp64,
    # router-order kbar fp32; q2bar fp64 and router-order variance fp32 with
    # the second order), write the table (and the gated w table)
    route_bytes = (B * H * N * D * 8 + B * H * NC16 * D * 4
                   + ((B * H * N * D * 8 + B * H * NC16 * D * 4) if so else 0)
                   + B * H * N * topk * 4
                   + (B * H * N * N * 4 if so else 0))
    route_gemm_flops = 2 * B * H * N * N * D * (2 if so else 1)   # fp32 score (and spread) products

    out = {
        "metric": ("pisa_attn_fwd ms & dense-equiv TFLOP/s, Wan2.1-14B shape, density 0.125"
                   if w.name == "wan14" else
                   f"pisa_attn_fwd ms & dense-equiv TFLOP/s, {w.name} shape, density {w.density}"),
        "value": round(dense_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s dense-equivalent (4 B H T^2 D per full step: stats + route + fused forward)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded spatially correlated q/k in 3D Morton order, v ~ N(0,1))",
        "config": {"workload": f"{w.name}: batch {B}, heads {H}, T {T}, head_dim {D}, {w.dtype}, "
                               f"block 64, density {w.density} (topk {topk}) + band {w.band}"
                               + (", second order" if so else ""),
                   "topk": topk, "band": w.band, "second_order": so},
        "ms_per_step_cache_flushed": cold_ms,
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 4),
        "pisa_attn_fwd": {"ms": round(attn_ms, 4), **spread(per_kernel[2]),
                          "dense_equiv_tflops": round(dense_flops / (attn_ms * 1e-3) / 1e12, 2),
                          "algorithmic_tflop": round(attn_flops / 1e12, 4)},
        "phase1_exact": None if phase1_ms is None else {
            "ms": round(phase1_ms, 4), "algorithmic_tflop": round(4 * D * exact_pairs / 1e12, 4),
            "tflops": round(phase1_tflops, 2), "frac_mfma": round(phase1_tflops / apeak, 4)},
        "morton_reorder": reorder,
        "pisa_block_stats": {"ms": round(stats_ms, 4), **spread(per_kernel[0]), "algorithmic_bytes": stats_bytes,
                             "gbs": round(stats_bytes / (stats_ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(stats_bytes / (stats_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "layout_overhead_bytes": stats_layout_bytes,
                             "note": "algorithmic bytes: Q, K, V read + the statistics written; the operand "
                                     "layouts and the partial-H round trip are layout_overhead_bytes, not rated"},
        "pisa_route_topk": {"ms": round(route_ms, 4), **spread(per_kernel[1]), "algorithmic_bytes": route_bytes,
                            "gbs": round(route_bytes / (route_ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(route_bytes / (route_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                            "score_gemm_tflop": round(route_gemm_flops / 1e12, 5),
                            "score_gemm_floor_ms": round(route_gemm_flops / (PEAK_FP32_TFLOPS * 1e12) * 1e3, 4),
                            "frac_fp32_mfma": round(route_gemm_flops / (route_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": apeak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / apeak, 4),
                     "frac_profile": (None if prof_ns is None else
                                      round(attn_flops / (prof_ns * 1e-9) / 1e12 / apeak, 4)),
                     "traffic": traffic,
                     "traffic_kind": ("L2-to-fabric bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, each "
                                      "scaled by its reading for a plain 1 GiB copy); requests the Infinity "
                                      "Cache serves are included, so this bounds HBM bytes from above"),
                     "traffic_over_unique": None if traffic is None else round(traffic / unique_bytes, 2),
                     "unique_bytes": unique_bytes,
                     "kernel": attn_kernel_name + " (pisa_attn_fwd)"},
        "input_generation_s": round(gen_s, 1),
    }
    if locality is not None:
        out["routing_locality"] = locality
    if bwd_ms is not None:
        # five products per attended pair (recomputed logits, dP, dV, dK, dQ; the
        # virtual tokens likewise with kbar and V-hat), plus H g and dH per row
        bwd_flops = 10 * D * (exact_pairs + virt_pairs) + 4 * D * D * B * H * T
        bwd_tflops = bwd_flops / (bwd_ms * 1e-3) / 1e12
        # bf16: the products run on bf16 MFMA; fp32: on the fp32 vector units
        bpeak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        out["pisa_attn_bwd"] = {
            "ms": round(bwd_ms, 3), "steps": args.bwd_steps, "algorithmic_tflop": round(bwd_flops / 1e12, 4),
            "ms_recomputing_row_stats": round(bwd_re_ms, 3),
            "note": "with the forward's row statistics (lse, c); ms_recomputing_row_stats without them",
            "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(bwd_tflops, 2),
                         "peak": bpeak, "unit": "TFLOP/s", "frac": round(bwd_tflops / bpeak, 4), "traffic": None,
                         "kernel": "pisa_attn_bwd (all its kernels: " + ("bf16 MFMA products, chain and dH; "
                                   "integer selection mask)" if w.dtype == "bf16" else "fp32 VALU)")}}

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, qa, ka, va, args.cpu_heads, topk)
    print(json.dumps(out), flush=True)


def cpu_baseline(w, qa, ka, va, nheads, topk):
    """The fp64 oracle (as it stands), timed on the first `nheads` heads of the
    same inputs: block statistics, routing and the forward of every query
    block; reported as dense-equivalent TFLOP/s of the rows it produced."""
    from block_sparse_taylor_amd import inputs as I
    from oracle import pisa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    nheads = min(nheads, qa.shape[1])
    T, D = qa.shape[2], qa.shape[3]
    dt = 0.0
    for h in range(nheads):
        q, k, v = (I.as_f64(x[0, h], w.dtype) for x in (qa, ka, va))
        t0 = time.time()
        o = O.pisa_forward_head(q, k, v, topk=topk, band=w.band, second_order=w.second_order)
        dt += time.time() - t0
        assert np.isfinite(o).all()
    dense_flops = 4.0 * nheads * T * T * D
    return {"value": round(dense_flops / dt / 1e12, 5), "unit": "TFLOP/s dense-equivalent",
            "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"heads 0..{nheads - 1} of {w.name} (of {qa.shape[1]}), every query block: "
                      f"statistics, routing and forward in float64 numpy; {dt:.1f} s",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
