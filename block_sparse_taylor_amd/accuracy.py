"""Accuracy of the operator's variants against dense attention, on the GPU.

The PISA paper's quantitative validation (§4.4, Fig. 8) reports the
normalised L1 error ||O - O_dense||_1 / ||O_dense||_1 of its attention output
for sparse attention alone, sparse + block zeroth order, and sparse + hybrid
(zeroth order + global first order), against density at 32K tokens and
against length at 20% density; the "Piecewise-Taylor-Attention" README adds
the gated second-order term (PWT) and compares variants by cosine similarity
with full attention. This module runs the same comparison with this
library's kernels on the seeded synthetic workloads (no model activations):

    sparse_only  exact blocks only (phase_mask 1: Eq. 2 over S_i)
    zeroth       + virtual tokens (first_order off; the paper's "-0th")
    pisa         + global first order (the hybrid; the default operator)
    pwt          + gated second-order term in routing and virtual logits

The dense reference is softmax(s Q K^T) V in fp32 on the GPU (torch matmuls,
query rows in chunks), from the same bf16 inputs.

    python -m block_sparse_taylor_amd.accuracy [--heads 4] [--json FILE]
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import math

import numpy as np
import torch

from . import (num_blocks, pisa_attn_fwd, pisa_block_stats, pisa_route_topk,
               topk_for_density)
from . import inputs as I

VARIANTS = ("sparse_only", "zeroth", "pisa", "pwt")


def dense_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                    chunk: int = 2048) -> torch.Tensor:
    """softmax(s Q K^T) V in fp32, [B,H,T,D] (query rows in chunks)."""
    torch.backends.cuda.matmul.allow_tf32 = False
    B, H, T, D = q.shape
    out = torch.empty(B, H, T, D, dtype=torch.float32, device=q.device)
    kt = k.float().transpose(-1, -2).contiguous()
    vf = v.float().contiguous()
    for t0 in range(0, T, chunk):
        s = torch.matmul(q[:, :, t0:t0 + chunk].float().contiguous(), kt) * scale
        s = s - s.amax(dim=-1, keepdim=True)
        p = torch.exp(s)
        out[:, :, t0:t0 + chunk] = torch.matmul(p, vf) / p.sum(dim=-1, keepdim=True)
    return out


def run_variant(q, k, v, topk: int, variant: str, band: int = 1, stats=None):
    """The operator's output for one variant (stats reused when given)."""
    so = variant == "pwt"
    st = stats if stats is not None else pisa_block_stats(q, k, v, second_order=so)
    idx, wg = pisa_route_topk(q, st, topk, band=band, second_order=so)
    idx = idx if topk else None
    if variant == "sparse_only":
        return pisa_attn_fwd(q, k, v, st, idx, wg, band=band, phase_mask=1)
    if variant == "zeroth":
        return pisa_attn_fwd(q, k, v, st, idx, wg, band=band, first_order=False)
    return pisa_attn_fwd(q, k, v, st, idx, wg, band=band, second_order=so)


def errors(o: torch.Tensor, ref: torch.Tensor):
    """(normalised L1 error, mean cosine similarity of the output rows)."""
    o = o.float()
    l1 = float((o - ref).abs().sum() / ref.abs().sum())
    cos = float(torch.nn.functional.cosine_similarity(o, ref, dim=-1).mean())
    return l1, cos


def _device_inputs(w, heads):
    qa, ka, va = I.make_inputs(w, heads=range(heads))
    dev = torch.device("cuda")
    if w.dtype == "bf16":
        return [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (qa, ka, va)]
    return [torch.from_numpy(x).to(dev) for x in (qa, ka, va)]


def sweep_point(w, heads: int, density: float):
    q, k, v = _device_inputs(w, heads)
    scale = 1.0 / math.sqrt(w.head_dim)
    ref = dense_attention(q, k, v, scale)
    topk = topk_for_density(density, num_blocks(w.seq_len))
    st1 = pisa_block_stats(q, k, v)
    st2 = pisa_block_stats(q, k, v, second_order=True)
    row = {"T": w.seq_len, "density": density, "topk": topk}
    for var in VARIANTS:
        o = run_variant(q, k, v, topk, var, band=w.band, stats=st2 if var == "pwt" else st1)
        row[var] = dict(zip(("l1", "cos"), errors(o, ref)))
    torch.cuda.synchronize()
    return row


def video_workload(frames: int, heads: int):
    """The Wan2.1-14B generator (30 x 52 latent frames) with `frames` frames."""
    w = I.WORKLOADS["wan14"]
    return dataclasses.replace(w, heads=heads, grid=(frames, 30, 52), seq_len=frames * 30 * 52)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=4)
    ap.add_argument("--densities", default="0.05,0.1,0.125,0.2,0.3,0.5")
    ap.add_argument("--frames", default="3,6,11,21,41", help="length sweep (20%% density)")
    ap.add_argument("--json", default=None)
    a = ap.parse_args()
    rows = []
    w32 = video_workload(21, a.heads)
    for d in (float(x) for x in a.densities.split(",")):
        rows.append(dict(sweep="density", **sweep_point(w32, a.heads, d)))
        print(json.dumps(rows[-1]), flush=True)
    for f in (int(x) for x in a.frames.split(",")):
        rows.append(dict(sweep="length", **sweep_point(video_workload(f, a.heads), a.heads, 0.2)))
        print(json.dumps(rows[-1]), flush=True)
    if a.json:
        with open(a.json, "w") as fh:
            json.dump(rows, fh, indent=1)


if __name__ == "__main__":
    main()
