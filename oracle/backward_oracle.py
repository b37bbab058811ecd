"""Plain CPU oracle for the gradients of the PISA / PWT forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP library.

Source: the "Piecewise-Taylor-Attention" README (the trainable regime: a
backward pass through both branches, with the routing detached and the
second-order spread gated, not clamped, in the virtual-token logits) over the
forward of "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
Transformers" (§3.2 Eqs. 3-5, §3.3 Eqs. 9-10, Algorithm 1), read as in
pisa_oracle.py (R1-R17).

The gradient is the derivative of the forward, so the oracle restates the
forward of one (batch, head) in float64 torch operations, step by step as
pisa_oracle.pisa_forward_head computes it, and differentiates it with
autograd. The routing table and the gate decision (w > ln B) are inputs /
constants: no gradient flows through a selection.

A backward that receives the forward's output o only to form
delta_t = dout_t . o_t computes, when handed some other o' (o rounded to the
storage dtype, say), the gradient of
    L' = sum_t dout_t . o_t - sum_t c_t log den_t,   c_t = dout_t . (o'_t - o_t)
with c held constant: delta enters every logit's gradient as -delta P (exact
keys) or -delta A n_j (virtual tokens), and those are the derivatives of
log den_t. grads(..., o_used=o') returns that gradient.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from . import pisa_oracle as O

__all__ = ["forward_torch", "grads", "grads_q_blocks"]


def forward_torch(q, k, v, idx, *, B=64, scale=None, band=1, n_sink=0, second_order=False,
                  first_order=True, gate_keep=None, return_logden=False, blocks=None):
    """o [T, D] of one head as a differentiable function of q, k, v (float64
    tensors). idx: the routing table [N, topk] (-1 padded). gate_keep: bool
    [N, N], True where w_ij <= ln B (second order only). With return_logden,
    also log den_t [T] (the log of each row's normaliser). With blocks (a list
    of query-block ids), only those blocks' rows are returned (in that order);
    the statistics still cover every block."""
    T, D = q.shape
    s = 1.0 / math.sqrt(D) if scale is None else scale
    N = O.num_blocks(T, B)
    sl = O.block_slices(T, B)
    n = torch.tensor([b - a for a, b in sl], dtype=torch.float64)
    kbar = torch.stack([k[a:b].mean(0) for a, b in sl])                    # [N, D]
    vhat = torch.stack([v[a:b].sum(0) for a, b in sl])                     # [N, D]
    H = sum((k[a:b] - kbar[j]).T @ v[a:b] for j, (a, b) in enumerate(sl))  # [D, D]
    if second_order:
        q2 = torch.stack([((s * q[a:b]) ** 2).mean(0) for a, b in sl])    # [N, D]
        sig2 = torch.stack([((k[a:b] - kbar[j]) ** 2).mean(0) for j, (a, b) in enumerate(sl)])
        w = 0.5 * q2 @ sig2.T                                              # [N, N]
        wg = torch.where(torch.as_tensor(gate_keep), w, torch.zeros_like(w))
    out, logden = [], []
    for i in (range(N) if blocks is None else blocks):
        a0, a1 = sl[i]
        S, U = O.selected_sets(np.asarray(idx[i]), i, N, band, n_sink)
        qp = s * q[a0:a1]
        keys = np.concatenate([np.arange(*sl[j]) for j in S])
        z = qp @ k[keys].T
        lam = qp @ kbar[U].T
        if second_order:
            lam = lam + wg[i, U][None, :]
        mass_logit = lam + torch.log(n[U])[None, :]
        m = torch.maximum(z.max(1).values, mass_logit.max(1).values if len(U) else z.max(1).values).detach()
        pe = torch.exp(z - m[:, None])
        a = torch.exp(lam - m[:, None])
        num = pe @ v[keys] + a @ vhat[U]
        ltail = a @ n[U]
        if first_order:
            num = num + (ltail / T)[:, None] * (qp @ H)
        den = pe.sum(1) + ltail
        out.append(num / den[:, None])
        logden.append(torch.log(den) + m)    # m is a constant: d/dz gives P, d/dlam gives A n
    if return_logden:
        return torch.cat(out), torch.cat(logden)
    return torch.cat(out)


def grads(q, k, v, do, idx, o_used=None, **kw):
    """(dq, dk, dv) float64 numpy arrays for one head, for the loss <do, o>;
    with o_used [T, D], the gradient a backward computes when its delta is
    formed from o_used instead of the exact o (module docstring)."""
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    gate_keep = None
    if kw.get("second_order"):
        # the gate decision of the forward (a constant here)
        _, parts = O.pisa_forward_head(q, k, v, B=kw.get("B", 64), scale=kw.get("scale"), topk=idx.shape[1],
                                       band=kw.get("band", 1), second_order=True, routing=idx,
                                       n_sink=kw.get("n_sink", 0), return_parts=True)
        gate_keep = parts["w"] <= math.log(kw.get("B", 64))
    g = torch.tensor(do, dtype=torch.float64)
    o, logden = forward_torch(*t, idx, gate_keep=gate_keep, return_logden=True, **kw)
    loss = (o * g).sum()
    if o_used is not None:
        c = (g * (torch.tensor(o_used, dtype=torch.float64) - o.detach())).sum(1)
        loss = loss - (c * logden).sum()
    loss.backward()
    return tuple(x.grad.numpy() for x in t)


def grads_q_blocks(q, k, v, do, idx, blocks, **kw):
    """dq rows of the listed query blocks [len(blocks) * rows, D] (float64
    numpy), for the loss <do, o>. q_t enters only its own block's outputs (its
    logits, and for second order that block's pooled q^2), so these rows of
    dq follow from those blocks' outputs alone: a sampled check at any size."""
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=(n == 0)) for n, x in enumerate((q, k, v))]
    gate_keep = None
    if kw.get("second_order"):
        _, parts = O.pisa_forward_head(q, k, v, B=kw.get("B", 64), scale=kw.get("scale"), topk=idx.shape[1],
                                       band=kw.get("band", 1), second_order=True, routing=idx,
                                       n_sink=kw.get("n_sink", 0), return_parts=True)
        gate_keep = parts["w"] <= math.log(kw.get("B", 64))
    o = forward_torch(*t, idx, gate_keep=gate_keep, blocks=list(blocks), **kw)
    sl = O.block_slices(q.shape[0], kw.get("B", 64))
    rows = np.concatenate([np.arange(*sl[i]) for i in blocks])
    (o * torch.tensor(do[rows], dtype=torch.float64)).sum().backward()
    return t[0].grad.numpy()[rows]
