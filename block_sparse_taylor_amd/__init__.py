"""PISA piecewise sparse attention forward for MI355X (gfx950).

Thin Python binding over libpisa's C ABI (include/pisa.h). Tensors are torch
tensors on a ROCm device; torch provides device memory and the current HIP
stream, the library does every step of the computation. There is no CPU or
eager fallback: if libpisa.so is missing, the calls raise.

The three calls follow the PISA paper's Algorithm 1 (prepare phase steps 1-2,
fused kernel Phases 1-3):

    stats     = pisa_block_stats(q, k, v, second_order=...)
    idx, wg   = pisa_route_topk(q, stats, topk=..., band=1, second_order=...)
    o         = pisa_attn_fwd(q, k, v, stats, idx, wg, ...)

``stats`` holds the paper's statistics and the operand buffer the kernels
read; ``pisa_prepare_operands(k, stats)`` builds that buffer from statistics
computed by any other means.

and ``pisa_attn_bwd(q, k, v, o, dout, stats, idx, wg, ...)`` returns the
gradients with the routing and gate held (the README's trainable regime).
``piecewise_sparse_attention`` chains them with topk = floor(density * N)
and is differentiable.
"""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import PISA_BF16, PISA_F32, PisaError

__all__ = ["PisaStats", "pisa_block_stats", "pisa_block_stats_noalloc", "pisa_prepare_operands", "pisa_route_topk", "pisa_attn_fwd",
           "pisa_attn_fwd_valu", "pisa_attn_bwd", "piecewise_sparse_attention", "num_blocks", "topk_for_density",
           "z_order", "reorder_gather", "reorder_scatter", "PisaError", "library"]

BLOCK = 64


def library():
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PISA_BF16
    if t.dtype == torch.float32:
        return PISA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _shape(q: torch.Tensor, scale) -> _lib.Shape:
    if q.dim() != 4:
        raise ValueError("expected [batch, heads, seq_len, head_dim]")
    B, H, T, D = q.shape
    return _lib.Shape(B, H, T, D, BLOCK, _dtype_code(q), float(scale) if scale else 0.0)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def num_blocks(seq_len: int) -> int:
    return -(-seq_len // BLOCK)


def topk_for_density(density: float, n_blocks: int) -> int:
    """k = floor(density * N) routed blocks per query block (band excluded)."""
    return max(0, min(n_blocks, int(math.floor(density * n_blocks + 1e-9))))


@dataclass
class PisaStats:
    """The paper's block statistics (pisa_stats_t) and the operand buffer the
    routing and attention kernels read (opaque, built from them)."""
    qbar: torch.Tensor | None     # fp64 [B,H,N,D]
    q2bar: torch.Tensor | None    # fp64 [B,H,N,D] (second order)
    kbar: torch.Tensor            # fp64 [B,H,N,D]
    vsum: torch.Tensor            # fp32 [B,H,N,D]
    ksig2: torch.Tensor | None    # fp64 [B,H,N,D] (second order)
    hsum: torch.Tensor            # fp32 [B,H,D,D]
    operands: torch.Tensor | None = None   # uint8 [pisa_operands_bytes]
    hnorm: torch.Tensor | None = None      # fp64 [B,H,N]: ||H_j - Hbar||_F (covariance prior)

    def as_c(self) -> _lib.Stats:
        return _lib.Stats(_ptr(self.qbar), _ptr(self.q2bar), _ptr(self.kbar), _ptr(self.vsum),
                          _ptr(self.ksig2), _ptr(self.hsum), _ptr(self.hnorm))

    def statistics_only(self) -> "PisaStats":
        """The same statistics without the operand buffer (what the backward reads)."""
        return PisaStats(self.qbar, self.q2bar, self.kbar, self.vsum, self.ksig2, self.hsum, None, self.hnorm)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def operands_bytes(x: torch.Tensor, scale=None) -> int:
    return int(library().pisa_operands_bytes(ctypes.byref(_shape(x, scale))))


def alloc_operands(x: torch.Tensor) -> torch.Tensor:
    return torch.empty(max(16, operands_bytes(x)), dtype=torch.uint8, device=x.device)


def alloc_stats(k: torch.Tensor, second_order: bool, operands: bool = True, cov_bias: bool = False) -> PisaStats:
    B, H, T, D = k.shape
    N = num_blocks(T)
    dev = k.device
    f64 = dict(dtype=torch.float64, device=dev)
    return PisaStats(
        qbar=torch.empty(B, H, N, D, **f64),
        q2bar=torch.empty(B, H, N, D, **f64) if second_order else None,
        kbar=torch.empty(B, H, N, D, **f64),
        vsum=torch.empty(B, H, N, D, dtype=torch.float32, device=dev),
        ksig2=torch.empty(B, H, N, D, **f64) if second_order else None,
        hsum=torch.empty(B, H, D, D, dtype=torch.float32, device=dev),
        operands=alloc_operands(k) if operands else None,
        hnorm=torch.empty(B, H, N, **f64) if cov_bias else None,
    )


def operand_views(stats: PisaStats, like: torch.Tensor) -> dict:
    """Views of the arrangements inside stats.operands (pisa_operands_offsets),
    for diagnostics and tests: name -> flat tensor of its element type."""
    lib = library()
    sh = _shape(like, None)
    off = (ctypes.c_int64 * len(_lib.OPERANDS))()
    _lib.check("pisa_operands_offsets", lib.pisa_operands_offsets(ctypes.byref(sh), off))
    ends = list(off[1:]) + [operands_bytes(like)]
    el = {"kbar_c": like.dtype, "vbar_c": like.dtype, "kbar_r": torch.bfloat16, "ksig2_r": torch.bfloat16,
          "kpack": torch.bfloat16, "kbpack": torch.bfloat16, "hpack": torch.bfloat16, "knorm": torch.float32}
    out = {}
    for n, name in enumerate(_lib.OPERANDS):
        raw = stats.operands[off[n]:ends[n]]
        size = torch.empty(0, dtype=el[name]).element_size()
        out[name] = raw[: raw.numel() // size * size].view(el[name])
    return out


def stats_workspace(k: torch.Tensor, scale=None) -> torch.Tensor:
    lib = library()
    sh = _shape(k, scale)
    n = lib.pisa_stats_workspace_bytes(ctypes.byref(sh))
    return torch.empty(max(16, n), dtype=torch.uint8, device=k.device)


def attn_bwd_workspace(q: torch.Tensor, scale=None) -> torch.Tensor:
    """A workspace of pisa_attn_bwd_workspace_bytes for tensors of q's shape."""
    lib = library()
    n = lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(_shape(q, scale)))
    return torch.empty(max(16, n), dtype=torch.uint8, device=q.device)


def pisa_block_stats(q, k, v, second_order=False, scale=None, out: PisaStats | None = None,
                     workspace: torch.Tensor | None = None, cov_bias=False) -> PisaStats:
    lib = library()
    _contig(q, k, v)
    sh = _shape(k, scale)
    out = out or alloc_stats(k, second_order, cov_bias=cov_bias)
    if out.operands is None:
        out.operands = alloc_operands(k)
    if cov_bias and out.hnorm is None:
        B, H, T, _ = k.shape
        out.hnorm = torch.empty(B, H, num_blocks(T), dtype=torch.float64, device=k.device)
    ws = workspace if workspace is not None else stats_workspace(k, scale)
    prm = _lib.Params(0, 0, int(second_order), 1, 0, 0, int(cov_bias))
    cs = out.as_c()
    _lib.check("pisa_block_stats", lib.pisa_block_stats(
        ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
        _ptr(out.operands), out.operands.numel(), _ptr(ws), ws.numel(), _stream(k.device)))
    return out


def pisa_block_stats_noalloc(q, k, v, out: PisaStats, second_order=False, scale=None) -> PisaStats:
    """pisa_block_stats_noalloc: the statistics pass with the library's static
    scratch instead of a workspace. `out` (statistics and operand buffer) must
    be allocated by the caller beforehand; the call allocates nothing."""
    lib = library()
    _contig(q, k, v)
    if out.operands is None:
        raise ValueError("out.operands must be allocated by the caller")
    sh = _shape(k, scale)
    prm = _lib.Params(0, 0, int(second_order), 1, 0)
    cs = out.as_c()
    _lib.check("pisa_block_stats_noalloc", lib.pisa_block_stats_noalloc(
        ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
        _ptr(out.operands), out.operands.numel(), _stream(k.device)))
    return out


def pisa_prepare_operands(k, stats: PisaStats, second_order=False, scale=None) -> PisaStats:
    """Fill stats.operands from the statistics in `stats` (any source) and k."""
    lib = library()
    _contig(k, stats.kbar, stats.vsum, stats.hsum, stats.ksig2)
    sh = _shape(k, scale)
    if stats.operands is None:
        stats.operands = alloc_operands(k)
    prm = _lib.Params(0, 0, int(second_order), 1, 0)
    cs = stats.as_c()
    _lib.check("pisa_prepare_operands", lib.pisa_prepare_operands(
        ctypes.byref(sh), ctypes.byref(prm), _ptr(k), ctypes.byref(cs), _ptr(stats.operands),
        stats.operands.numel(), _stream(k.device)))
    return stats


def _operands(stats, required):
    if stats.operands is None:
        if required:
            raise ValueError("stats carry no operand buffer: run pisa_block_stats or pisa_prepare_operands")
        return None, 0
    return _ptr(stats.operands), stats.operands.numel()


def pisa_route_topk(q, stats: PisaStats, topk: int, band: int = 1, second_order=False, scale=None,
                    idx: torch.Tensor | None = None, wgate: torch.Tensor | None = None, n_sink: int = 0,
                    cov_bias=False):
    """q is used for its shape and device only; routing reads the pooled
    statistics (and with cov_bias the block heterogeneity stats.hnorm)."""
    lib = library()
    sh = _shape(q, scale)
    B, H, T, D = q.shape
    N = num_blocks(T)
    if idx is None:
        idx = torch.empty(B, H, N, topk, dtype=torch.int32, device=q.device)
    if second_order and wgate is None:
        wgate = torch.empty(B, H, N, N, dtype=torch.float32, device=q.device)
    prm = _lib.Params(int(topk), int(band), int(second_order), 1, 0, int(n_sink), int(cov_bias))
    cs = stats.as_c()
    ops, nops = _operands(stats, True)
    _lib.check("pisa_route_topk", lib.pisa_route_topk(
        ctypes.byref(sh), ctypes.byref(prm), ctypes.byref(cs), ops, nops,
        _ptr(idx) if topk else None, _ptr(wgate) if second_order else None, _stream(q.device)))
    return idx, (wgate if second_order else None)


def alloc_row_stats(q: torch.Tensor) -> torch.Tensor:
    """[B, H, T, 2] fp32: each row's lse and first-order weight c, as
    pisa_attn_fwd writes them for pisa_attn_bwd."""
    B, H, T, _ = q.shape
    return torch.empty(B, H, T, 2, dtype=torch.float32, device=q.device)


def _attn(fn_name, q, k, v, stats, idx, wgate, topk, band, second_order, first_order,
          phase_mask, scale, out, n_sink=0, row_stats=None):
    lib = library()
    _contig(q, k, v, idx, wgate, row_stats)
    if row_stats is not None and (row_stats.dtype != torch.float32 or row_stats.shape != (*q.shape[:3], 2)):
        raise ValueError("row_stats must be a float32 tensor of shape [B, H, T, 2]")
    sh = _shape(q, scale)
    o = out if out is not None else torch.empty_like(q)
    prm = _lib.Params(int(topk), int(band), int(second_order), int(first_order), int(phase_mask),
                      int(n_sink))
    cs = stats.as_c()
    ops, nops = _operands(stats, fn_name == "pisa_attn_fwd" and q.dtype == torch.bfloat16)
    fn = getattr(lib, fn_name)
    _lib.check(fn_name, fn(ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v),
                           ctypes.byref(cs), ops, nops, _ptr(idx) if topk else None,
                           _ptr(wgate) if second_order else None, _ptr(o),
                           None if row_stats is None else _ptr(row_stats), _stream(q.device)))
    return o


def pisa_attn_fwd(q, k, v, stats, idx, wgate=None, band=1, second_order=False, first_order=True,
                  phase_mask=0, scale=None, out=None, n_sink=0, row_stats=None):
    """o; with ``row_stats`` (alloc_row_stats) also each row's lse and c."""
    topk = 0 if idx is None else idx.shape[-1]
    return _attn("pisa_attn_fwd", q, k, v, stats, idx, wgate, topk, band, second_order,
                 first_order, phase_mask, scale, out, n_sink, row_stats)


def pisa_attn_fwd_valu(q, k, v, stats, idx, wgate=None, band=1, second_order=False,
                       first_order=True, phase_mask=0, scale=None, out=None, n_sink=0, row_stats=None):
    topk = 0 if idx is None else idx.shape[-1]
    return _attn("pisa_attn_fwd_valu", q, k, v, stats, idx, wgate, topk, band, second_order,
                 first_order, phase_mask, scale, out, n_sink, row_stats)


def pisa_attn_bwd(q, k, v, o, dout, stats, idx, wgate=None, band=1, second_order=False,
                  first_order=True, scale=None, n_sink=0, workspace=None, out=None, row_stats=None):
    """(dq, dk, dv) of sum(dout * o) for o = pisa_attn_fwd(q, k, v, stats, idx,
    wgate, ...) with the same arguments; the routing and the gate are held
    constant (pisa_attn_bwd). ``out`` may pass three preallocated tensors;
    ``row_stats`` what the forward wrote for this o (optional)."""
    lib = library()
    _contig(q, k, v, o, dout, idx, wgate, row_stats)
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, dout must share shape, dtype and device")
    sh = _shape(q, scale)
    topk = 0 if idx is None else idx.shape[-1]
    need = lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(sh))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    prm = _lib.Params(int(topk), int(band), int(second_order), int(first_order), 0, int(n_sink))
    cs = stats.as_c()
    _lib.check("pisa_attn_bwd", lib.pisa_attn_bwd(
        ctypes.byref(sh), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
        ctypes.byref(cs), _ptr(idx) if topk else None, _ptr(wgate) if second_order else None,
        None if row_stats is None else _ptr(row_stats),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def attn_fwd_plan(batch, heads, seq_len, head_dim, dtype, topk, band=1, second_order=False, n_sink=0) -> int:
    """The kernel pisa_attn_fwd runs for these arguments (pisa_attn_fwd_plan;
    host only): 1 persistent bf16 matrix-core kernel, 2 the non-persistent
    bf16 matrix-core kernel, 3 the fp32 matrix-core kernel (0, the vector
    kernel, only runs as pisa_attn_fwd_valu)."""
    code = PISA_BF16 if dtype in ("bf16", torch.bfloat16) else PISA_F32
    sh = _lib.Shape(batch, heads, seq_len, head_dim, BLOCK, code, 0.0)
    prm = _lib.Params(int(topk), int(band), int(second_order), 1, 0, int(n_sink))
    kern = ctypes.c_int32(-1)
    _lib.check("pisa_attn_fwd_plan", library().pisa_attn_fwd_plan(ctypes.byref(sh), ctypes.byref(prm),
                                                                   ctypes.byref(kern), None))
    return kern.value


def z_order(grid, prefix: int = 0) -> torch.Tensor:
    """Z-order (Morton) visiting order of ``prefix`` fixed tokens then a grid
    (slowest axis first), as an int32 CPU tensor: perm[i] is the raster token
    index placed at position i (pisa_z_order; host work, no GPU)."""
    grid = [int(g) for g in grid]
    n = int(prefix) + math.prod(grid)
    perm = torch.empty(n, dtype=torch.int32)
    g = (ctypes.c_int64 * len(grid))(*grid)
    _lib.check("pisa_z_order", _lib.load().pisa_z_order(
        g, len(grid), int(prefix), ctypes.cast(perm.data_ptr(), ctypes.POINTER(ctypes.c_int32)), n))
    return perm


def _reorder(fn_name, src, perm, bhtd, out_shape, out):
    if perm.dtype != torch.int32 or perm.dim() != 1 or perm.device != src.device:
        raise ValueError("perm must be an int32 vector on the tensor's device")
    if perm.numel() != bhtd[2]:
        raise ValueError("perm must have one entry per token")
    out = torch.empty(out_shape, dtype=src.dtype, device=src.device) if out is None else out
    _contig(src, perm, out)
    sh = _lib.Shape(*bhtd, BLOCK, _dtype_code(src), 0.0)
    _lib.check(fn_name, getattr(_lib.load(), fn_name)(
        ctypes.byref(sh), perm.data_ptr(), src.data_ptr(), out.data_ptr(), _stream(src.device)))
    return out


def reorder_gather(x: torch.Tensor, perm: torch.Tensor, out=None) -> torch.Tensor:
    """[B,T,H,D] -> [B,H,T,D] with out[b,h,i] = x[b, perm[i], h] (pisa_reorder_gather)."""
    B, T, H, D = x.shape
    return _reorder("pisa_reorder_gather", x, perm, (B, H, T, D), (B, H, T, D), out)


def reorder_scatter(o: torch.Tensor, perm: torch.Tensor, out=None) -> torch.Tensor:
    """[B,H,T,D] -> [B,T,H,D] with y[b, perm[i], h] = o[b,h,i] (pisa_reorder_scatter)."""
    B, H, T, D = o.shape
    return _reorder("pisa_reorder_scatter", o, perm, (B, H, T, D), (B, T, H, D), out)


class _Attention(torch.autograd.Function):
    """The three forward calls; backward = pisa_attn_bwd with the routing and
    gate of the forward (argument marshalling only)."""

    @staticmethod
    def forward(ctx, q, k, v, topk, band, second_order, scale, n_sink, cov_bias):
        st = pisa_block_stats(q, k, v, second_order=second_order, scale=scale, cov_bias=cov_bias)
        idx, wg = pisa_route_topk(q, st, topk, band=band, second_order=second_order, scale=scale,
                                  n_sink=n_sink, cov_bias=cov_bias)
        idx = idx if topk else None
        rs = alloc_row_stats(q)
        o = pisa_attn_fwd(q, k, v, st, idx, wg, band=band, second_order=second_order, scale=scale,
                          n_sink=n_sink, row_stats=rs)
        # the backward reads the statistics (not the operand buffer), the
        # routing table, the gated table and each row's lse and c: kept as
        # saved tensors
        ctx.save_for_backward(q, k, v, o, st.kbar, st.vsum, st.hsum, st.q2bar, st.ksig2, idx, wg, rs)
        ctx.cfg = (band, second_order, scale, n_sink)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, kbar, vsum, hsum, q2bar, ksig2, idx, wg, rs = ctx.saved_tensors
        band, so, scale, n_sink = ctx.cfg
        st = PisaStats(None, q2bar, kbar, vsum, ksig2, hsum, None)
        dq, dk, dv = pisa_attn_bwd(q, k, v, o, do.contiguous(), st, idx, wg, band=band,
                                   second_order=so, scale=scale, n_sink=n_sink, row_stats=rs)
        return dq, dk, dv, None, None, None, None, None, None


class _Gather(torch.autograd.Function):
    """reorder_gather; its adjoint is reorder_scatter."""

    @staticmethod
    def forward(ctx, x, perm):
        ctx.perm = perm
        return reorder_gather(x, perm)

    @staticmethod
    def backward(ctx, g):
        return reorder_scatter(g.contiguous(), ctx.perm), None


class _Scatter(torch.autograd.Function):
    """reorder_scatter; its adjoint is reorder_gather."""

    @staticmethod
    def forward(ctx, o, perm):
        ctx.perm = perm
        return reorder_scatter(o, perm)

    @staticmethod
    def backward(ctx, g):
        return reorder_gather(g.contiguous(), ctx.perm), None


def piecewise_sparse_attention(q, k, v, density=0.125, variant="pisa", band=1, scale=None,
                               n_sink_blocks=0, cov_bias=False, reorder="none", grid=None,
                               prefix=0):
    """PISA (variant="pisa") or PISA with the gated second-order term ("pwt").

    q, k, v: [B, H, T, D] bf16 or fp32 on the GPU. topk = floor(density * N)
    routed blocks per query block, plus the +-band and the first
    ``n_sink_blocks`` KV blocks (e.g. an MMDiT text prefix), are computed
    exactly. cov_bias=True routes with the covariance-aware prior
    log(||H_j - Hbar||_F + 1e-6) of the PISA paper's Eq. 11.
    With reorder="morton", q, k, v are token-major [B, T, H, D] in raster
    order over ``prefix`` fixed tokens then ``grid`` (slowest axis first); the
    tokens are gathered into Z-order (and [B, H, T, D]) before the operator and
    the output is scattered back to [B, T, H, D].
    Differentiable: with inputs that require grad, backward runs
    pisa_attn_bwd (the routing and gate of the forward held constant) and the
    reorder's adjoint.
    """
    if reorder not in ("none", "morton"):
        raise ValueError(reorder)
    if variant not in ("pisa", "pwt"):
        raise ValueError(variant)
    perm = None
    if reorder == "morton":
        if grid is None:
            raise ValueError('reorder="morton" needs the token grid')
        perm = z_order(grid, prefix).to(q.device)
        if perm.numel() != q.shape[1]:
            raise ValueError("prefix + prod(grid) must equal the token count")
        q, k, v = (_Gather.apply(t, perm) for t in (q, k, v))
    so = variant == "pwt"
    N = num_blocks(q.shape[2])
    topk = topk_for_density(density, N)
    topk = min(topk, N)
    n_sink_blocks = min(int(n_sink_blocks), N)
    o = _Attention.apply(q, k, v, topk, band, so, scale, n_sink_blocks, bool(cov_bias))
    return o if perm is None else _Scatter.apply(o, perm)
