"""CPU checks of the C ABI: the library loads, exports every function that
include/pisa.h declares, and rejects invalid arguments before any HIP call
(so these run on a host without a GPU)."""

import ctypes
import os
import re

import pytest

from block_sparse_taylor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "pisa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pisa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.pisa_abi_version() == 15
    for code in range(9):
        assert lib.pisa_status_str(code)
    assert lib.pisa_status_str(99) == b"unknown status"


def shape(T=1024, D=64, dtype=_lib.PISA_BF16, B=1, H=2, block=64, scale=0.0):
    return _lib.Shape(B, H, T, D, block, dtype, scale)


@pytest.mark.parametrize("T,N", [(1, 1), (64, 1), (65, 2), (32760, 512), (118800, 1857), (524288, 8192)])
def test_num_blocks(lib, T, N):
    assert lib.pisa_num_blocks(ctypes.byref(shape(T=T))) == N


@pytest.mark.parametrize("bad", [
    dict(T=0), dict(T=524289), dict(D=96), dict(D=256), dict(block=32), dict(dtype=7),
    dict(B=0), dict(H=0), dict(B=300, H=300), dict(scale=float("nan")),
])
def test_invalid_shapes(lib, bad):
    s = shape(**bad)
    assert lib.pisa_num_blocks(ctypes.byref(s)) == -1
    assert lib.pisa_stats_workspace_bytes(ctypes.byref(s)) == 0


def test_workspace_bytes_fit_the_covariance_prior(lib):
    """With the prior the workspace also holds fp64 partial sums of H_j (half
    as many ranges as the fp32 partials, less one) and Hbar: never more than
    the fp32 partials when a head has four or more ranges."""
    for T, D, H in ((32760, 128, 40), (118800, 128, 24), (4608, 128, 24), (1000, 64, 2)):
        s = shape(T=T, D=D, H=H)
        N = -(-T // 64)
        groups = min(max(1, 512 // H), -(-N // 4))
        G = -(-N // -(-N // groups))
        fp32 = H * G * D * D * 4
        G2 = max(1, min(N, G // 2 - 1))
        assert lib.pisa_stats_workspace_bytes(ctypes.byref(s)) == max(fp32, H * (G2 + 1) * D * D * 8)


def test_workspace_bytes(lib):
    # one D x D fp32 partial per block range; a head gets max(1, 512 / heads)
    # ranges of at least 4 blocks: 12 ranges of 43 blocks for 40 heads of 512
    s = shape(T=32760, D=128, H=40)
    assert lib.pisa_stats_workspace_bytes(ctypes.byref(s)) == 40 * 12 * 128 * 128 * 4
    s = shape(T=1000, D=64, H=2)       # 16 blocks: four ranges of 4
    assert lib.pisa_stats_workspace_bytes(ctypes.byref(s)) == 2 * 4 * 64 * 64 * 4
    s = shape(T=4608, D=128, H=24)     # FLUX: 72 blocks, 18 ranges of 4
    assert lib.pisa_stats_workspace_bytes(ctypes.byref(s)) == 24 * 18 * 128 * 128 * 4


FAKE = 1 << 20          # 16-byte aligned fake device address: only used where validation fails first
MIS = FAKE + 4
GAP = 1 << 32           # fake buffers this far apart never overlap


def fake(n):
    """The n-th fake device buffer (distinct, non-overlapping)."""
    return FAKE + n * GAP


def stats(**kw):
    d = dict(qbar=fake(10), q2bar=None, kbar=fake(11), vsum=fake(12), ksig2=None, hsum=fake(13))
    d.update(kw)
    return _lib.Stats(**d)


OPS = fake(20)          # operand buffer
OPSB = 1 << 31          # its size (enough for every shape used here)


def call_stats(lib, s=None, p=None, q=fake(1), k=fake(2), v=fake(3), st=None, ops=OPS, opsb=OPSB,
               ws=fake(21), wsb=1 << 30):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_block_stats(ctypes.byref(s), ctypes.byref(p), q, k, v, ctypes.byref(st), ops, opsb, ws, wsb,
                                None)


def call_prepare(lib, s=None, p=None, k=fake(2), st=None, ops=OPS, opsb=OPSB):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_prepare_operands(ctypes.byref(s), ctypes.byref(p), k, ctypes.byref(st), ops, opsb, None)


def call_route(lib, s=None, p=None, st=None, ops=OPS, opsb=OPSB, idx=fake(30), wg=None):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_route_topk(ctypes.byref(s), ctypes.byref(p), ctypes.byref(st), ops, opsb, idx, wg, None)


def call_attn(lib, name="pisa_attn_fwd", s=None, p=None, q=fake(1), k=fake(2), v=fake(3),
              st=None, ops=OPS, opsb=OPSB, idx=fake(30), wg=None, o=fake(4), rs=None):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    fn = getattr(lib, name)
    return fn(ctypes.byref(s), ctypes.byref(p), q, k, v, ctypes.byref(st), ops, opsb, idx, wg, o, rs, None)


E = {n: c for c, n in _lib.STATUS_NAMES.items()}


def test_operand_buffer_layout(lib):
    """pisa_operands_bytes / pisa_operands_offsets: the arrangements in
    pisa_operand_t order, each 256-byte aligned; the bf16-only ones are empty
    for fp32 inputs."""
    def layout(**kw):
        sh = shape(**kw)
        off = (ctypes.c_int64 * len(_lib.OPERANDS))()
        assert lib.pisa_operands_offsets(ctypes.byref(sh), off) == 0
        return list(off), lib.pisa_operands_bytes(ctypes.byref(sh))
    rnd = lambda x: -(-x // 256) * 256
    B, H, N, D = 1, 40, 512, 128                        # Wan2.1-14B
    off, total = layout(T=32760, D=D, H=H)
    sizes = [H * N * D * 2, H * N * D * 2, H * 512 * D * 4, H * 512 * D * 4, H * N * 64 * D * 2,
             H * 8 * 64 * D * 2, H * 2 * D * D * 2, H * 512 * 4]
    want, at = [], 0
    for sz in sizes:
        want.append(at)
        at += rnd(sz)
    assert off == want and total == at
    off, total = layout(T=1000, D=64, H=2, dtype=_lib.PISA_F32)   # N = 16, fp32: no packed layouts
    sizes = [2 * 16 * 64 * 4, 2 * 16 * 64 * 4, 2 * 16 * 64 * 4, 2 * 16 * 64 * 4, 0, 0, 0, 2 * 16 * 4]
    want, at = [], 0
    for sz in sizes:
        want.append(at)
        at += rnd(sz)
    assert off == want and total == at
    assert lib.pisa_operands_bytes(ctypes.byref(shape(T=0))) == 0
    assert lib.pisa_operands_offsets(ctypes.byref(shape()), None) == E["PISA_ERR_NULL"]


def test_stats_validation(lib):
    assert call_stats(lib, k=None) == E["PISA_ERR_NULL"]
    assert call_stats(lib, q=MIS) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, st=stats(qbar=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, v=MIS) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, s=shape(D=32)) == E["PISA_ERR_SHAPE"]
    assert call_stats(lib, st=stats(hsum=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kbar=MIS)) == E["PISA_ERR_ALIGN"]
    # the operand buffer: required, aligned, at least pisa_operands_bytes
    need = lib.pisa_operands_bytes(ctypes.byref(shape()))
    assert call_stats(lib, ops=None) == E["PISA_ERR_NULL"]
    assert call_stats(lib, ops=MIS) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, opsb=need - 1) == E["PISA_ERR_WORKSPACE"]
    # second order needs ksig2 and q2bar
    assert call_stats(lib, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=fake(14))) == E["PISA_ERR_NULL"]
    assert call_stats(lib, ws=None) == E["PISA_ERR_NULL"]
    assert call_stats(lib, wsb=16) == E["PISA_ERR_WORKSPACE"]
    assert call_stats(lib, p=_lib.Params(4, 1, 2, 1, 0)) == E["PISA_ERR_PARAM"]
    # the covariance prior's block norms need hnorm
    assert call_stats(lib, p=_lib.Params(4, 1, 0, 1, 0, 0, 1)) == E["PISA_ERR_NULL"]
    # the operand buffer or the workspace inside an input, or each other
    assert call_stats(lib, ops=fake(2) + 4096) == E["PISA_ERR_PARAM"]
    assert call_stats(lib, ws=fake(3) + 256) == E["PISA_ERR_PARAM"]
    assert call_stats(lib, ws=OPS + 1024) == E["PISA_ERR_PARAM"]


def test_prepare_validation(lib):
    assert call_prepare(lib, k=None) == E["PISA_ERR_NULL"]               # bf16: kpack needs k
    assert call_prepare(lib, st=stats(kbar=None)) == E["PISA_ERR_NULL"]
    assert call_prepare(lib, st=stats(vsum=MIS)) == E["PISA_ERR_ALIGN"]
    assert call_prepare(lib, ops=None) == E["PISA_ERR_NULL"]
    assert call_prepare(lib, opsb=64) == E["PISA_ERR_WORKSPACE"]
    assert call_prepare(lib, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]   # second order: ksig2
    assert call_prepare(lib, ops=fake(2) + 256) == E["PISA_ERR_PARAM"]              # inside k
    assert call_prepare(lib, s=shape(dtype=5)) == E["PISA_ERR_DTYPE"]


def test_route_validation(lib):
    N = 16
    assert call_route(lib, p=_lib.Params(N + 1, 1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(-1, 1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(4, -1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, st=stats(qbar=None)) == E["PISA_ERR_NULL"]
    assert call_route(lib, idx=None) == E["PISA_ERR_NULL"]
    assert call_route(lib, st=stats(kbar=None)) == E["PISA_ERR_NULL"]
    assert call_route(lib, ops=None) == E["PISA_ERR_NULL"]
    assert call_route(lib, opsb=0) == E["PISA_ERR_WORKSPACE"]
    # second order: q2bar, ksig2 and wgate required
    so = _lib.Params(4, 1, 1, 1, 0)
    assert call_route(lib, p=so) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=so, st=stats(ksig2=fake(14))) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=so, st=stats(ksig2=fake(14), q2bar=fake(15))) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=so, st=stats(ksig2=fake(14), q2bar=MIS), wg=fake(31)) == E["PISA_ERR_ALIGN"]
    assert call_route(lib, s=shape(block=128)) == E["PISA_ERR_PARAM"]
    # covariance prior: 0 or 1, and it needs hnorm
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, 0, 2)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, 0, 1)) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, 0, 1), st=stats(hnorm=MIS)) == E["PISA_ERR_ALIGN"]
    # sink blocks: 0..N
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, -1)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, 17)) == E["PISA_ERR_PARAM"]


@pytest.mark.parametrize("name", ["pisa_attn_fwd", "pisa_attn_fwd_valu"])
def test_attn_validation(lib, name):
    assert call_attn(lib, name, o=None) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, o=fake(1)) == E["PISA_ERR_PARAM"]          # o aliases q
    assert call_attn(lib, name, o=fake(3) + 1024) == E["PISA_ERR_PARAM"]   # o overlaps v
    assert call_attn(lib, name, k=MIS) == E["PISA_ERR_ALIGN"]
    assert call_attn(lib, name, idx=None) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]   # wgate
    assert call_attn(lib, name, p=_lib.Params(4, 1, 0, 1, 8)) == E["PISA_ERR_PARAM"]  # phase mask
    assert call_attn(lib, name, p=_lib.Params(4, 1, 0, 3, 0)) == E["PISA_ERR_PARAM"]
    assert call_attn(lib, name, st=stats(hsum=None)) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, s=shape(dtype=2)) == E["PISA_ERR_DTYPE"]
    assert call_attn(lib, name, s=shape(T=10 ** 7)) == E["PISA_ERR_SHAPE"]
    # the optional row statistics: aligned, and sharing no byte with o or the inputs
    assert call_attn(lib, name, rs=MIS) == E["PISA_ERR_ALIGN"]
    assert call_attn(lib, name, rs=fake(4) + 4096) == E["PISA_ERR_PARAM"]   # inside o
    assert call_attn(lib, name, rs=fake(2)) == E["PISA_ERR_PARAM"]          # k
    assert call_attn(lib, name, rs=fake(4) - 1024) == E["PISA_ERR_PARAM"]   # runs into o
    if name == "pisa_attn_fwd":   # bf16: the matrix-core kernels read the operand buffer
        assert call_attn(lib, name, ops=None) == E["PISA_ERR_NULL"]
        assert call_attn(lib, name, opsb=1024) == E["PISA_ERR_WORKSPACE"]


def call_bwd(lib, s=None, p=None, q=fake(1), k=fake(2), v=fake(3), o=fake(4), do=fake(5),
             st=None, idx=fake(30), wg=None, dq=fake(6), dk=fake(7), dv=fake(8), ws=fake(9),
             wsb=1 << 31, rs=None):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_attn_bwd(ctypes.byref(s), ctypes.byref(p), q, k, v, o, do, ctypes.byref(st), idx, wg,
                             rs, dq, dk, dv, ws, wsb, None)


def test_bwd_workspace_bytes(lib):
    s = shape(T=1000, D=128, H=3)
    n = lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(s))
    N = 16
    # per-row statistics, bitmask rows, three per-block gradients, dH and its partial sums
    assert n >= 3 * 1000 * 16 + 3 * N * 4 + 3 * 3 * N * 128 * 4 + 3 * 2 * 128 * 128 * 4
    assert lib.pisa_attn_bwd_workspace_bytes(ctypes.byref(shape(T=0))) == 0


def test_bwd_validation(lib):
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv", "ws"):
        assert call_bwd(lib, **{name: None}) == E["PISA_ERR_NULL"], name
        assert call_bwd(lib, **{name: MIS}) == E["PISA_ERR_ALIGN"], name
    assert call_bwd(lib, idx=None) == E["PISA_ERR_NULL"]
    assert call_bwd(lib, st=stats(hsum=None)) == E["PISA_ERR_NULL"]
    assert call_bwd(lib, st=stats(qbar=None), wsb=0) == E["PISA_ERR_WORKSPACE"]        # qbar not needed
    so = _lib.Params(4, 1, 1, 1, 0)
    assert call_bwd(lib, p=so, wg=fake(31)) == E["PISA_ERR_NULL"]                          # ksig2
    assert call_bwd(lib, p=so, wg=fake(31), st=stats(ksig2=fake(14))) == E["PISA_ERR_NULL"]  # q2bar
    assert call_bwd(lib, p=so, st=stats(ksig2=fake(14), q2bar=fake(15))) == E["PISA_ERR_NULL"]  # wgate
    assert call_bwd(lib, p=_lib.Params(4, 1, 0, 1, 1)) == E["PISA_ERR_UNSUPPORTED"]   # phase mask
    assert call_bwd(lib, wsb=100) == E["PISA_ERR_WORKSPACE"]
    assert call_bwd(lib, dk=fake(6)) == E["PISA_ERR_PARAM"]                 # dq == dk
    assert call_bwd(lib, dk=fake(6) + 512) == E["PISA_ERR_PARAM"]           # dq overlaps dk
    assert call_bwd(lib, dv=fake(1)) == E["PISA_ERR_PARAM"]                 # dv == q
    assert call_bwd(lib, dv=fake(5) + 2048) == E["PISA_ERR_PARAM"]          # dv overlaps dout
    assert call_bwd(lib, dq=fake(9) + (1 << 20)) == E["PISA_ERR_PARAM"]     # dq inside the workspace
    assert call_bwd(lib, p=_lib.Params(4, 1, 0, 1, 0, 99)) == E["PISA_ERR_PARAM"]      # sinks > N
    assert call_bwd(lib, rs=MIS) == E["PISA_ERR_ALIGN"]                     # row statistics
    assert call_bwd(lib, rs=fake(6) + 4096) == E["PISA_ERR_PARAM"]          # inside dq
    assert call_bwd(lib, rs=fake(9) + 4096) == E["PISA_ERR_PARAM"]          # inside the workspace


def test_null_structs(lib):
    st = stats()
    p = _lib.Params(4, 1, 0, 1, 0)
    s = shape()
    assert lib.pisa_block_stats(None, ctypes.byref(p), fake(1), fake(2), fake(3), ctypes.byref(st), OPS, OPSB,
                                fake(21), 1 << 30, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_route_topk(ctypes.byref(s), None, ctypes.byref(st), OPS, OPSB, fake(30), None,
                               None) == E["PISA_ERR_NULL"]
    assert lib.pisa_route_topk(ctypes.byref(s), ctypes.byref(p), None, OPS, OPSB, fake(30), None,
                               None) == E["PISA_ERR_NULL"]
    assert lib.pisa_attn_fwd(ctypes.byref(s), ctypes.byref(p), fake(1), fake(2), fake(3), None, OPS, OPSB,
                             fake(30), None, fake(4), None, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_prepare_operands(ctypes.byref(s), ctypes.byref(p), fake(2), None, OPS, OPSB,
                                     None) == E["PISA_ERR_NULL"]


# ---------------------------------------------------------------- Morton reorder

def z_order_call(lib, grid, prefix=0, n=None):
    g = (ctypes.c_int64 * len(grid))(*grid)
    cells = 1
    for x in grid:
        cells *= x
    n = prefix + cells if n is None else n
    perm = (ctypes.c_int32 * max(n, 1))()
    return lib.pisa_z_order(g, len(grid), prefix, perm, n), list(perm)[:n]


@pytest.mark.parametrize("grid,prefix", [((21, 30, 52), 0), ((64, 64), 512), ((3, 5, 7), 2), ((1,), 0),
                                         ((2, 3, 5, 7), 1), ((33, 45, 80), 0)])
def test_z_order_host_helper_matches_oracle(lib, grid, prefix):
    """The library's host-side Z-order (C++) against the oracle's (numpy), bit for bit."""
    from oracle import reorder_oracle as R
    code, perm = z_order_call(lib, grid, prefix)
    assert code == 0
    assert perm == R.z_order(grid, prefix).tolist()


def test_z_order_validation(lib):
    g = (ctypes.c_int64 * 3)(4, 4, 4)
    perm = (ctypes.c_int32 * 64)()
    assert lib.pisa_z_order(None, 3, 0, perm, 64) == E["PISA_ERR_NULL"]
    assert lib.pisa_z_order(g, 3, 0, None, 64) == E["PISA_ERR_NULL"]
    assert lib.pisa_z_order(g, 0, 0, perm, 64) == E["PISA_ERR_SHAPE"]
    assert lib.pisa_z_order(g, 5, 0, perm, 64) == E["PISA_ERR_SHAPE"]
    assert lib.pisa_z_order(g, 3, -1, perm, 64) == E["PISA_ERR_SHAPE"]
    assert lib.pisa_z_order(g, 3, 0, perm, 63) == E["PISA_ERR_SHAPE"]        # n != prefix + cells
    assert z_order_call(lib, (0, 4))[0] == E["PISA_ERR_SHAPE"]
    assert z_order_call(lib, (1 << 16, 1 << 16), n=1)[0] == E["PISA_ERR_SHAPE"]   # > 2^31 - 1 tokens
    assert z_order_call(lib, (1 << 30,) * 3, n=1)[0] == E["PISA_ERR_SHAPE"]


@pytest.mark.parametrize("name", ["pisa_reorder_gather", "pisa_reorder_scatter"])
def test_reorder_validation(lib, name):
    fn = getattr(lib, name)
    s = shape(T=1000, D=64, H=2)
    nbytes = 2 * 1000 * 64 * 2
    ok_dst = FAKE + nbytes + 256
    assert fn(None, FAKE, FAKE, ok_dst, None) == E["PISA_ERR_NULL"]
    assert fn(ctypes.byref(s), None, FAKE, ok_dst, None) == E["PISA_ERR_NULL"]
    assert fn(ctypes.byref(s), FAKE, None, ok_dst, None) == E["PISA_ERR_NULL"]
    assert fn(ctypes.byref(s), FAKE, FAKE, None, None) == E["PISA_ERR_NULL"]
    assert fn(ctypes.byref(s), MIS, FAKE, ok_dst, None) == E["PISA_ERR_ALIGN"]
    assert fn(ctypes.byref(s), FAKE, MIS, ok_dst, None) == E["PISA_ERR_ALIGN"]
    assert fn(ctypes.byref(s), FAKE, FAKE, FAKE + 1024, None) == E["PISA_ERR_PARAM"]   # overlap
    assert fn(ctypes.byref(shape(D=96)), FAKE, FAKE, ok_dst, None) == E["PISA_ERR_SHAPE"]
    assert fn(ctypes.byref(shape(dtype=3)), FAKE, FAKE, ok_dst, None) == E["PISA_ERR_DTYPE"]


def plan(lib, T, D, topk, band=1, n_sink=0, second_order=0, dtype=_lib.PISA_BF16, phase_mask=0):
    sh = shape(T=T, D=D, dtype=dtype, H=1)
    prm = _lib.Params(topk, band, second_order, 1, phase_mask, n_sink)
    kern, items = ctypes.c_int32(-1), ctypes.c_int64(-1)
    st = lib.pisa_attn_fwd_plan(ctypes.byref(sh), ctypes.byref(prm), ctypes.byref(kern), ctypes.byref(items))
    return st, kern.value, items.value


ASM, MFMA, F32 = 1, 2, 3


@pytest.mark.parametrize("T,D,topk,band,n_sink,so,want_items,want_kernel", [
    # Wan2.1-14B: 3 forced + 64 routed = 67 exact items + 8 virtual groups
    (32760, 128, 64, 1, 0, 0, 75, ASM),
    # Hunyuan: 3 + 232 = 235 + 30 groups; second order changes nothing
    (118800, 128, 232, 1, 0, 1, 265, ASM),
    (118800, 128, 232, 1, 0, 0, 265, ASM),
    # N = 2048: 3 + 477 + 32 groups = 512 fills the list exactly; one more
    # routed id does not fit, with or without second order
    (131072, 128, 477, 1, 0, 1, 512, ASM),
    (131072, 128, 478, 1, 0, 1, 513, MFMA),
    (131072, 128, 478, 1, 0, 0, 513, MFMA),
    (131072, 128, 1000, 1, 0, 1, 1035, MFMA),
    # N = 8192, density 0.12: 3 + 983 + 128 groups = 1114
    (524288, 128, 983, 1, 0, 1, 1114, MFMA),
    # sinks count as forced blocks: N = 64, 3 + 32 + 4 = 39 + 1 group
    (4096, 128, 4, 1, 32, 0, 40, ASM),
    # ... but never more than N of them: N = 32, all forced, 32 + 4 = 36 + 1
    (2048, 128, 4, 1, 32, 0, 37, ASM),
    # head_dim 64 always runs the C++ matrix-core kernel; fp32 the fp32
    # matrix-core kernel (either head_dim)
    (32760, 64, 64, 1, 0, 0, 75, MFMA),
    (32760, 128, 64, 1, 0, 0, 75, F32),
    (1024, 64, 4, 1, 0, 0, 8, F32),
])
def test_attn_fwd_dispatch_rule(lib, T, D, topk, band, n_sink, so, want_items, want_kernel):
    """pisa_attn_fwd_plan: a wave of the persistent bf16 kernel lists a query
    block's E exact items and G virtual-token groups in a 512-entry LDS list, so
    it is chosen only where E + G fits, whatever the second-order switch says."""
    dtype = _lib.PISA_F32 if want_kernel == F32 else _lib.PISA_BF16
    st, kern, items = plan(lib, T, D, topk, band, n_sink, so, dtype)
    assert st == 0
    assert items == want_items
    assert kern == want_kernel


def test_attn_fwd_plan_clamps_band_and_validates(lib):
    # a band beyond N makes every block forced: N exact items, clamped in
    # 64-bit arithmetic (no int overflow for a band near 2^31)
    N = 1857
    for band in (N, N + 5, (1 << 31) - 1):
        st, kern, items = plan(lib, 118800, 128, 0, band=band)
        assert st == 0 and items == N + -(-N // 64)
        assert kern == MFMA     # 1857 + 30 > 512
    assert plan(lib, 118800, 128, 0, band=-1)[0] == 4          # PISA_ERR_PARAM
    assert plan(lib, 118800, 128, 1858)[0] == 4                 # topk > N
    assert plan(lib, 0, 128, 0)[0] == 2                         # PISA_ERR_SHAPE
    sh = shape(T=1024, D=128)
    prm = _lib.Params(4, 1, 0, 1, 0, 0)
    assert lib.pisa_attn_fwd_plan(ctypes.byref(sh), ctypes.byref(prm), None, None) == 0


def test_noalloc_stats_rejects_shapes_beyond_its_scratch(lib):
    """pisa_block_stats_noalloc runs only where the partial H sums fit the
    library's static scratch (PISA_STATS_SCRATCH_BYTES); beyond it the call
    returns PISA_ERR_WORKSPACE before any HIP call (so on this GPU-less host)."""
    p = _lib.Params(0, 0, 0, 1, 0)
    st = stats()
    def call(s):
        return lib.pisa_block_stats_noalloc(ctypes.byref(s), ctypes.byref(p), fake(1), fake(2), fake(3),
                                            ctypes.byref(st), OPS, OPSB, None)
    # 1024 heads of head_dim 128: one 64 KiB partial per head, 64 MiB
    big = _lib.Shape(1, 1024, 4096, 128, 64, _lib.PISA_BF16, 0.0)
    assert lib.pisa_stats_workspace_bytes(ctypes.byref(big)) > _lib.STATS_SCRATCH_BYTES
    assert call(big) == E["PISA_ERR_WORKSPACE"]
    # the Wan2.1-14B and Hunyuan shapes fit
    for T, H in ((32760, 40), (118800, 24)):
        sh = _lib.Shape(1, H, T, 128, 64, _lib.PISA_BF16, 0.0)
        assert lib.pisa_stats_workspace_bytes(ctypes.byref(sh)) <= _lib.STATS_SCRATCH_BYTES
    # validation as pisa_block_stats
    assert lib.pisa_block_stats_noalloc(ctypes.byref(shape()), ctypes.byref(p), None, fake(2), fake(3),
                                        ctypes.byref(st), OPS, OPSB, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_block_stats_noalloc(ctypes.byref(shape()), ctypes.byref(p), fake(1), fake(2), fake(3),
                                        ctypes.byref(st), OPS, 16, None) == E["PISA_ERR_WORKSPACE"]
