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
    assert lib.pisa_abi_version() == 10
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


def stats(**kw):
    d = dict(qbar=FAKE, q2bar=None, kbar=FAKE, vsum=FAKE, ksig2=None, hsum=FAKE, kbar_c=FAKE, vbar_c=FAKE,
             kpack=FAKE, hpack=FAKE, kbpack=FAKE, kbar_r=FAKE, ksig2_r=None)
    d.update(kw)
    return _lib.Stats(**d)


def call_stats(lib, s=None, p=None, q=FAKE, k=FAKE, v=FAKE, st=None, ws=FAKE, wsb=1 << 30):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_block_stats(ctypes.byref(s), ctypes.byref(p), q, k, v, ctypes.byref(st), ws, wsb, None)


def call_route(lib, s=None, p=None, st=None, idx=FAKE, wg=None):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_route_topk(ctypes.byref(s), ctypes.byref(p), ctypes.byref(st), idx, wg, None)


def call_attn(lib, name="pisa_attn_fwd", s=None, p=None, q=FAKE, k=FAKE + 64, v=FAKE + 128,
              st=None, idx=FAKE, wg=None, o=FAKE + 256):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    fn = getattr(lib, name)
    return fn(ctypes.byref(s), ctypes.byref(p), q, k, v, ctypes.byref(st), idx, wg, o, None)


E = {n: c for c, n in _lib.STATUS_NAMES.items()}


def test_stats_validation(lib):
    assert call_stats(lib, k=None) == E["PISA_ERR_NULL"]
    assert call_stats(lib, q=MIS) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, st=stats(qbar=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, v=MIS) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, s=shape(D=32)) == E["PISA_ERR_SHAPE"]
    assert call_stats(lib, st=stats(hsum=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kbar_c=MIS)) == E["PISA_ERR_ALIGN"]
    # kpack: required for bf16 inputs, ignored for fp32
    assert call_stats(lib, st=stats(kpack=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kpack=MIS)) == E["PISA_ERR_ALIGN"]
    assert call_stats(lib, st=stats(hpack=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kbpack=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kbar_r=None)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, st=stats(kbar_r=MIS)) == E["PISA_ERR_ALIGN"]
    # second order needs ksig2 and q2bar
    assert call_stats(lib, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=FAKE)) == E["PISA_ERR_NULL"]
    assert call_stats(lib, ws=None) == E["PISA_ERR_NULL"]
    assert call_stats(lib, wsb=16) == E["PISA_ERR_WORKSPACE"]
    assert call_stats(lib, p=_lib.Params(4, 1, 2, 1, 0)) == E["PISA_ERR_PARAM"]


def test_route_validation(lib):
    N = 16
    assert call_route(lib, p=_lib.Params(N + 1, 1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(-1, 1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(4, -1, 0, 1, 0)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, st=stats(qbar=None)) == E["PISA_ERR_NULL"]
    assert call_route(lib, idx=None) == E["PISA_ERR_NULL"]
    assert call_route(lib, st=stats(kbar=None)) == E["PISA_ERR_NULL"]
    assert call_route(lib, st=stats(kbar_r=None)) == E["PISA_ERR_NULL"]
    # second order: q2bar, ksig2 and wgate required
    assert call_route(lib, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=FAKE)) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=FAKE, q2bar=FAKE)) == E["PISA_ERR_NULL"]
    # ... and ksig2_r
    assert call_route(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=FAKE, q2bar=FAKE), wg=FAKE) == E["PISA_ERR_NULL"]
    assert call_route(lib, p=_lib.Params(4, 1, 1, 1, 0), st=stats(ksig2=FAKE, q2bar=FAKE, ksig2_r=MIS),
                      wg=FAKE) == E["PISA_ERR_ALIGN"]
    assert call_route(lib, s=shape(block=128)) == E["PISA_ERR_PARAM"]
    # sink blocks: 0..N
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, -1)) == E["PISA_ERR_PARAM"]
    assert call_route(lib, p=_lib.Params(4, 1, 0, 1, 0, 17)) == E["PISA_ERR_PARAM"]


@pytest.mark.parametrize("name", ["pisa_attn_fwd", "pisa_attn_fwd_valu"])
def test_attn_validation(lib, name):
    assert call_attn(lib, name, o=None) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, o=FAKE) == E["PISA_ERR_PARAM"]          # o aliases q
    assert call_attn(lib, name, k=MIS) == E["PISA_ERR_ALIGN"]
    assert call_attn(lib, name, idx=None) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, p=_lib.Params(4, 1, 1, 1, 0)) == E["PISA_ERR_NULL"]   # wgate
    assert call_attn(lib, name, p=_lib.Params(4, 1, 0, 1, 8)) == E["PISA_ERR_PARAM"]  # phase mask
    assert call_attn(lib, name, st=stats(kpack=None)) == E["PISA_ERR_NULL"]           # bf16 needs kpack
    assert call_attn(lib, name, st=stats(hpack=None)) == E["PISA_ERR_NULL"]           # and hpack
    assert call_attn(lib, name, p=_lib.Params(4, 1, 0, 3, 0)) == E["PISA_ERR_PARAM"]
    assert call_attn(lib, name, st=stats(vbar_c=None)) == E["PISA_ERR_NULL"]
    assert call_attn(lib, name, s=shape(dtype=2)) == E["PISA_ERR_DTYPE"]
    assert call_attn(lib, name, s=shape(T=10 ** 7)) == E["PISA_ERR_SHAPE"]


def call_bwd(lib, s=None, p=None, q=FAKE, k=FAKE + 64, v=FAKE + 128, o=FAKE + 192, do=FAKE + 256,
             st=None, idx=FAKE, wg=None, dq=FAKE + 320, dk=FAKE + 384, dv=FAKE + 448, ws=FAKE + 512,
             wsb=1 << 40):
    s = s or shape()
    p = p or _lib.Params(4, 1, 0, 1, 0)
    st = st or stats()
    return lib.pisa_attn_bwd(ctypes.byref(s), ctypes.byref(p), q, k, v, o, do, ctypes.byref(st), idx, wg,
                             dq, dk, dv, ws, wsb, None)


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
    assert call_bwd(lib, st=stats(kpack=None, hpack=None, kbpack=None, kbar_c=None, vbar_c=None),
                    wsb=0) == E["PISA_ERR_WORKSPACE"]                                  # packs not needed
    so = _lib.Params(4, 1, 1, 1, 0)
    assert call_bwd(lib, p=so, wg=FAKE) == E["PISA_ERR_NULL"]                          # ksig2
    assert call_bwd(lib, p=so, wg=FAKE, st=stats(ksig2=FAKE)) == E["PISA_ERR_NULL"]    # q2bar
    assert call_bwd(lib, p=so, st=stats(ksig2=FAKE, q2bar=FAKE)) == E["PISA_ERR_NULL"]  # wgate
    assert call_bwd(lib, p=_lib.Params(4, 1, 0, 1, 1)) == E["PISA_ERR_UNSUPPORTED"]   # phase mask
    assert call_bwd(lib, wsb=100) == E["PISA_ERR_WORKSPACE"]
    assert call_bwd(lib, dk=FAKE + 320) == E["PISA_ERR_PARAM"]                          # dq == dk
    assert call_bwd(lib, dv=FAKE) == E["PISA_ERR_PARAM"]                                # dv == q
    assert call_bwd(lib, dq=FAKE + 512) == E["PISA_ERR_PARAM"]                          # dq == workspace
    assert call_bwd(lib, p=_lib.Params(4, 1, 0, 1, 0, 99)) == E["PISA_ERR_PARAM"]      # sinks > N


def test_null_structs(lib):
    st = stats()
    p = _lib.Params(4, 1, 0, 1, 0)
    s = shape()
    assert lib.pisa_block_stats(None, ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(st), FAKE, 1 << 30, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_route_topk(ctypes.byref(s), None, ctypes.byref(st), FAKE, None, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_route_topk(ctypes.byref(s), ctypes.byref(p), None, FAKE, None, None) == E["PISA_ERR_NULL"]
    assert lib.pisa_attn_fwd(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE + 64, FAKE + 128, None, FAKE, None, FAKE + 256, None) == E["PISA_ERR_NULL"]


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


ASM, MFMA, VALU = 1, 2, 0


@pytest.mark.parametrize("T,D,topk,band,n_sink,so,want_items,want_kernel", [
    # Wan2.1-14B: 3 forced + 64 routed = 67 exact (17 on wave 0) + 8 groups (2)
    (32760, 128, 64, 1, 0, 0, 19, ASM),
    # Hunyuan: 3 + 232 = 235 (59) + 30 groups (8); second order changes nothing
    (118800, 128, 232, 1, 0, 1, 67, ASM),
    (118800, 128, 232, 1, 0, 0, 67, ASM),
    # the window the persistent kernel must leave: N = 2048, 3 + 1000 exact
    # (251 on wave 0) + 32 groups (8) = 259 > 256, with or without second order
    (131072, 128, 1000, 1, 0, 1, 259, MFMA),
    (131072, 128, 1000, 1, 0, 0, 259, MFMA),
    # largest list that still fits: 3 + 989 = 992 (248) + 8 = 256
    (131072, 128, 989, 1, 0, 1, 256, ASM),
    (131072, 128, 990, 1, 0, 1, 257, MFMA),
    # N = 8192, density 0.12: 3 + 983 (247) + 128 groups (32) = 279
    (524288, 128, 983, 1, 0, 1, 279, MFMA),
    # sinks count as forced blocks: N = 64, 3 + 32 + 4 = 39 (10) + 1 group (1)
    (4096, 128, 4, 1, 32, 0, 11, ASM),
    # ... but never more than N of them: N = 32, all forced, 32 + 4 = 36 (9) + 1
    (2048, 128, 4, 1, 32, 0, 10, ASM),
    # head_dim 64 always runs the C++ matrix-core kernel; fp32 the VALU kernel
    (32760, 64, 64, 1, 0, 0, 19, MFMA),
    (32760, 128, 64, 1, 0, 0, 19, VALU),
])
def test_attn_fwd_dispatch_rule(lib, T, D, topk, band, n_sink, so, want_items, want_kernel):
    """pisa_attn_fwd_plan: the persistent bf16 kernel lists ceil(E/4) exact items
    and ceil(G/4) virtual-token groups per wave in a 256-entry LDS list, so it is
    chosen only where that bound fits, whatever the second-order switch says."""
    dtype = _lib.PISA_F32 if want_kernel == VALU else _lib.PISA_BF16
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
        assert st == 0 and items == -(-N // 4) + -(-(-(-N // 64)) // 4)
        assert kern == MFMA     # 465 + 8 > 256
    assert plan(lib, 118800, 128, 0, band=-1)[0] == 4          # PISA_ERR_PARAM
    assert plan(lib, 118800, 128, 1858)[0] == 4                 # topk > N
    assert plan(lib, 0, 128, 0)[0] == 2                         # PISA_ERR_SHAPE
    sh = shape(T=1024, D=128)
    prm = _lib.Params(4, 1, 0, 1, 0, 0)
    assert lib.pisa_attn_fwd_plan(ctypes.byref(sh), ctypes.byref(prm), None, None) == 0
