"""ctypes declarations of libpisa's C ABI (include/pisa.h)."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpisa.so")

PISA_OK = 0
STATUS_NAMES = {
    0: "PISA_OK", 1: "PISA_ERR_NULL", 2: "PISA_ERR_SHAPE", 3: "PISA_ERR_DTYPE",
    4: "PISA_ERR_PARAM", 5: "PISA_ERR_ALIGN", 6: "PISA_ERR_UNSUPPORTED", 7: "PISA_ERR_HIP",
    8: "PISA_ERR_WORKSPACE",
}
PISA_F32, PISA_BF16 = 0, 1

EXPORTED = (
    "pisa_abi_version", "pisa_status_str", "pisa_num_blocks", "pisa_stats_workspace_bytes",
    "pisa_block_stats", "pisa_route_topk", "pisa_attn_fwd", "pisa_attn_fwd_valu",
    "pisa_z_order", "pisa_reorder_gather", "pisa_reorder_scatter", "pisa_attn_bwd_workspace_bytes",
    "pisa_attn_bwd", "pisa_attn_fwd_plan", "pisa_operands_bytes", "pisa_operands_offsets",
    "pisa_prepare_operands", "pisa_block_stats_noalloc",
)
STATS_SCRATCH_BYTES = 32 << 20   # PISA_STATS_SCRATCH_BYTES
COV_EPS = 1e-6                   # PISA_COV_EPS
# pisa_operand_t: the arrangements inside the operand buffer
OPERANDS = ("kbar_c", "vbar_c", "kbar_r", "ksig2_r", "kpack", "kbpack", "hpack", "knorm")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class Params(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_int32), ("band", ctypes.c_int32), ("second_order", ctypes.c_int32),
                ("first_order", ctypes.c_int32), ("phase_mask", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("cov_bias", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("qbar", ctypes.c_void_p), ("q2bar", ctypes.c_void_p), ("kbar", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p), ("ksig2", ctypes.c_void_p), ("hsum", ctypes.c_void_p),
                ("hnorm", ctypes.c_void_p)]


class PisaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(code, code)}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpisa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m block_sparse_taylor_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.pisa_abi_version.restype = ctypes.c_int
    lib.pisa_abi_version.argtypes = []
    lib.pisa_status_str.restype = ctypes.c_char_p
    lib.pisa_status_str.argtypes = [ctypes.c_int]
    lib.pisa_num_blocks.restype = ctypes.c_int64
    lib.pisa_num_blocks.argtypes = [P(Shape)]
    lib.pisa_stats_workspace_bytes.restype = ctypes.c_size_t
    lib.pisa_stats_workspace_bytes.argtypes = [P(Shape)]
    lib.pisa_operands_bytes.restype = ctypes.c_size_t
    lib.pisa_operands_bytes.argtypes = [P(Shape)]
    lib.pisa_operands_offsets.restype = ctypes.c_int
    lib.pisa_operands_offsets.argtypes = [P(Shape), P(ctypes.c_int64)]
    lib.pisa_block_stats.restype = ctypes.c_int
    lib.pisa_block_stats.argtypes = [P(Shape), P(Params), vp, vp, vp, P(Stats), vp, ctypes.c_size_t, vp,
                                     ctypes.c_size_t, vp]
    lib.pisa_block_stats_noalloc.restype = ctypes.c_int
    lib.pisa_block_stats_noalloc.argtypes = [P(Shape), P(Params), vp, vp, vp, P(Stats), vp, ctypes.c_size_t, vp]
    lib.pisa_prepare_operands.restype = ctypes.c_int
    lib.pisa_prepare_operands.argtypes = [P(Shape), P(Params), vp, P(Stats), vp, ctypes.c_size_t, vp]
    lib.pisa_route_topk.restype = ctypes.c_int
    lib.pisa_route_topk.argtypes = [P(Shape), P(Params), P(Stats), vp, ctypes.c_size_t, vp, vp, vp]
    for name in ("pisa_attn_fwd", "pisa_attn_fwd_valu"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P(Shape), P(Params), vp, vp, vp, P(Stats), vp, ctypes.c_size_t, vp, vp, vp, vp, vp]
    lib.pisa_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.pisa_attn_bwd_workspace_bytes.argtypes = [P(Shape)]
    lib.pisa_attn_bwd.restype = ctypes.c_int
    lib.pisa_attn_bwd.argtypes = [P(Shape), P(Params), vp, vp, vp, vp, vp, P(Stats), vp, vp, vp, vp, vp, vp,
                                  vp, ctypes.c_size_t, vp]
    lib.pisa_attn_fwd_plan.restype = ctypes.c_int
    lib.pisa_attn_fwd_plan.argtypes = [P(Shape), P(Params), P(ctypes.c_int32), P(ctypes.c_int64)]
    lib.pisa_z_order.restype = ctypes.c_int
    lib.pisa_z_order.argtypes = [P(ctypes.c_int64), ctypes.c_int32, ctypes.c_int64, P(ctypes.c_int32),
                                 ctypes.c_int64]
    for name in ("pisa_reorder_gather", "pisa_reorder_scatter"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P(Shape), vp, vp, vp, vp]
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != PISA_OK:
        raise PisaError(fn, code)
