"""ctypes binding of libprism.so: the C structs and the function prototypes of
include/prism.h.  Loading fails loudly when the library has not been built; there is no
other implementation behind these names."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprism.so")
MAX_SHAPES = 32

PRISM_OK, PRISM_ERR_ARG, PRISM_ERR_DTYPE, PRISM_ERR_SHAPE, PRISM_ERR_LAUNCH = range(5)
PRISM_F32, PRISM_BF16 = 0, 1
STATUS_NAMES = {0: "PRISM_OK", 1: "PRISM_ERR_ARG", 2: "PRISM_ERR_DTYPE", 3: "PRISM_ERR_SHAPE", 4: "PRISM_ERR_LAUNCH"}


class PrismGrid(ctypes.Structure):
    _fields_ = [("T", c_int32), ("H", c_int32), ("W", c_int32), ("zt", c_int32), ("zh", c_int32), ("zw", c_int32)]


class PrismShapes(ctypes.Structure):
    _fields_ = [("n", c_int32), ("vol", c_int32), ("bt", c_int32 * MAX_SHAPES),
                ("bh", c_int32 * MAX_SHAPES), ("bw", c_int32 * MAX_SHAPES)]


class PrismShapeParams(ctypes.Structure):
    _fields_ = [("alpha", c_float), ("tau_lo", c_float), ("tau_hi", c_float), ("g_min", c_float), ("eps", c_float)]


class PrismSelectParams(ctypes.Structure):
    _fields_ = [("top_p", c_float), ("k_min", c_int32), ("k_max", c_int32)]


_P = c_void_p
_GP, _SP = POINTER(PrismGrid), POINTER(PrismShapes)
_SHP, _SLP = POINTER(PrismShapeParams), POINTER(PrismSelectParams)

# name -> (restype, argtypes), in the order of include/prism.h
PROTOTYPES = {
    "prism_num_zones": (c_int64, [_GP]),
    "prism_num_blocks": (c_int64, [_GP, _SP]),
    "prism_zone_stats": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, _P, _P]),
    "prism_zone_stats_global": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, _P, _P]),
    "prism_a2v_attn_norm": (c_int, [_P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, c_float, _P, _P, _P]),
    "prism_zone_stats_from_norm": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, c_int, _P, _P]),
    "prism_zone_stats_ex": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, c_int, _P, _P, _P]),
    "prism_assign_shapes_multi": (c_int, [_P, _P, c_int, c_int, _GP, _SP, _SHP, c_float, c_float, _P, _P, _P]),
    "prism_block_heads": (c_int, [_P, _P, c_int, c_int, _GP, _SP, _P, _P]),
    "prism_tiles_mixed_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "prism_blocks_to_tiles_mixed": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, _P, _P, _P, _P,
                                            _P, c_size_t, _P]),
    "prism_assign_shapes": (c_int, [_P, c_int, c_int, _GP, _SP, _SHP, _P, _P, _P]),
    "prism_permute": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, _SP, _P, c_int, _P, _P]),
    "prism_permute_pool": (c_int, [_P, _P, c_int, c_int, c_int, c_int, _GP, _SP, _P, _P, _P, _P]),
    "prism_select_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "prism_select_pooled_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "prism_select_blocks_pooled": (c_int, [_P, _P, _P, c_int, c_int, c_int, c_int, c_float, _SLP, _P, _P, _P, _P, _P,
                                           _P, c_size_t, _P]),
    "prism_tiles_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int]),
    "prism_blocks_to_tiles": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, _P, _P, _P, _P, _P,
                                      _P, c_size_t, _P]),
    "prism_select_blocks": (c_int, [_P, _P, c_int, _P, c_int, c_int, c_int, c_int, c_int, c_float, _SLP,
                                    _P, _P, _P, _P, _P, _P, c_size_t, _P]),
    "prism_fwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "prism_sparse_attn_fwd": (c_int, [_P, _P, _P, c_int, _P, _P, _P, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_float, _P, _P, _P, c_size_t, _P]),
    "prism_bwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "prism_sparse_attn_bwd": (c_int, [_P, _P, _P, _P, _P, _P, c_int, _P, _P, _P, c_int, _P, _P, c_int, c_int,
                                      c_int, c_int, c_int, c_float, _P, _P, _P, _P, c_size_t, _P, _P]),
    "prism_sparse_attn_bwd_noalloc": (c_int, [_P, _P, _P, _P, _P, _P, c_int, _P, _P, _P, c_int, _P, _P, c_int,
                                              c_int, c_int, c_int, c_int, c_float, _P, _P, _P, _P, _P]),
    "prism_dense_fwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "prism_dense_attn_fwd": (c_int, [_P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_float, _P, _P, _P,
                                     c_size_t, _P]),
    "prism_dense_bwd_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "prism_dense_attn_bwd": (c_int, [_P, _P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_float,
                                     _P, _P, _P, _P, c_size_t, _P, _P]),
    "prism_bench_mfma_peak": (c_int, [c_int, c_int, _P, _P, _P]),
    "prism_bench_tile_gather": (c_int, [_P, _P, _P, c_int, _P, _P, _P, c_int, c_int, c_int, c_int, c_int, c_int, _P,
                                        _P, c_size_t, _P]),
    "prism_bench_stream_read": (c_int, [_P, _P, c_size_t, _P, _P]),
    "prism_last_error": (c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises if libprism.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m content_adaptive_block_zone_amd.build`")
        lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class PrismError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, fn: str) -> None:
    if status != PRISM_OK:
        msg = load().prism_last_error().decode(errors="replace")
        raise PrismError(status, fn, msg)
