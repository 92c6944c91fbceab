"""ctypes declarations of the C ABI in include/awq_mi355x.h."""
from __future__ import annotations

import ctypes
import os

#: the in-tree library; AWQ_MI355X_LIB may name another build of the same sources
LIB_PATH = os.environ.get("AWQ_MI355X_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libawq_mi355x.so")

AWQ_OK = 0
AWQ_ERR_INVALID_ARG = -1
AWQ_ERR_UNSUPPORTED = -2
AWQ_ERR_WORKSPACE = -3
AWQ_ERR_HIP = -4
AWQ_ERR_NONFINITE = -5
STAGE_PREPARE, STAGE_GRID, STAGE_SELECT, STAGE_ALL = 1, 2, 4, 7
STATUS_NAMES = {0: "AWQ_OK", -1: "AWQ_ERR_INVALID_ARG", -2: "AWQ_ERR_UNSUPPORTED",
                -3: "AWQ_ERR_WORKSPACE", -4: "AWQ_ERR_HIP", -5: "AWQ_ERR_NONFINITE"}

#: every symbol the header declares
EXPORTS = (
    "awq_default_config", "awq_last_error", "awq_version",
    "awq_act_stats_workspace_size", "awq_act_stats", "awq_act_stats_noalloc",
    "awq_search_plan_query", "awq_search_workspace_size", "awq_search_layer",
    "awq_search_layer_stages", "awq_pack", "awq_w4a16_matmul", "awq_fold_inverse_scale",
    "awq_select_top_channels",
)


class AwqConfig(ctypes.Structure):
    _fields_ = [("w_bit", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("n_grid", ctypes.c_int32), ("sal_floor", ctypes.c_float),
                ("zero_point", ctypes.c_int32)]


class AwqSearchPlan(ctypes.Structure):
    _fields_ = [("tile_tokens", ctypes.c_int64), ("tile_out", ctypes.c_int64),
                ("n_token_tiles", ctypes.c_int64), ("n_out_tiles", ctypes.c_int64),
                ("partials_offset", ctypes.c_size_t), ("scales_offset", ctypes.c_size_t),
                ("workspace_bytes", ctypes.c_size_t)]


class AwqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with post_bit_weight_awq_amd/build.py "
            "(hipcc, gfx950); the AWQ path has no CPU fallback")
    lib = ctypes.CDLL(path)
    P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    lib.awq_default_config.argtypes = [ctypes.POINTER(AwqConfig)]
    lib.awq_default_config.restype = None
    lib.awq_last_error.argtypes = []
    lib.awq_last_error.restype = ctypes.c_char_p
    lib.awq_version.argtypes = []
    lib.awq_version.restype = ctypes.c_char_p
    lib.awq_act_stats_workspace_size.argtypes = [I64, I64]
    lib.awq_act_stats_workspace_size.restype = SZ
    lib.awq_act_stats.argtypes = [P, I64, I64, P, P, SZ, P]
    lib.awq_act_stats.restype = I32
    lib.awq_act_stats_noalloc.argtypes = [P, I64, I64, P, P]
    lib.awq_act_stats_noalloc.restype = I32
    lib.awq_search_plan_query.argtypes = [I64, I64, I64, ctypes.POINTER(AwqConfig),
                                          ctypes.POINTER(AwqSearchPlan)]
    lib.awq_search_plan_query.restype = I32
    lib.awq_search_workspace_size.argtypes = [I64, I64, I64, ctypes.POINTER(AwqConfig)]
    lib.awq_search_workspace_size.restype = SZ
    lib.awq_search_layer.argtypes = [P, P, P, I64, I64, I64, ctypes.POINTER(AwqConfig),
                                     P, P, P, P, SZ, P]
    lib.awq_search_layer.restype = I32
    lib.awq_search_layer_stages.argtypes = [I32] + lib.awq_search_layer.argtypes
    lib.awq_search_layer_stages.restype = I32
    lib.awq_pack.argtypes = [P, P, I64, I64, ctypes.POINTER(AwqConfig), P, P, P, P]
    lib.awq_pack.restype = I32
    lib.awq_w4a16_matmul.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    lib.awq_w4a16_matmul.restype = I32
    lib.awq_fold_inverse_scale.argtypes = [P, P, I64, I64, P, P]
    lib.awq_fold_inverse_scale.restype = I32
    lib.awq_select_top_channels.argtypes = [P, I64, I64, P, P]
    lib.awq_select_top_channels.restype = I32
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != AWQ_OK:
        raise AwqError(rc, load().awq_last_error().decode())
