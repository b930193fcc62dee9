"""ctypes loader for libdynrad.so (the C ABI declared in include/dynrad.h).

The library must have been built (python -m block_sparse_attention_candidates_amd.build);
there is no fallback: loading fails loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdynrad.so")

DR_OK, DR_ERR_INVALID_ARG, DR_ERR_UNSUPPORTED, DR_ERR_CAPACITY, DR_ERR_HIP, DR_ERR_WAIT = range(6)
WAIT_ATTN_LOADER, WAIT_ATTN_COMPUTE, WAIT_TOKEN = 1, 2, 4
DR_STATIC_RATIO, DR_DYNAMIC_THRESHOLD = 0, 1


class RadialCfg(ctypes.Structure):
    _fields_ = [("num_frames", ctypes.c_int32), ("tokens_per_frame", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("gamma", ctypes.c_double), ("lambda_", ctypes.c_double),
                ("theta_c", ctypes.c_double), ("theta_m", ctypes.c_double)]


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SelectCfg(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("score_heads", ctypes.c_int32),
                ("ratio", ctypes.c_double), ("tau", ctypes.c_double)]


class TokenCfg(ctypes.Structure):
    _fields_ = [("fused_heads", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tau_near", ctypes.c_double), ("tau_far", ctypes.c_double), ("eps", ctypes.c_double)]


PROXY_WS_BYTES = 24576   # DR_PROXY_WS_BYTES


class StaticCfg(ctypes.Structure):
    _fields_ = [("rho_near", ctypes.c_double), ("rho_far", ctypes.c_double), ("seed", ctypes.c_uint64)]


class DynradError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"dynrad status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python -m block_sparse_attention_candidates_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    c_void_p, c_int32, c_int64, c_float, c_size_t = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                     ctypes.c_float, ctypes.c_size_t)
    sig = {
        "dr_num_blocks": (c_int64, [P(RadialCfg)]),
        "dr_distance_table": (c_int32, [P(RadialCfg), c_void_p, c_void_p]),
        "dr_build_candidates": (c_int32, [P(RadialCfg), c_void_p, c_void_p, c_int64, P(c_int64), c_void_p]),
        "dr_score_select_workspace": (c_int32, [P(Dims), P(RadialCfg), P(SelectCfg), c_int64, P(c_size_t)]),
        "dr_score_select": (c_int32, [P(Dims), P(RadialCfg), P(SelectCfg), c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]),
        "dr_token_select_workspace": (c_int32, [P(Dims), P(RadialCfg), P(TokenCfg), c_int64, P(c_size_t)]),
        "dr_token_select": (c_int32, [P(Dims), P(RadialCfg), P(TokenCfg), c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int64, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "dr_static_select_workspace": (c_int32, [P(RadialCfg), c_int64, P(c_size_t)]),
        "dr_static_select": (c_int32, [P(Dims), P(RadialCfg), P(StaticCfg), c_void_p, c_void_p, c_int64, c_void_p,
                                       c_void_p, c_void_p, c_size_t, c_void_p]),
        "dr_proxy_error": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_size_t,
                                     c_void_p]),
        "dr_proxy_loss": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_int64, ctypes.c_double,
                                    ctypes.c_double, c_void_p, c_void_p, c_size_t, c_void_p]),
        "dr_wait_report": (c_int32, [c_void_p, P(ctypes.c_uint32)]),
        "dr_set_wait_limit": (c_int32, [c_int64]),
        "dr_sparse_attn": (c_int32, [P(Dims), P(RadialCfg), c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                     c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
        "dr_sparse_attn_grouped": (c_int32, [P(Dims), P(RadialCfg), c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                             c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
        "dr_query_group_table": (c_int64, [P(RadialCfg), c_int32, c_void_p, c_int64]),
        "dr_query_groups_workspace": (c_int32, [P(Dims), P(c_size_t)]),
        "dr_query_groups": (c_int32, [P(Dims), P(RadialCfg), c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
        "dr_query_groups_noalloc": (c_int32, [P(Dims), P(RadialCfg), c_void_p, c_int64, c_void_p, c_void_p,
                                              c_void_p, c_void_p]),
        "dr_attn": (c_int32, [P(Dims), c_int32, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
        "dr_status_string": (ctypes.c_char_p, [c_int32]),
        "dr_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(status: int) -> None:
    if status != DR_OK:
        raise DynradError(status, lib().dr_last_error().decode())
