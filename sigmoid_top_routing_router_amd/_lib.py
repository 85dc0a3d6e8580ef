"""ctypes view of the C ABI declared in include/moe_mi355x.h.

Loading imports torch first so that the library binds to the HIP runtime that
torch already loaded (one runtime per process, so torch streams are valid
handles for the library).  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_RECOMPUTE_BIAS = 0x1
MOE_KEY32 = 0x2
MOE_PACKED_GATEUP = 0x4
MOE_ROUTE_FUSED = 0x8

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED_SHAPE",
                3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

EXPORTED = ["moe_route", "moe_eqb_workspace_bytes", "moe_eqb_bias", "moe_eqb_state_bytes",
            "moe_eqb_begin", "moe_eqb_accumulate", "moe_eqb_select", "moe_route_stats",
            "moe_lei_workspace_bytes", "moe_lei_backward",
            "moe_forward_workspace_bytes", "moe_forward", "moe_pack_gateup_weights",
            "moe_fp8_quantize_blocks",
            "moe_fp8_quantize_rows", "moe_forward_fp8_workspace_bytes", "moe_forward_fp8",
            "moe_forward_noalloc",
            "moe_status_string",
            "moe_last_error_message", "moe_abi_version", "moe_stage_timing",
            "moe_stage_times", "moe_stage_name"]
NUM_STAGES = 7
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


class MoeProblem(C.Structure):
    _fields_ = [("N", C.c_int64), ("d", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("h", C.c_int32), ("n_shared", C.c_int32), ("h_shared", C.c_int32),
                ("flags", C.c_uint32), ("logit_offset", C.c_void_p),
                ("logits_in", C.c_void_p)]


class MoeWeights(C.Structure):
    _fields_ = [("w_router", C.c_void_p), ("w_gate", C.c_void_p), ("w_up", C.c_void_p),
                ("w_down", C.c_void_p), ("ws_gate", C.c_void_p), ("ws_up", C.c_void_p),
                ("ws_down", C.c_void_p)]


class MoeFp8Weights(C.Structure):
    _fields_ = [("w_router", C.c_void_p), ("w_gate", C.c_void_p), ("s_gate", C.c_void_p),
                ("w_up", C.c_void_p), ("s_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_down", C.c_void_p), ("ws_gate", C.c_void_p), ("ss_gate", C.c_void_p),
                ("ws_up", C.c_void_p), ("ss_up", C.c_void_p), ("ws_down", C.c_void_p),
                ("ss_down", C.c_void_p)]


class MoeAux(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("topk_ids", C.c_void_p),
                ("topk_weights", C.c_void_p), ("alpha", C.c_void_p), ("margin", C.c_void_p),
                ("beta_out", C.c_void_p), ("quantile_out", C.c_void_p),
                ("counts_before", C.c_void_p), ("counts", C.c_void_p),
                ("offsets", C.c_void_p), ("sorted_src", C.c_void_p),
                ("src_pos", C.c_void_p)]


class MoeRouteStats(C.Structure):
    _fields_ = [("max_vio", C.c_double), ("intervention_rate", C.c_double),
                ("overlap", C.c_int64), ("near_ties", C.c_int64), ("max_load", C.c_int32),
                ("min_load", C.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sigmoid_top_routing_router_amd.build`")
    lib = C.CDLL(path)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    lib.moe_route.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_route.restype = C.c_int
    lib.moe_eqb_workspace_bytes.argtypes = [i64, i32, i32]
    lib.moe_eqb_workspace_bytes.restype = C.c_size_t
    lib.moe_eqb_bias.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, C.c_size_t, vp]
    lib.moe_eqb_bias.restype = C.c_int
    lib.moe_eqb_state_bytes.argtypes = [i32, i32]
    lib.moe_eqb_state_bytes.restype = C.c_size_t
    lib.moe_eqb_begin.argtypes = [i32, i32, vp, C.c_size_t, vp]
    lib.moe_eqb_begin.restype = C.c_int
    lib.moe_eqb_accumulate.argtypes = [i32, vp, vp, i64, i32, i32, vp, C.c_size_t, vp]
    lib.moe_eqb_accumulate.restype = C.c_int
    lib.moe_eqb_select.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp, C.c_size_t, vp]
    lib.moe_eqb_select.restype = C.c_int
    lib.moe_route_stats.argtypes = [vp, vp, vp, i64, i32, i32, C.c_float, vp, vp, vp]
    lib.moe_route_stats.restype = C.c_int
    lib.moe_lei_workspace_bytes.argtypes = [i32]
    lib.moe_lei_workspace_bytes.restype = C.c_size_t
    lib.moe_lei_backward.argtypes = [vp, vp, vp, i64, i32, i32, C.c_float, C.c_float, vp, vp, vp,
                                     vp, C.c_size_t, vp]
    lib.moe_lei_backward.restype = C.c_int
    lib.moe_forward_workspace_bytes.argtypes = [C.POINTER(MoeProblem)]
    lib.moe_forward_workspace_bytes.restype = C.c_size_t
    lib.moe_forward.argtypes = [C.POINTER(MoeProblem), C.POINTER(MoeWeights), vp, vp, vp,
                                C.POINTER(MoeAux), vp, C.c_size_t, vp]
    lib.moe_forward.restype = C.c_int
    lib.moe_pack_gateup_weights.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.moe_pack_gateup_weights.restype = C.c_int
    lib.moe_fp8_quantize_blocks.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.moe_fp8_quantize_blocks.restype = C.c_int
    lib.moe_fp8_quantize_rows.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_fp8_quantize_rows.restype = C.c_int
    lib.moe_forward_fp8_workspace_bytes.argtypes = [C.POINTER(MoeProblem)]
    lib.moe_forward_fp8_workspace_bytes.restype = C.c_size_t
    lib.moe_forward_fp8.argtypes = [C.POINTER(MoeProblem), C.POINTER(MoeFp8Weights), vp, vp, vp,
                                    C.POINTER(MoeAux), vp, C.c_size_t, vp]
    lib.moe_forward_fp8.restype = C.c_int
    lib.moe_forward_noalloc.argtypes = [C.POINTER(MoeProblem), C.POINTER(MoeWeights), vp, vp, vp,
                                        C.POINTER(MoeAux), vp]
    lib.moe_forward_noalloc.restype = C.c_int
    lib.moe_status_string.argtypes = [C.c_int]
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_last_error_message.argtypes = []
    lib.moe_last_error_message.restype = C.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = C.c_int32
    lib.moe_stage_timing.argtypes = [i32]
    lib.moe_stage_timing.restype = C.c_int
    lib.moe_stage_times.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int64)]
    lib.moe_stage_times.restype = C.c_int
    lib.moe_stage_name.argtypes = [i32]
    lib.moe_stage_name.restype = C.c_char_p
    _lib = lib
    return lib


def check(status: int):
    if status != MOE_OK:
        msg = _lib.moe_last_error_message().decode()
        raise MoeError(status, msg)
