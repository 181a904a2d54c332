"""ctypes declarations for libfp8attn.so (include/fp8attn.h).

Argument marshalling only.  The library must have been built in-tree
(``python -m fp8_flash_attention_amd.build``); if it is missing, loading fails
loudly instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8attn.so")

OK, EINVAL, EUNSUPPORTED, ENOMEM, EWORKSPACE, EHIP = range(6)
STATUS_NAMES = {0: "FP8ATTN_OK", 1: "FP8ATTN_EINVAL", 2: "FP8ATTN_EUNSUPPORTED",
                3: "FP8ATTN_ENOMEM", 4: "FP8ATTN_EWORKSPACE", 5: "FP8ATTN_EHIP"}
REGION_Q, REGION_K, REGION_V, REGION_SCALES, REGION_MU, REGION_ROWMAP = range(6)
REGION_Q_BSCALES, REGION_K_BSCALES, REGION_V_BSCALES, REGION_QM_CODES, REGION_QM_SCALES = range(6, 11)
REGION_STATS = 11
REGION_QMEAN, REGION_QM_TERM = 12, 13
PLAN_SEGMENT_SCALES = 1          # FP8ATTN_PLAN_SEGMENT_SCALES
PLAN_MXFP4 = 2                   # FP8ATTN_PLAN_MXFP4
PLAN_Q_CENTRE = 4                # FP8ATTN_PLAN_Q_CENTRE
PLAN_CAUSAL = 8                  # FP8ATTN_PLAN_CAUSAL
PLAN_HEAD_DIM_64 = 16            # FP8ATTN_PLAN_HEAD_DIM_64
PLAN_EXACT_PROBS = 32            # FP8ATTN_PLAN_EXACT_PROBS


def plan_head_dim(d: int) -> int:
    """FP8ATTN_PLAN_HEAD_DIM(d): the head size in bits 8..12 of the plan flags."""
    return (int(d) // 8) << 8
PLAN_INFO_LEN = 14

# Every symbol include/fp8attn.h declares, with (restype, argtypes).
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
SIGNATURES = {
    "fp8attn_plan": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64, ctypes.c_int32,
                                    _i32p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32]),
    "fp8attn_plan_ex": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64, ctypes.c_int32,
                                       _i32p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_uint32]),
    "fp8attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p]),
    "fp8attn_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        _i64p, _i64p, _i64p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fp8attn_quantize_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, _i64p, _i64p, _i64p, ctypes.c_void_p,
                                                ctypes.c_size_t, ctypes.c_void_p]),
    "fp8attn_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       _i64p, ctypes.c_void_p, ctypes.c_void_p]),
    "fp8attn_workspace_region": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_void_p), _i64p]),
    "fp8attn_plan_info": (ctypes.c_int, [ctypes.c_void_p, _i64p]),
    "fp8attn_plan_work_items": (ctypes.c_int, [ctypes.c_void_p, _i32p, ctypes.c_int64, _i64p]),
    "fp8attn_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "fp8attn_last_error": (ctypes.c_char_p, []),
    # include/fp8attn_bench.h
    "fp8attn_mfma_peak": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double)]),
}

_lib = None


class Fp8AttnError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {text}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m fp8_flash_attention_amd.build` "
                "(the HIP library is required; there is no other code path)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def check(status: int, where: str) -> None:
    if status != OK:
        raise Fp8AttnError(status, where, lib().fp8attn_last_error().decode())


def i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))(*vals)
    return arr
