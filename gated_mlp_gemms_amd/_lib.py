"""ctypes view of ``include/mlp.h`` and the loaded ``libgated_mlp.so`` (marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgated_mlp.so")

# enums of mlp.h
MLP_OK, MLP_ERR_INVALID_ARG, MLP_ERR_UNSUPPORTED, MLP_ERR_ALIGNMENT, MLP_ERR_WORKSPACE, MLP_ERR_HIP = range(6)
MLP_ACT_SWIGLU, MLP_ACT_RELU_SQ, MLP_ACT_GEGLU, MLP_ACT_REGLU, MLP_ACT_GLU, MLP_ACT_GELU_TANH, MLP_ACT_RELU = range(7)
MLP_F32, MLP_BF16, MLP_F16 = 0, 1, 2
MLP_GATE_OUTSIDE, MLP_GATE_INSIDE = 0, 1
MLP_PHASE_FWD, MLP_PHASE_FWD_INFER, MLP_PHASE_BWD = 0, 1, 2
MLP_FP8_E4M3, MLP_FP8_E5M2 = 0, 1
MLP_NOALLOC_SCRATCH_BYTES = 64 << 20
MLP_BWD_GROUPED, MLP_BWD_DW_DOWN_WITH_DACT = 1, 2
STAGES = ("up", "down", "recompute", "dact", "dw_down", "dx", "dw_up", "act", "widen", "bwd_gemms")


class MlpDesc(C.Structure):
    _fields_ = [
        ("M", C.c_int64), ("d_in", C.c_int64), ("hidden", C.c_int64), ("d_out", C.c_int64),
        ("act", C.c_int32), ("dtype", C.c_int32), ("gate_mult", C.c_float), ("down_mult", C.c_float),
        ("gate_mode", C.c_int32), ("recompute", C.c_int32), ("fp8_fwd", C.c_int32), ("fp8_bwd", C.c_int32),
        ("save_act", C.c_int32),
    ]


class MlpFp8(C.Structure):
    _fields_ = [
        ("x_q", C.c_void_p), ("w1_q", C.c_void_p), ("w2_q", C.c_void_p),
        ("s_x", C.c_void_p), ("s_w1", C.c_void_p), ("s_w2", C.c_void_p),
        ("s_post", C.c_void_p), ("post_amax", C.c_void_p),
        ("w1t_q", C.c_void_p), ("w2t_q", C.c_void_p), ("s_grad", C.c_void_p), ("s_dpre", C.c_void_p),
        ("dpre_amax", C.c_void_p),
    ]


_P = C.c_void_p
_SIGNATURES = {
    "mlp_workspace_bytes": (C.c_size_t, [C.POINTER(MlpDesc), C.c_int]),
    "mlp_fwd": (C.c_int, [C.POINTER(MlpDesc), _P, _P, _P, _P, _P, _P, C.POINTER(MlpFp8), _P, C.c_size_t, _P]),
    "mlp_fwd_infer": (C.c_int, [C.POINTER(MlpDesc), _P, _P, _P, _P, _P, C.POINTER(MlpFp8), _P, C.c_size_t, _P]),
    "mlp_fwd_infer_noalloc": (C.c_int, [C.POINTER(MlpDesc), _P, _P, _P, _P, _P, C.POINTER(MlpFp8), _P]),
    "mlp_bwd": (C.c_int, [C.POINTER(MlpDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_int,
                          C.POINTER(MlpFp8), _P, C.c_size_t, _P]),
    "mlp_quantize_workspace_bytes": (C.c_size_t, []),
    "mlp_quantize_e4m3": (C.c_int, [_P, C.c_int, C.c_int64, _P, _P, _P, C.c_size_t, _P]),
    "mlp_quantize_fp8": (C.c_int, [_P, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_int, _P, _P, _P, C.c_int64, _P]),
    "mlp_fp8_next_scale": (C.c_float, [C.c_float, C.c_float, C.c_float, C.c_float]),
    "mlp_quantize_weight_e4m3": (C.c_int, [_P, C.c_int, C.c_int64, C.c_int64, C.c_int, _P, _P, _P, _P, C.c_int64, _P]),
    "mlp_weight_amax_slots": (C.c_int64, [C.c_int64, C.c_int64]),
    "mlp_status_string": (C.c_char_p, [C.c_int]),
    "mlp_last_error": (C.c_char_p, []),
    "mlp_abi_version": (C.c_int, []),
    "mlp_time_stage_once": (C.c_int, [C.c_int, _P, _P]),
    "mlp_bwd_grouped": (C.c_int, [C.POINTER(MlpDesc), C.POINTER(C.c_int)]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gated_mlp_gemms_amd.build` "
                "(the MLP engine has no non-HIP fallback)")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class MlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        self.status = status
        super().__init__(f"{where}: {L.mlp_status_string(status).decode()}: {L.mlp_last_error().decode()}")


def check(status: int, where: str) -> None:
    if status != MLP_OK:
        raise MlpError(status, where)
