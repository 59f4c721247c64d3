"""ctypes loader for libvdtq.so (the C ABI declared in include/vdtq.h).

There is no fallback: if the library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvdtq.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
FMT_NVFP4, FMT_INT8, FMT_BF16, FMT_MXFP4, FMT_MXFP8 = 0, 1, 2, 3, 4
OUT_BF16, OUT_F32 = 0, 1
AMAX_GIVEN, STATS, GELU = 1, 2, 4
ACT_SKIP, ACT_NVFP4, ACT_INT8, ACT_BF16 = 0, 1, 2, 3
OP_HADAMARD_QUANTIZE, OP_BLOCK_STATS, OP_QGEMM = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 8 << 20      # VDTQ_NOALLOC_SCRATCH_BYTES

# every extern "C" symbol include/vdtq.h declares
EXPORTED = ["vdtq_last_error", "vdtq_version", "vdtq_workspace_bytes", "hadamard_quantize", "hadamard_quantize_noalloc",
            "qgemm_w4a4", "qgemm_w4a8", "qgemm_w4a16", "qgemm_mx", "qgemm_mx_quant", "block_stats", "block_stats_mx8", "dmpq_state_init", "dmpq_step", "dmpq_budget_gamma", "dmpq_depth_params",
            "vdtq_outlier_ratio"]


class DmpqParams(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_double), ("tau", ctypes.c_double), ("tau_acc", ctypes.c_double),
                ("rho", ctypes.c_double), ("tau_u", ctypes.c_double), ("warmup", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


class DmpqState(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("has_d1", ctypes.c_int32), ("has_d2", ctypes.c_int32),
                ("skipped_last", ctypes.c_int32), ("has_gamma", ctypes.c_int32),
                ("gamma_prev", ctypes.c_double), ("r_last", ctypes.c_double), ("acc", ctypes.c_double)]


class VdtqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vdtq error {code}: {msg}")
        self.code = code


_lib = None
_lock = threading.Lock()

vp, i64, sz, u32, i32, dbl = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint,
                              ctypes.c_int, ctypes.c_double)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built: run "
                                  "`python -m video_diffusion_transformer_block_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            L.vdtq_last_error.restype = ctypes.c_char_p
            L.vdtq_last_error.argtypes = []
            L.vdtq_version.restype = ctypes.c_char_p
            L.vdtq_version.argtypes = []
            L.vdtq_workspace_bytes.restype = sz
            L.vdtq_workspace_bytes.argtypes = [i32, i64, i64]
            L.hadamard_quantize.restype = i32
            L.hadamard_quantize.argtypes = [vp, i64, i64, i64, i32, i32, u32, vp, vp, vp, vp, vp, sz, vp]
            L.hadamard_quantize_noalloc.restype = i32
            L.hadamard_quantize_noalloc.argtypes = [vp, i64, i64, i64, i32, i32, u32, vp, vp, vp, vp, vp]
            L.qgemm_w4a4.restype = i32
            L.qgemm_w4a4.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i64, i64, i64, vp, sz, vp]
            L.qgemm_w4a16.restype = i32
            L.qgemm_w4a16.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i64, i64, i64, vp, sz, vp]
            L.qgemm_mx.restype = i32
            L.qgemm_mx.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i32, i64, i64, i64, vp, sz, vp]
            L.qgemm_mx_quant.restype = i32
            L.qgemm_mx_quant.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, u32, vp, vp, i64, i64, i64, vp]
            L.qgemm_w4a8.restype = i32
            L.qgemm_w4a8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i64, i64, i64, vp, sz, vp]
            L.block_stats_mx8.restype = i32
            L.block_stats_mx8.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
            L.block_stats.restype = i32
            L.block_stats.argtypes = [vp, vp, vp, vp, i64, vp, vp, sz, vp]
            L.dmpq_budget_gamma.restype = dbl
            L.dmpq_budget_gamma.argtypes = [ctypes.POINTER(ctypes.c_double), i32, dbl]
            L.dmpq_state_init.restype = None
            L.dmpq_state_init.argtypes = [ctypes.POINTER(DmpqState)]
            L.dmpq_step.restype = i32
            L.dmpq_step.argtypes = [ctypes.POINTER(DmpqParams), ctypes.POINTER(DmpqState),
                                    ctypes.POINTER(ctypes.c_double), dbl, ctypes.POINTER(ctypes.c_int)]
            L.dmpq_depth_params.restype = i32
            L.dmpq_depth_params.argtypes = [ctypes.POINTER(DmpqParams), i32, i32, dbl, dbl,
                                            ctypes.POINTER(DmpqParams)]
            L.vdtq_outlier_ratio.restype = dbl
            L.vdtq_outlier_ratio.argtypes = [dbl, dbl, i64]
            _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != OK:
        raise VdtqError(rc, lib().vdtq_last_error().decode())
