"""ctypes mirror of include/miconv.h and the loader of the in-tree library.

The library is loaded on first use.  There is no fallback: if
``libmiconv.so`` is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

MAX_RANK = 5
MAX_SPATIAL = 3

F32, F16, BF16 = 0, 1, 2
OK, EINVAL, EUNSUPPORTED, ELAYOUT, EALIGN, EDEVICE, ENOSPACE = range(7)
NOALLOC_SCRATCH_BYTES = 32 << 20
PLAN_ONE_BY_ONE = 1
PLAN_TUNED = 2
PAD_EXPLICIT, PAD_SAME, PAD_VALID = 0, 1, 2
K_AUTO, K_DW_CL, K_PLANE, K_GRP, K_REDUCE, K_IGEMM, K_IGEMM_T = -1, 1, 2, 3, 4, 5, 6
KERNELS = {"auto": K_AUTO, "dw_cl": K_DW_CL, "plane": K_PLANE, "grp": K_GRP, "reduce": K_REDUCE,
           "igemm": K_IGEMM, "igemm_t": K_IGEMM_T}

_i32, _i64 = ctypes.c_int32, ctypes.c_int64


class ConvTensor(ctypes.Structure):
    _fields_ = [("rank", _i32), ("dtype", _i32), ("sizes", _i64 * MAX_RANK),
                ("strides", _i64 * MAX_RANK)]


class ConvArgs(ctypes.Structure):
    _fields_ = [("transposed", _i32), ("padding_mode", _i32), ("groups", _i64),
                ("n_stride", _i32), ("n_padding", _i32), ("n_dilation", _i32),
                ("n_output_padding", _i32),
                ("stride", _i64 * MAX_SPATIAL), ("padding_before", _i64 * MAX_SPATIAL),
                ("padding_after", _i64 * MAX_SPATIAL), ("dilation", _i64 * MAX_SPATIAL),
                ("output_padding", _i64 * MAX_SPATIAL)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("spatial", _i32), ("transposed", _i32), ("unbatched", _i32), ("dtype", _i32),
                ("has_bias", _i32), ("reserved0", _i32),
                ("N", _i64), ("C_in", _i64), ("C_out", _i64), ("groups", _i64),
                ("in_", _i64 * MAX_SPATIAL), ("k", _i64 * MAX_SPATIAL),
                ("out", _i64 * MAX_SPATIAL), ("stride", _i64 * MAX_SPATIAL),
                ("padding_before", _i64 * MAX_SPATIAL), ("padding_after", _i64 * MAX_SPATIAL),
                ("dilation", _i64 * MAX_SPATIAL), ("output_padding", _i64 * MAX_SPATIAL),
                ("x", ConvTensor), ("w", ConvTensor), ("b", ConvTensor)]


class ConvPlan(ctypes.Structure):
    _fields_ = [("d", ConvDesc), ("y", ConvTensor),
                ("kernel", _i32), ("variant", _i32), ("vec_ok", _i32), ("index64", _i32),
                ("workspace_bytes", _i64), ("tile", _i64 * 8), ("grid", _i64 * 3),
                ("block", _i32), ("lds_bytes", _i32), ("flags", _i32), ("batch_chunk", _i32), ("flops", _i64),
                ("bytes", _i64)]


class ConvBwdPlan(ctypes.Structure):
    _fields_ = [("d", ConvDesc), ("gy", ConvTensor), ("dx", ConvTensor), ("dw", ConvTensor), ("db", ConvTensor),
                ("need_dx", _i32), ("need_dw", _i32), ("need_db", _i32), ("dgrad_flip", _i32),
                ("dgrad", ConvPlan), ("wg_tile", _i64 * 8), ("db_splits", _i64), ("workspace_bytes", _i64),
                ("flops", _i64 * 3), ("bytes", _i64 * 3)]


class ConvPlanOpts(ctypes.Structure):
    _fields_ = [("force_kernel", _i32), ("force_variant", _i32), ("reserved", _i32 * 6)]


LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmiconv.so")

# Every symbol include/miconv.h declares.
EXPORTS = ("conv_bind", "conv_out_shape", "conv_plan", "conv_plan_ex", "conv_run", "conv_run_noalloc",
           "conv_backward_layout", "conv_plan_backward", "conv_run_backward",
           "conv_plan_candidates", "conv_tune", "conv_plan_tuned",
           "conv_kernel_name", "conv_status_string", "conv_abi_version")

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m depthwise_stencil_implicit_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.conv_bind.argtypes = [P(ConvTensor), P(ConvTensor), P(ConvTensor), P(ConvArgs),
                                P(ConvDesc), ctypes.c_char_p, ctypes.c_size_t]
        L.conv_bind.restype = ctypes.c_int
        L.conv_out_shape.argtypes = [P(ConvDesc), P(ConvTensor)]
        L.conv_out_shape.restype = ctypes.c_int
        L.conv_plan.argtypes = [P(ConvDesc), P(ConvTensor), _i32, P(ConvPlan)]
        L.conv_plan.restype = ctypes.c_int
        L.conv_plan_ex.argtypes = [P(ConvDesc), P(ConvTensor), P(ConvPlanOpts), P(ConvPlan)]
        L.conv_plan_ex.restype = ctypes.c_int
        L.conv_run.argtypes = [P(ConvPlan), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.conv_run.restype = ctypes.c_int
        L.conv_run_noalloc.argtypes = [P(ConvPlan), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.conv_run_noalloc.restype = ctypes.c_int
        L.conv_backward_layout.argtypes = [P(ConvDesc), P(ConvTensor), P(ConvTensor), P(ConvTensor), P(ConvTensor)]
        L.conv_backward_layout.restype = ctypes.c_int
        L.conv_plan_backward.argtypes = [P(ConvDesc), P(ConvTensor), _i32, _i32, _i32, P(ConvBwdPlan)]
        L.conv_plan_backward.restype = ctypes.c_int
        L.conv_run_backward.argtypes = [P(ConvBwdPlan)] + [ctypes.c_void_p] * 7 + [ctypes.c_size_t, ctypes.c_void_p]
        L.conv_run_backward.restype = ctypes.c_int
        L.conv_plan_candidates.argtypes = [P(ConvDesc), P(ConvTensor), P(ConvPlan), _i32, P(_i32)]
        L.conv_plan_candidates.restype = ctypes.c_int
        L.conv_tune.argtypes = [P(ConvDesc), P(ConvTensor)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t,
                                                                                        ctypes.c_void_p, _i32,
                                                                                        P(ConvPlan)]
        L.conv_tune.restype = ctypes.c_int
        L.conv_plan_tuned.argtypes = [P(ConvDesc), P(ConvTensor), P(ConvPlan)]
        L.conv_plan_tuned.restype = ctypes.c_int
        L.conv_kernel_name.argtypes = [_i32]
        L.conv_kernel_name.restype = ctypes.c_char_p
        L.conv_status_string.argtypes = [_i32]
        L.conv_status_string.restype = ctypes.c_char_p
        L.conv_abi_version.argtypes = []
        L.conv_abi_version.restype = _i32
        _lib = L
    return _lib
