"""ctypes declarations of the C ABI in include/hadarot.h.

Loads the in-tree ``lib/libhadarot.so``; raises if it has not been built.
There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# HADAROT_LIBRARY selects another build of the same ABI (the host-only
# sanitizer build of the validation layer used by the CPU tests)
LIB_PATH = os.environ.get("HADAROT_LIBRARY") or os.path.join(_PKG, "lib", "libhadarot.so")

HR_OK, HR_EINVAL, HR_EUNSUPPORTED, HR_EDEVICE = 0, -1, -2, -3
HR_F32, HR_BF16, HR_E8M0, HR_E4M3 = 0, 1, 2, 3
HR_Q_INT, HR_Q_MXFP4, HR_Q_NVFP4 = 0, 1, 2

# every exported symbol declared in include/hadarot.h
EXPORTS = ("hadamard_rotate", "rotate_quantize_act", "rotate_fuse_weight",
           "dequant_check", "hr_last_error", "hr_kron_order",
           "hadamard_rotate_mixed", "rotate_quantize_act_mixed", "rotate_fuse_weight_mixed",
           "rotate_fuse_weight_out", "hr_check_shape", "hr_set_generic_only", "dequant_check_noalloc")
HR_DQ_WORK_BYTES = 65536


class hr_qspec(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("sym", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32), ("tensor_scale", ctypes.c_float)]


class hr_qout(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p)]


class hr_mix(ctypes.Structure):
    _fields_ = [("perm", ctypes.c_void_p), ("in_signs", ctypes.c_void_p),
                ("out_signs", ctypes.c_void_p)]


class hr_dq_stats(ctypes.Structure):
    _fields_ = [("max_err_steps", ctypes.c_double), ("n_over_half_step", ctypes.c_int64),
                ("n_clamped", ctypes.c_int64), ("rel_l2_err", ctypes.c_double)]


class HadarotError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("hadarot status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "HIP library not built: %s is missing (run __graft_entry__.build() or "
                "python -m hadamard_rotation_preprocessing_amd.build)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        L.hadamard_rotate.argtypes = [vp, vp, ci, i64, i64, i64, vp]
        L.hadamard_rotate.restype = ci
        L.rotate_quantize_act.argtypes = [vp, ci, i64, i64, i64, ctypes.POINTER(hr_qspec),
                                          vp, vp, vp, vp, vp]
        L.rotate_quantize_act.restype = ci
        L.rotate_fuse_weight.argtypes = [vp, ci, i64, i64, i64, vp, ctypes.POINTER(hr_qspec), ci,
                                         ctypes.POINTER(hr_qout), vp]
        L.rotate_fuse_weight.restype = ci
        L.dequant_check.argtypes = [vp, vp, vp, ctypes.POINTER(hr_qspec), i64, i64, vp, ci, vp,
                                    ctypes.POINTER(hr_dq_stats), vp, vp]
        L.dequant_check.restype = ci
        L.dequant_check_noalloc.argtypes = [vp, vp, vp, ctypes.POINTER(hr_qspec), i64, i64, vp, ci, vp,
                                            ctypes.POINTER(hr_dq_stats), vp]
        L.dequant_check_noalloc.restype = ci
        L.hr_last_error.argtypes = []
        L.hr_last_error.restype = ctypes.c_char_p
        L.hr_kron_order.argtypes = [i64, ctypes.POINTER(i32), ctypes.POINTER(i64), vp]
        L.hr_kron_order.restype = ci
        mp = ctypes.POINTER(hr_mix)
        L.hadamard_rotate_mixed.argtypes = [vp, vp, ci, i64, i64, i64, mp, vp]
        L.hadamard_rotate_mixed.restype = ci
        L.rotate_quantize_act_mixed.argtypes = [vp, ci, i64, i64, i64, ctypes.POINTER(hr_qspec),
                                                vp, vp, vp, vp, mp, vp]
        L.rotate_quantize_act_mixed.restype = ci
        L.rotate_fuse_weight_mixed.argtypes = [vp, ci, i64, i64, i64, vp, ctypes.POINTER(hr_qspec), ci,
                                               ctypes.POINTER(hr_qout), mp, vp]
        L.rotate_fuse_weight_mixed.restype = ci
        L.rotate_fuse_weight_out.argtypes = [vp, ci, i64, i64, i64, vp, vp]
        L.rotate_fuse_weight_out.restype = ci
        L.hr_check_shape.argtypes = [ci, i64, i64, i64, ctypes.POINTER(hr_qspec), ci]
        L.hr_check_shape.restype = ci
        L.hr_set_generic_only.argtypes = [ci]
        L.hr_set_generic_only.restype = None
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != HR_OK:
        raise HadarotError(status, lib().hr_last_error().decode())
