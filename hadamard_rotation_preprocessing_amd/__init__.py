"""hadarot: Hadamard rotation fused with group quantization on MI355X (gfx950).

Thin Python binding over the C ABI of ``include/hadarot.h``.  It marshals
torch tensors (device pointers, sizes, the current HIP stream) and allocates
outputs with torch; every step of the computation runs in the HIP kernels of
``lib/libhadarot.so``.  There is no CPU or PyTorch fallback: if the library
is missing, the calls raise.

Entry points (same names as the C ABI):
    rotate(x, block=0, out=None)                       -> hadamard_rotate
    rotate_quantize_act(x, block, qspec, y_rot=False)  -> rotate_quantize_act
    rotate_fuse_weight(w, block, qspecs, w_rot=True)   -> rotate_fuse_weight
    dequant_check(q, qspec, ref=None, ...)             -> dequant_check
    dequant_check_noalloc(q, qspec, ref=None, ...)     -> dequant_check_noalloc
    rotate_fuse_weight_out(w, block=0, out=None)       -> rotate_fuse_weight_out
With ``mix=dict(perm=..., in_signs=..., out_signs=...)`` (device tensors,
int32 / int8 / int8, any subset) the first three call the ``*_mixed`` entry
points (randomised rotations, hr_mix in the header).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L
from ._lib import HadarotError, check, lib  # noqa: F401

__all__ = ["QSpec", "rotate", "rotate_quantize_act", "rotate_fuse_weight", "rotate_fuse_weight_out", "dequant_check",
           "dequant_check_noalloc",
           "hadamard_rotate", "kron_order", "check_shape", "set_generic_only", "HadarotError", "alloc_quant_outputs"]

_SCALE_CODES = {"f32": L.HR_F32, "bf16": L.HR_BF16, "e8m0": L.HR_E8M0, "e4m3": L.HR_E4M3}
_SCALE_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "e8m0": torch.uint8, "e4m3": torch.uint8}


@dataclass(frozen=True)
class QSpec:
    """Quantizer spec: the pages' (wbits, groupsize, sym) plus format and
    scale storage dtype ("f32" | "bf16" for INT, "e8m0" for MXFP4, "e4m3"
    for NVFP4, whose tensor_scale g multiplies every block scale)."""
    format: str = "int"
    bits: int = 4
    group_size: int = 128
    sym: bool = True
    scale_dtype: str = "bf16"
    tensor_scale: float = 1.0

    @staticmethod
    def mxfp4() -> "QSpec":
        return QSpec("mxfp4", 4, 32, True, "e8m0")

    @staticmethod
    def nvfp4(tensor_scale: float = 1.0) -> "QSpec":
        return QSpec("nvfp4", 4, 16, True, "e4m3", tensor_scale)

    @staticmethod
    def from_dict(d: dict) -> "QSpec":
        return QSpec(d["format"], int(d["bits"]), int(d["group_size"]), bool(d["sym"]), d["scale_dtype"],
                     float(d.get("tensor_scale", 1.0)))

    def c(self) -> L.hr_qspec:
        fmt = {"int": L.HR_Q_INT, "mxfp4": L.HR_Q_MXFP4, "nvfp4": L.HR_Q_NVFP4}[self.format]
        return L.hr_qspec(fmt, self.bits, self.group_size, 1 if self.sym else 0,
                          _SCALE_CODES[self.scale_dtype], self.tensor_scale)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return L.HR_F32
    if t.dtype == torch.bfloat16:
        return L.HR_BF16
    raise ValueError("dtype must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows_n(x: torch.Tensor):
    if x.dim() < 1:
        raise ValueError("tensor must have at least one dimension")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    n = x.shape[-1]
    return (x.numel() // n if n else 0), n


def alloc_quant_outputs(rows: int, n: int, spec: QSpec, device) -> dict:
    """Allocate codes [rows, n/2] uint8, scales [rows, n/g], zeros (asym INT)."""
    g = spec.group_size
    groups = rows * n // g if g > 0 and n % g == 0 else 0
    out = {
        "codes": torch.empty((rows, n // 2), dtype=torch.uint8, device=device),
        "scales": torch.empty((rows, n // g if g > 0 else 0), dtype=_SCALE_TORCH[spec.scale_dtype],
                              device=device),
        "zeros": None,
    }
    if spec.format == "int" and not spec.sym:
        out["zeros"] = torch.empty(((groups + 1) // 2,), dtype=torch.uint8, device=device)
    return out


def _mix(mix: dict | None, n: int):
    """hr_mix from dict(perm=int32, in_signs=int8, out_signs=int8) of n
    contiguous device entries each (any subset), or None."""
    if mix is None:
        return None
    want = {"perm": torch.int32, "in_signs": torch.int8, "out_signs": torch.int8}
    for k, t in mix.items():
        if k not in want:
            raise ValueError("unknown mix entry %r" % k)
        if t is not None and (t.dtype != want[k] or t.numel() != n or not t.is_contiguous()):
            raise ValueError("mix[%r] must be a contiguous %s tensor of n = %d entries" % (k, want[k], n))
    m = L.hr_mix(*[(mix[k].data_ptr() if mix.get(k) is not None else None) for k in want])
    return ctypes.byref(m), m


def rotate(x: torch.Tensor, block: int = 0, out: torch.Tensor | None = None,
           mix: dict | None = None) -> torch.Tensor:
    """y = x . R on the last dimension (block <= 0: full width)."""
    rows, n = _rows_n(x)
    y = torch.empty_like(x) if out is None else out
    m = _mix(mix, n)
    if m is None:
        check(lib().hadamard_rotate(_ptr(x), _ptr(y), _dt(x), rows, n, block, _stream(x)))
    else:
        check(lib().hadamard_rotate_mixed(_ptr(x), _ptr(y), _dt(x), rows, n, block, m[0], _stream(x)))
    return y


hadamard_rotate = rotate


def rotate_quantize_act(x: torch.Tensor, block: int, qspec: QSpec, y_rot: bool = False,
                        out: dict | None = None, mix: dict | None = None) -> dict:
    """Rotate and quantize activations; returns dict(codes, scales, zeros, y_rot)."""
    rows, n = _rows_n(x)
    o = out if out is not None else alloc_quant_outputs(rows, n, qspec, x.device)
    if y_rot and o.get("y_rot") is None:
        o["y_rot"] = torch.empty_like(x)
    yr = o.get("y_rot") if y_rot else None
    spec = qspec.c()
    args = (_ptr(x), _dt(x), rows, n, block, ctypes.byref(spec), _ptr(o["codes"]), _ptr(o["scales"]),
            _ptr(o["zeros"]), _ptr(yr))
    m = _mix(mix, n)
    if m is None:
        check(lib().rotate_quantize_act(*args, _stream(x)))
    else:
        check(lib().rotate_quantize_act_mixed(*args, m[0], _stream(x)))
    o["y_rot"] = yr
    return o


def rotate_fuse_weight(w: torch.Tensor, block: int, qspecs, w_rot: bool = True,
                       out: dict | None = None, mix: dict | None = None) -> dict:
    """W' = W . R on in_features plus up to two quantized forms of W' from one
    read; returns dict(w_rot, quant=[dict(codes, scales, zeros), ...])."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [out_features, in_features]")
    rows, n = _rows_n(w)
    qspecs = list(qspecs)
    if out is None:
        out = {"w_rot": torch.empty_like(w) if w_rot else None,
               "quant": [alloc_quant_outputs(rows, n, q, w.device) for q in qspecs]}
    specs = (L.hr_qspec * max(1, len(qspecs)))(*[q.c() for q in qspecs])
    outs = (L.hr_qout * max(1, len(qspecs)))(
        *[L.hr_qout(o["codes"].data_ptr(), o["scales"].data_ptr(),
                    o["zeros"].data_ptr() if o["zeros"] is not None else None)
          for o in out["quant"]])
    args = (_ptr(w), _dt(w), rows, n, block, _ptr(out["w_rot"]), specs, len(qspecs), outs)
    m = _mix(mix, n)
    if m is None:
        check(lib().rotate_fuse_weight(*args, _stream(w)))
    else:
        check(lib().rotate_fuse_weight_mixed(*args, m[0], _stream(w)))
    return out


def rotate_fuse_weight_out(w: torch.Tensor, block: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """W' = R^T . W along out_features (output-side fusion); returns W'."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D [out_features, in_features]")
    if not w.is_contiguous():
        raise ValueError("tensor must be contiguous")
    y = torch.empty_like(w) if out is None else out
    check(lib().rotate_fuse_weight_out(_ptr(w), _dt(w), w.shape[0], w.shape[1], block, _ptr(y), _stream(w)))
    return y


def dequant_check(q: dict, qspec: QSpec, rows: int, n: int, ref: torch.Tensor | None = None,
                  want_deq: bool = True, want_stats: bool = True, deq: torch.Tensor | None = None,
                  work: torch.Tensor | None = None):
    """Dequantize packed outputs; returns (deq float32 [rows, n] or None,
    stats dict or None).  Stats need ``ref`` and synchronise the stream; their
    workspace (``work``, HR_DQ_WORK_BYTES bytes) is allocated with torch when
    not given."""
    codes = q["codes"]
    dev = codes.device
    if want_deq and deq is None:
        deq = torch.empty((rows, n), dtype=torch.float32, device=dev)
    if not want_deq:
        deq = None
    st = L.hr_dq_stats()
    spec = qspec.c()
    ref_dt = _dt(ref) if ref is not None else L.HR_F32
    if want_stats and work is None:
        work = torch.empty(L.HR_DQ_WORK_BYTES, dtype=torch.uint8, device=dev)
    check(lib().dequant_check(_ptr(codes), _ptr(q["scales"]), _ptr(q.get("zeros")),
                              ctypes.byref(spec), rows, n, _ptr(ref), ref_dt, _ptr(deq),
                              ctypes.byref(st) if want_stats else None, _ptr(work) if want_stats else None,
                              _stream(codes)))
    return deq, (_stats(st) if want_stats else None)


def dequant_check_noalloc(q: dict, qspec: QSpec, rows: int, n: int, ref: torch.Tensor | None = None,
                          deq: torch.Tensor | None = None, want_stats: bool = True):
    """dequant_check with the library's static device scratch instead of a
    workspace: the C call allocates nothing (``deq``, if wanted, is the
    caller's float32 [rows, n] tensor).  Returns (deq, stats or None)."""
    codes = q["codes"]
    st = L.hr_dq_stats()
    spec = qspec.c()
    ref_dt = _dt(ref) if ref is not None else L.HR_F32
    check(lib().dequant_check_noalloc(_ptr(codes), _ptr(q["scales"]), _ptr(q.get("zeros")),
                                      ctypes.byref(spec), rows, n, _ptr(ref), ref_dt, _ptr(deq),
                                      ctypes.byref(st) if want_stats else None, _stream(codes)))
    return deq, (_stats(st) if want_stats else None)


def _stats(st) -> dict:
    return dict(max_err_steps=st.max_err_steps, n_over_half_step=st.n_over_half_step,
                n_clamped=st.n_clamped, rel_l2_err=st.rel_l2_err)


def check_shape(dtype: torch.dtype, rows: int, n: int, block: int, qspecs=()) -> None:
    """Raise HadarotError if the library does not implement this shape and
    quantizer specs (host-only planning: nothing is allocated or launched)."""
    qspecs = list(qspecs)
    dt = {torch.float32: L.HR_F32, torch.bfloat16: L.HR_BF16}[dtype]
    specs = (L.hr_qspec * max(1, len(qspecs)))(*[q.c() for q in qspecs])
    check(lib().hr_check_shape(dt, rows, n, block, specs, len(qspecs)))


def set_generic_only(on: bool) -> None:
    """Route every later call through the generic kernel (testing aid)."""
    lib().hr_set_generic_only(1 if on else 0)


def kron_order(n: int, with_matrix: bool = False):
    """(K, M) the library uses for a full-width rotation of a non-power-of-two
    width n, and optionally its K x K base matrix (int8 +-1)."""
    K = ctypes.c_int32()
    M = ctypes.c_int64()
    buf = None
    if with_matrix:
        K0 = ctypes.c_int32()
        M0 = ctypes.c_int64()
        check(lib().hr_kron_order(n, ctypes.byref(K0), ctypes.byref(M0), None))
        buf = (ctypes.c_int8 * (K0.value * K0.value))()
    check(lib().hr_kron_order(n, ctypes.byref(K), ctypes.byref(M), buf))
    if with_matrix:
        import numpy as np
        h = np.frombuffer(bytes(buf), dtype=np.int8).reshape(K.value, K.value).copy()
        return K.value, M.value, h
    return K.value, M.value
