"""dequant_check_noalloc (statistics partials in the library's static device
scratch, no allocation) against dequant_check (caller-owned workspace), through
the C ABI: identical dequantized values and statistics, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
partials, which the second must not pick up)."""
import ctypes
import sys

import pytest
import torch

import synth
import hadamard_rotation_preprocessing_amd as hr
from hadamard_rotation_preprocessing_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def call(fn, out, spec, rows, n, ref, deq, work=None):
    st = L.hr_dq_stats()
    args = [ctypes.c_void_p(out["codes"].data_ptr()), ctypes.c_void_p(out["scales"].data_ptr()),
            ctypes.c_void_p(out["zeros"].data_ptr()) if out["zeros"] is not None else None,
            ctypes.byref(spec.c()), rows, n, ctypes.c_void_p(ref.data_ptr()), L.HR_BF16,
            ctypes.c_void_p(deq.data_ptr()), ctypes.byref(st)]
    if work is not None:
        args.append(ctypes.c_void_p(work.data_ptr()))
    args.append(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    hr.check(fn(*args))
    return (st.max_err_steps, st.n_over_half_step, st.n_clamped, st.rel_l2_err)


@pytest.mark.parametrize("spec", [hr.QSpec("int", 4, 128, False, "bf16"), hr.QSpec.mxfp4()], ids=["int-asym", "mxfp4"])
def test_noalloc_matches_workspace_entry_point(spec):
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    lib = L.lib()
    work = torch.empty(L.HR_DQ_WORK_BYTES, dtype=torch.uint8, device=DEV)
    # first call: a grid of the full 1024 workgroups; second: 7 workgroups
    for rows, n in ((600, 4096), (3, 2048)):
        say("dequant_check_noalloc vs dequant_check", rows, n, spec)
        x = synth.gaussian((rows, n), seed=77 + rows, dtype=torch.bfloat16).to(DEV)
        out = hr.rotate_quantize_act(x, 0, spec, y_rot=True)
        ref = out["y_rot"]
        d1 = torch.empty((rows, n), dtype=torch.float32, device=DEV)
        d2 = torch.full((rows, n), float("nan"), dtype=torch.float32, device=DEV)
        s1 = call(lib.dequant_check, out, spec, rows, n, ref, d1, work)
        s2 = call(lib.dequant_check_noalloc, out, spec, rows, n, ref, d2)
        torch.cuda.synchronize()
        assert torch.equal(d1, d2)
        assert s1 == s2, (s1, s2)
        assert s1[3] > 0 and s1[0] > 0
