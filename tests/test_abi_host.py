"""CPU tests of the C ABI (no GPU): the library loads, exports every symbol
declared in include/hadarot.h, and rejects every invalid argument with the
documented status before anything touches the device.  Pointers here are
fake, aligned addresses: every case fails validation, so nothing is
dereferenced and no HIP call is made."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from hadamard_rotation_preprocessing_amd import _lib as L
from hadamard_rotation_preprocessing_amd import kron_order

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

P = 0x7F0000000000           # fake 16-byte-aligned device addresses, far apart
A, B, C, D, Z = (ctypes.c_void_p(P + i * (1 << 36)) for i in range(5))
NUL = None


def header_functions():
    text = open(os.path.join(ROOT, "include", "hadarot.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_exports_every_header_symbol():
    lib = L.lib()
    names = header_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def q(fmt=L.HR_Q_INT, bits=4, g=128, sym=1, sd=L.HR_BF16, ts=0.0):
    return ctypes.byref(L.hr_qspec(fmt, bits, g, sym, sd, ts))


def rqa(x=A, dt=L.HR_BF16, rows=16, n=4096, block=0, qs=None, codes=B, scales=C, zeros=NUL, yrot=NUL):
    return L.lib().rotate_quantize_act(x, dt, rows, n, block, qs if qs is not None else q(),
                                       codes, scales, zeros, yrot, None)


def msg():
    return L.lib().hr_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(dt=7), L.HR_EINVAL, "dtype"),
    (dict(rows=-1), L.HR_EINVAL, "rows"),
    (dict(n=0), L.HR_EINVAL, "n = 0"),
    (dict(block=3), L.HR_EINVAL, "power of two"),
    (dict(n=4096, block=8192), L.HR_EINVAL, "does not divide"),
    (dict(qs=q(bits=3)), L.HR_EUNSUPPORTED, "bits"),
    (dict(qs=q(g=0)), L.HR_EINVAL, "group_size"),
    (dict(qs=q(g=7)), L.HR_EINVAL, "even"),
    (dict(n=4096, qs=q(g=96)), L.HR_EINVAL, "divide"),
    (dict(n=96 * 64, block=32, qs=q(g=96)), L.HR_EUNSUPPORTED, "power of two"),
    (dict(qs=q(sym=2)), L.HR_EINVAL, "sym"),
    (dict(qs=q(sd=L.HR_E8M0)), L.HR_EINVAL, "INT scales"),
    (dict(qs=q(fmt=L.HR_Q_MXFP4, g=64, sd=L.HR_E8M0)), L.HR_EINVAL, "32"),
    (dict(qs=q(fmt=L.HR_Q_MXFP4, g=32, sd=L.HR_BF16)), L.HR_EINVAL, "E8M0"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=32, sd=L.HR_E4M3)), L.HR_EINVAL, "16"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E8M0)), L.HR_EINVAL, "E4M3"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E4M3, ts=-1.0)), L.HR_EINVAL, "tensor_scale"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E4M3, ts=float("inf"))), L.HR_EINVAL, "tensor_scale"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E4M3, ts=float("nan"))), L.HR_EINVAL, "tensor_scale"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E4M3, ts=1e-40)), L.HR_EINVAL, "float range"),
    (dict(qs=q(fmt=L.HR_Q_NVFP4, g=16, sd=L.HR_E4M3), zeros=D), L.HR_EINVAL, "NULL"),
    (dict(qs=q(sd=L.HR_E4M3)), L.HR_EINVAL, "INT scales"),
    (dict(qs=q(fmt=5)), L.HR_EINVAL, "format"),
    (dict(x=NUL), L.HR_EINVAL, "x is NULL"),
    (dict(x=ctypes.c_void_p(P + 8)), L.HR_EINVAL, "aligned"),
    (dict(codes=NUL), L.HR_EINVAL, "codes is NULL"),
    (dict(codes=ctypes.c_void_p(P + (1 << 36) + 4)), L.HR_EINVAL, "aligned"),
    (dict(scales=ctypes.c_void_p(P + 2 * (1 << 36) + 1)), L.HR_EINVAL, "aligned"),
    (dict(qs=q(sym=0), zeros=NUL), L.HR_EINVAL, "zeros is NULL"),
    (dict(zeros=D), L.HR_EINVAL, "must be NULL"),
    (dict(codes=ctypes.c_void_p(P + 1024)), L.HR_EINVAL, "overlaps x"),
    (dict(scales=ctypes.c_void_p(P + (1 << 36) + 64)), L.HR_EINVAL, "overlap"),
    (dict(yrot=ctypes.c_void_p(P + 4096)), L.HR_EINVAL, "partially overlaps"),
    (dict(n=4097 * 2, block=0, qs=q(g=2)), L.HR_EUNSUPPORTED, "base Hadamard"),
    (dict(n=65536, block=0), L.HR_EUNSUPPORTED, "exceeds"),
    (dict(n=131072, block=65536), L.HR_EUNSUPPORTED, "exceeds 32768"),
    (dict(n=244 * 64, block=0), L.HR_EUNSUPPORTED, "exceeds 160"),
])
def test_rotate_quantize_act_validation(kw, status, text):
    st = rqa(**kw)
    assert st == status, (st, msg())
    assert text in msg(), msg()


def test_empty_tensor_is_ok_without_device():
    assert rqa(rows=0, x=NUL, codes=NUL, scales=NUL) == L.HR_OK
    assert L.lib().hadamard_rotate(None, None, L.HR_BF16, 0, 128, 0, None) == L.HR_OK
    assert msg() == ""


def test_hadamard_rotate_validation():
    lib = L.lib()
    assert lib.hadamard_rotate(A, ctypes.c_void_p(P + 16), L.HR_F32, 4, 128, 0, None) == L.HR_EINVAL
    assert "partially overlaps" in msg()
    assert lib.hadamard_rotate(A, B, L.HR_F32, 4, 100, 0, None) == L.HR_EUNSUPPORTED   # 100 = 25 * 4: no order
    assert lib.hadamard_rotate(A, B, L.HR_F32, 4, 128, 6, None) == L.HR_EINVAL
    assert lib.hadamard_rotate(NUL, B, L.HR_F32, 4, 128, 0, None) == L.HR_EINVAL


def test_rotate_fuse_weight_validation():
    lib = L.lib()
    specs = (L.hr_qspec * 3)(L.hr_qspec(1, 4, 32, 1, 2), L.hr_qspec(0, 4, 128, 1, 1), L.hr_qspec(0, 4, 128, 1, 1))
    outs = (L.hr_qout * 3)(L.hr_qout(B.value, C.value, None), L.hr_qout(D.value, Z.value, None),
                           L.hr_qout(D.value, Z.value, None))
    assert lib.rotate_fuse_weight(A, L.HR_BF16, 64, 4096, 0, None, specs, 0, outs, None) == L.HR_EINVAL
    assert "nothing to compute" in msg()
    assert lib.rotate_fuse_weight(A, L.HR_BF16, 64, 4096, 0, None, specs, 3, outs, None) == L.HR_EINVAL
    assert lib.rotate_fuse_weight(A, L.HR_BF16, 64, 4096, 0, None, None, 1, outs, None) == L.HR_EINVAL
    # two quantizers writing the same codes buffer
    outs2 = (L.hr_qout * 2)(L.hr_qout(B.value, C.value, None), L.hr_qout(B.value, D.value, None))
    assert lib.rotate_fuse_weight(A, L.HR_BF16, 64, 4096, 0, None, specs, 2, outs2, None) == L.HR_EINVAL
    assert "overlap" in msg()
    # w_rot aliasing w is not allowed for the weight pass
    assert lib.rotate_fuse_weight(A, L.HR_BF16, 64, 4096, 0, A, specs, 1, outs, None) == L.HR_EINVAL


def test_dequant_check_validation():
    lib = L.lib()
    st = L.hr_dq_stats()
    spec = q(sym=1)
    W = ctypes.c_void_p(P + 7 * (1 << 36))
    f = lib.dequant_check
    assert f(B, C, None, spec, 4, 4096, None, L.HR_F32, None, None, None, None) == L.HR_EINVAL
    assert "nothing to compute" in msg()
    assert f(B, C, None, spec, 4, 4096, None, L.HR_F32, None, ctypes.byref(st), W, None) == L.HR_EINVAL
    assert "requires ref" in msg()
    assert f(B, C, None, spec, 4, 4096, A, L.HR_F32, None, ctypes.byref(st), None, None) == L.HR_EINVAL
    assert "requires work" in msg()
    assert f(B, C, None, spec, 4, 4096, A, 9, None, ctypes.byref(st), W, None) == L.HR_EINVAL
    assert f(B, C, None, spec, 4, 4096, A, L.HR_F32, ctypes.c_void_p(P + 64), None, None, None) == L.HR_EINVAL
    assert "deq overlaps" in msg()
    # the workspace is written: it may not overlap an input or deq
    assert f(B, C, None, spec, 4, 4096, A, L.HR_F32, None, ctypes.byref(st), ctypes.c_void_p(P + 4096),
             None) == L.HR_EINVAL
    assert "work overlaps" in msg()
    assert f(B, C, None, spec, 4, 4096, A, L.HR_F32, D, ctypes.byref(st), ctypes.c_void_p(D.value + 256),
             None) == L.HR_EINVAL
    assert "overlap" in msg()
    assert f(B, C, None, spec, 4, 4096, A, L.HR_F32, None, ctypes.byref(st), ctypes.c_void_p(W.value + 8),
             None) == L.HR_EINVAL
    assert "aligned" in msg()
    # empty: stats zeroed without touching the device
    st.n_clamped = 5
    assert f(None, None, None, spec, 0, 4096, A, L.HR_F32, None, ctypes.byref(st), W, None) == L.HR_OK
    assert st.n_clamped == 0


def cs(dt=L.HR_BF16, rows=4, n=4096, block=0, specs=(), nq=None):
    arr = (L.hr_qspec * max(1, len(specs)))(*specs)
    return L.lib().hr_check_shape(dt, rows, n, block, arr, len(specs) if nq is None else nq)


def spec_int(g, sym):
    return L.hr_qspec(L.HR_Q_INT, 4, g, 1 if sym else 0, L.HR_BF16, 0.0)


@pytest.mark.parametrize("n,block,g", [(16384, 0, 16384), (14336, 0, 2048), (12288, 0, 4096), (16384, 0, 8192),
                                       (32768, 16384, 16384), (4096, 0, 4096)])
def test_wide_asymmetric_groups_are_planned(n, block, g):
    """Asymmetric groups so wide that a chunk holds an odd number of them
    (chunks are then paired so that zero-point bytes are whole): planned with
    at most 1024 threads per workgroup."""
    assert cs(n=n, block=block, specs=[spec_int(g, False)]) == L.HR_OK, msg()


def test_check_shape_refusals():
    # a single asymmetric group of 32768: a pair of chunks needs 2048 threads
    assert cs(n=32768, specs=[spec_int(32768, False)]) == L.HR_EUNSUPPORTED
    assert "threads" in msg()
    assert cs(n=32768, specs=[spec_int(32768, True)]) == L.HR_OK
    assert cs(n=128 * 108, specs=[spec_int(128, True)]) == L.HR_OK          # K = 108, q = 107 prime
    assert cs(n=128 * 140, specs=[spec_int(128, False)]) == L.HR_OK         # K = 140, q = 139 prime
    assert cs(n=244 * 64, specs=[spec_int(128, True)]) == L.HR_EUNSUPPORTED
    assert "exceeds 160" in msg()
    assert cs(n=4096, block=3) == L.HR_EINVAL
    assert cs(n=4096, specs=[spec_int(128, True)], nq=3) == L.HR_EINVAL
    assert cs(dt=7) == L.HR_EINVAL
    assert cs(n=4096, specs=[spec_int(128, True), L.hr_qspec(L.HR_Q_MXFP4, 4, 32, 1, L.HR_E8M0, 0.0)]) == L.HR_OK
    assert cs(rows=0, n=4096) == L.HR_OK


@pytest.mark.parametrize("n", [14336, 96, 5120, 12, 20 * 32, 60 * 8, 108 * 128, 140 * 128, 132 * 64])
def test_kron_order_matches_oracle_factorisation(n):
    """The library's base matrix (its own Paley construction in C++) equals the
    oracle's (built independently in Python) and both factorisations agree."""
    k, m, h = kron_order(n, with_matrix=True)
    assert (k, m) == oracle.kron_factor(n)
    assert np.array_equal(h.astype(np.int64), oracle.paley_hadamard(k))


@pytest.mark.parametrize("k", [60, 108, 140])
def test_wide_base_matrices_are_bordered_circulants(k):
    """The wide Kronecker kernel reads its +-1 operands from a table of
    windows over one sequence, which relies on this shape of the library's
    base matrices for prime q = K - 1 (AutoRound "Rotation Transform",
    section 1.5): row 0 all +1, column 0 -1 below it, and the rest a
    function of (r - c) mod q alone."""
    kk, m, h = kron_order(k * 128, with_matrix=True)
    assert (kk, m) == (k, 128)
    h = h.astype(np.int64)
    q = k - 1
    assert np.all(h[0] == 1) and np.all(h[1:, 0] == -1)
    r, c = np.meshgrid(np.arange(1, k), np.arange(1, k), indexing="ij")
    seq = h[1:, 1][np.arange(q)]               # value at (r - c) mod q = d is h[1 + d][1]
    assert np.array_equal(h[1:, 1:], seq[(r - c) % q])


def test_kron_order_errors():
    lib = L.lib()
    K, M = ctypes.c_int32(), ctypes.c_int64()
    assert lib.hr_kron_order(4096, ctypes.byref(K), ctypes.byref(M), None) == L.HR_EINVAL
    assert lib.hr_kron_order(18, ctypes.byref(K), ctypes.byref(M), None) == L.HR_EUNSUPPORTED


def mix(perm=NUL, si=NUL, so=NUL):
    return ctypes.byref(L.hr_mix(perm, si, so))


def test_mixed_validation():
    lib = L.lib()
    E = ctypes.c_void_p(P + 6 * (1 << 36))
    # a permuted rotation cannot run in place
    assert lib.hadamard_rotate_mixed(A, A, L.HR_BF16, 16, 4096, 0, mix(perm=E), None) == L.HR_EINVAL
    assert "in place" in msg()
    # perm must be 4-byte aligned
    assert lib.hadamard_rotate_mixed(A, B, L.HR_BF16, 16, 4096, 0, mix(perm=ctypes.c_void_p(P + 6 * (1 << 36) + 2)),
                                     None) == L.HR_EINVAL
    assert "aligned" in msg()
    # the vectors are inputs: outputs may not overlap them
    assert lib.hadamard_rotate_mixed(A, B, L.HR_BF16, 16, 4096, 0, mix(perm=B), None) == L.HR_EINVAL
    assert "overlaps" in msg()
    assert lib.rotate_quantize_act_mixed(A, L.HR_BF16, 16, 4096, 0, q(), B, C, NUL, A, mix(perm=E),
                                         None) == L.HR_EINVAL
    assert "in place" in msg()
    assert lib.rotate_quantize_act_mixed(A, L.HR_BF16, 16, 4096, 0, q(), B, C, NUL, NUL, mix(so=B),
                                         None) == L.HR_EINVAL
    assert "overlaps" in msg()
    outs = (L.hr_qout * 1)(L.hr_qout(C.value, D.value, None))
    assert lib.rotate_fuse_weight_mixed(A, L.HR_BF16, 16, 4096, 0, B, q(), 1, outs, mix(si=B),
                                        None) == L.HR_EINVAL
    assert "overlaps" in msg()
    # invalid shapes are still reported first
    assert lib.hadamard_rotate_mixed(A, B, L.HR_BF16, 16, 4096, 3, mix(perm=E), None) == L.HR_EINVAL
    assert "power of two" in msg()


def test_weight_out_validation():
    lib = L.lib()
    f = lib.rotate_fuse_weight_out
    assert f(A, L.HR_BF16, 4096, 4096, 3, B, None) == L.HR_EINVAL and "power of two" in msg()
    assert f(A, L.HR_BF16, 4096, 4096, 16, B, None) == L.HR_EUNSUPPORTED and "32..4096" in msg()
    assert f(A, L.HR_BF16, 16384, 4096, 0, B, None) == L.HR_EUNSUPPORTED      # taller than 8192 rows
    assert f(A, L.HR_BF16, 10240, 4096, 0, B, None) == L.HR_EUNSUPPORTED      # 20 x 512 > 8192 rows
    assert f(A, L.HR_BF16, 5120, 4098, 0, B, None) == L.HR_EUNSUPPORTED and "multiple of 4" in msg()
    assert f(A, L.HR_BF16, 96, 4096, 0, B, None) == L.HR_EUNSUPPORTED
    assert f(A, L.HR_BF16, 4096, 4096, 8192, B, None) == L.HR_EINVAL and "divide" in msg()
    assert f(A, L.HR_BF16, 4096, 100, 0, B, None) == L.HR_EUNSUPPORTED and "multiple" in msg()
    assert f(A, L.HR_BF16, 64, 32, 32, B, None) == L.HR_EUNSUPPORTED       # 32 x 32 < one tile of 2048
    assert f(A, 5, 4096, 4096, 0, B, None) == L.HR_EINVAL and "dtype" in msg()
    assert f(A, L.HR_BF16, 4096, 4096, 0, ctypes.c_void_p(A.value + 64), None) == L.HR_EINVAL
    assert "overlaps" in msg()
    assert f(NUL, L.HR_BF16, 4096, 4096, 0, B, None) == L.HR_EINVAL
    assert f(NUL, L.HR_BF16, 0, 4096, 0, NUL, None) == L.HR_OK


def test_planning_sweep():
    """Plan a broad set of shapes, blocks and quantizer specs through
    hr_check_shape (under the sanitizer build this exercises the planner's
    arithmetic everywhere); every status is one of the documented ones and
    every refusal carries a message."""
    widths = [2 ** k for k in range(1, 16)] + [12 * 512, 20 * 256, 28 * 512, 60 * 512, 12 * 1024, 96, 100, 108 * 128]
    specs = [spec_int(g, s) for g in (2, 4, 8, 16, 32, 64, 128, 256, 2048, 32768) for s in (True, False)]
    specs += [L.hr_qspec(L.HR_Q_MXFP4, 4, 32, 1, L.HR_E8M0, 0.0), L.hr_qspec(L.HR_Q_NVFP4, 4, 16, 1, L.HR_E4M3, 0.5)]
    seen = set()
    for n in widths:
        for block in (0, 16, 32, 128, 2048, n):
            for dt in (L.HR_BF16, L.HR_F32):
                st = cs(dt=dt, rows=3, n=n, block=block)
                assert st in (L.HR_OK, L.HR_EINVAL, L.HR_EUNSUPPORTED)
                for sp in specs:
                    st = cs(dt=dt, rows=5, n=n, block=block, specs=[sp])
                    assert st in (L.HR_OK, L.HR_EINVAL, L.HR_EUNSUPPORTED)
                    assert (st == L.HR_OK) == (msg() == ""), (n, block, st, msg())
                    seen.add(st)
                st = cs(dt=dt, rows=7, n=n, block=block, specs=[specs[-2], specs[13]])
                assert st in (L.HR_OK, L.HR_EINVAL, L.HR_EUNSUPPORTED)
    assert seen == {L.HR_OK, L.HR_EINVAL, L.HR_EUNSUPPORTED}
