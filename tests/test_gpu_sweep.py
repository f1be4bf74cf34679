"""GPU parity over a seeded sample of shapes, blocks and quantizer specs.

The hand-written parity tests name the shapes each kernel was built for.
This file draws its cases from a fixed-seed generator over the library's
supported space instead: widths that are powers of two and Kronecker widths
(base orders 12, 20, 28, 44, 60, 108, 140), full-width and block-diagonal
rotations, INT groups of 16 to 2048 (sym and asym, bf16 and float32 scales),
MXFP4 and NVFP4, bf16 and float32 inputs, and row counts that leave partial
waves and workgroups.  Each case is kept only if hr_check_shape (host-side
planning) accepts it, and is compared with the oracle through both kernel
families (the default dispatch, and the generic kernel forced).  Sizes stay
small (at most 2^17 elements, widths up to 8192) so that the oracle's dense
products finish quickly.
"""
import random
import sys

import pytest
import torch

import oracle
import synth
import hadamard_rotation_preprocessing_amd as hr
from parity import Report, check_int, check_mxfp4, check_nvfp4, check_rotated, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 160
N_WEIGHT = 48
N_ROTATE = 48


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    hr.lib()


@pytest.fixture(params=["fast", "generic"])
def kernel_path(request):
    hr.set_generic_only(request.param == "generic")
    yield request.param
    hr.set_generic_only(False)


POW2 = [2 ** k for k in range(5, 14)]                      # 32 .. 8192
KRON = [12 * 256, 12 * 512, 20 * 256, 28 * 256, 60 * 128, 60 * 64, 44 * 32, 108 * 64, 140 * 32, 12 * 64,
        20 * 128, 28 * 64]


def _spec(rng, n):
    r = rng.random()
    if r < 0.15 and n % 32 == 0:
        return hr.QSpec.mxfp4()
    if r < 0.3 and n % 16 == 0:
        return hr.QSpec.nvfp4(rng.choice([1.0, 0.5, 3.0]))
    gs = [g for g in (16, 32, 64, 128, 256, 512, 2048) if n % g == 0]
    return hr.QSpec("int", 4, rng.choice(gs), rng.random() < 0.5, rng.choice(["bf16", "bf16", "f32"]))


def _draw_cases():
    rng = random.Random(20260)
    cases = []
    while len(cases) < N_CASES:
        n = rng.choice(POW2 + KRON)
        blocks = [0] + [b for b in (16, 32, 64, 128, 256, 512, 1024, 2048, 4096) if b < n and n % b == 0]
        block = rng.choice(blocks)
        dtype = torch.float32 if rng.random() < 0.2 else torch.bfloat16
        spec = _spec(rng, n)
        rows = rng.randint(1, max(1, min(37, (1 << 17) // n)))
        y_rot = rng.random() < 0.5
        try:
            hr.check_shape(dtype, rows, n, block, [spec])
        except hr.HadarotError:
            continue
        cases.append((len(cases), rows, n, block, dtype, spec, y_rot))
    return cases


CASES = _draw_cases()


def _draw_weight_cases():
    """rotate_fuse_weight: one or two specs from one read, with or without W.R."""
    rng = random.Random(20261)
    cases = []
    while len(cases) < N_WEIGHT:
        n = rng.choice(POW2 + KRON)
        blocks = [0] + [b for b in (16, 32, 64, 128, 256, 512, 1024, 2048, 4096) if b < n and n % b == 0]
        block = rng.choice(blocks)
        dtype = torch.float32 if rng.random() < 0.2 else torch.bfloat16
        specs = [_spec(rng, n) for _ in range(rng.choice([1, 2]))]
        rows = rng.randint(1, max(1, min(41, (1 << 17) // n)))
        w_rot = rng.random() < 0.6
        try:
            hr.check_shape(dtype, rows, n, block, specs)
        except hr.HadarotError:
            continue
        cases.append((len(cases), rows, n, block, dtype, specs, w_rot))
    return cases


def _draw_rotate_cases():
    """hadamard_rotate alone, including widths up to 8192 and float32."""
    rng = random.Random(20262)
    cases = []
    while len(cases) < N_ROTATE:
        n = rng.choice(POW2 + KRON + [2, 4, 8, 16])
        blocks = [0] + [b for b in (2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096) if b < n and n % b == 0]
        block = rng.choice(blocks)
        dtype = torch.float32 if rng.random() < 0.4 else torch.bfloat16
        rows = rng.randint(1, max(1, min(61, (1 << 17) // n)))
        try:
            hr.check_shape(dtype, rows, n, block, [])
        except hr.HadarotError:
            continue
        cases.append((len(cases), rows, n, block, dtype))
    return cases


WEIGHT_CASES = _draw_weight_cases()
ROTATE_CASES = _draw_rotate_cases()


def _check_quant(out, y, spec, kk, rep):
    if spec.format == "mxfp4":
        check_mxfp4(out, y, rep, kron_k=kk)
    elif spec.format == "nvfp4":
        check_nvfp4(out, y, rep, spec.tensor_scale, kron_k=kk)
    else:
        check_int(out, y, spec.group_size, spec.sym, spec.scale_dtype, rep, kron_k=kk)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "c%02d-%dx%d-b%d-%s-%s%s" % (
    c[0], c[1], c[2], c[3], "f32" if c[4] == torch.float32 else "bf16", c[5].format,
    ("-g%d%s" % (c[5].group_size, "s" if c[5].sym else "a")) if c[5].format == "int" else ""))
def test_sampled_case(kernel_path, case):
    idx, rows, n, block, dtype, spec, y_rot = case
    x = synth.gaussian((rows, n), seed=9000 + idx, dtype=dtype)
    if rows > 2:
        x[1] = 0.0                      # an all-zero row
        x[rows - 1] *= 1e3              # a row of large values
    say("sampled case", idx, rows, n, block, dtype, spec, "y_rot" if y_rot else "")
    out = hr.rotate_quantize_act(x.to(DEV), block, spec, y_rot=y_rot)
    torch.cuda.synchronize()
    y = oracle.rotate(x, n, block).reshape(-1, n)
    kk = oracle.kron_factor(n)[0] if (block <= 0 and n & (n - 1)) else 0
    rep = Report()
    if y_rot:
        check_rotated(to_np64(out["y_rot"]).reshape(-1, n), y, "f32" if dtype == torch.float32 else "bf16", rep)
    _check_quant(out, y, spec, kk, rep)
    say("  ", rep)


def _spec_id(q):
    return q.format + (("-g%d%s" % (q.group_size, "s" if q.sym else "a")) if q.format == "int" else "")


@pytest.mark.parametrize("case", WEIGHT_CASES, ids=lambda c: "w%02d-%dx%d-b%d-%s-%s%s" % (
    c[0], c[1], c[2], c[3], "f32" if c[4] == torch.float32 else "bf16", "+".join(_spec_id(q) for q in c[5]),
    "-wrot" if c[6] else ""))
def test_sampled_weight_case(kernel_path, case):
    idx, rows, n, block, dtype, specs, w_rot = case
    w = synth.gaussian((rows, n), seed=9500 + idx, dtype=dtype) * 0.02
    if rows > 3:
        w[2, : n // 3] *= 20.0          # outliers
    say("sampled weight case", idx, rows, n, block, dtype, specs, "w_rot" if w_rot else "")
    out = hr.rotate_fuse_weight(w.to(DEV), block, specs, w_rot=w_rot)
    torch.cuda.synchronize()
    y = oracle.rotate(w, n, block).reshape(-1, n)
    kk = oracle.kron_factor(n)[0] if (block <= 0 and n & (n - 1)) else 0
    rep = Report()
    if w_rot:
        check_rotated(to_np64(out["w_rot"]).reshape(-1, n), y, "f32" if dtype == torch.float32 else "bf16", rep)
    for q, o in zip(specs, out["quant"]):
        _check_quant(o, y, q, kk, rep)
    say("  ", rep)


@pytest.mark.parametrize("case", ROTATE_CASES, ids=lambda c: "r%02d-%dx%d-b%d-%s" % (
    c[0], c[1], c[2], c[3], "f32" if c[4] == torch.float32 else "bf16"))
def test_sampled_rotate_case(kernel_path, case):
    idx, rows, n, block, dtype = case
    x = synth.gaussian((rows, n), seed=9800 + idx, dtype=dtype)
    say("sampled rotate case", idx, rows, n, block, dtype)
    y_gpu = hr.rotate(x.to(DEV), block)
    torch.cuda.synchronize()
    check_rotated(to_np64(y_gpu).reshape(-1, n), oracle.rotate(x, n, block).reshape(-1, n),
                  "f32" if dtype == torch.float32 else "bf16")
