"""GPU parity: every C-ABI entry point against the oracle on seeded inputs.

Sizes are chosen so that the oracle finishes in seconds while the launches
still span many workgroups and a ragged tail (a row count that leaves the
last workgroup partly empty).  Tolerances are those of tests/parity.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import hadamard_rotation_preprocessing_amd as hr
from parity import Report, check_int, check_mxfp4, check_nvfp4, check_rotated, to_np64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    hr.lib()


@pytest.fixture(params=["fast", "generic"])
def kernel_path(request):
    """Run a test through the specialised bf16 kernels (default dispatch) and
    again with the generic kernel forced (hr_set_generic_only)."""
    hr.set_generic_only(request.param == "generic")
    yield request.param
    hr.set_generic_only(False)


def dtname(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def run_act(x, n, block, spec, y_rot=False, ref_y=None, out=None):
    """Rotate+quantize x (CPU tensor [..., n]) on the GPU and check it
    (into the caller's output buffers if `out` is given)."""
    say("rotate_quantize_act", tuple(x.shape), x.dtype, "block", block, spec)
    xg = x.to(DEV)
    out = hr.rotate_quantize_act(xg, block, spec, y_rot=y_rot, out=out)
    torch.cuda.synchronize()
    y = oracle.rotate(x, n, block).reshape(-1, n) if ref_y is None else ref_y
    kk = oracle.kron_factor(n)[0] if (block <= 0 and n & (n - 1)) else 0
    rep = Report()
    if y_rot:
        check_rotated(to_np64(out["y_rot"]).reshape(-1, n), y, dtname(x), rep)
    if spec.format == "mxfp4":
        check_mxfp4(out, y, rep, kron_k=kk)
    elif spec.format == "nvfp4":
        check_nvfp4(out, y, rep, spec.tensor_scale, kron_k=kk)
    else:
        check_int(out, y, spec.group_size, spec.sym, spec.scale_dtype, rep, kron_k=kk)
    say("  ", rep)
    return out, rep


# ------------------------------------------------------------ named workloads

def test_tiny_workload():
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w)
    run_act(x, w.n, w.block, hr.QSpec.from_dict(w.qspecs[0]), y_rot=True)


@pytest.mark.parametrize("y_rot", [False, True])
def test_r1_reduced_rows(kernel_path, y_rot):
    w = synth.WORKLOADS["r1"]
    x = synth.make_inputs(w, tokens=67)
    run_act(x, w.n, w.block, hr.QSpec.from_dict(w.qspecs[0]), y_rot=y_rot)


@pytest.mark.parametrize("y_rot", [False, True])
def test_r4_reduced_rows(kernel_path, y_rot):
    w = synth.WORKLOADS["r4"]
    x = synth.make_inputs(w, tokens=37)
    run_act(x, w.n, w.block, hr.QSpec.from_dict(w.qspecs[0]), y_rot=y_rot)


@pytest.mark.parametrize("y_rot", [False, True])
def test_r4_kronecker_reduced_rows(kernel_path, y_rot):
    w = synth.WORKLOADS["r4_kron"]
    x = synth.make_inputs(w, tokens=13)
    run_act(x, w.n, w.block, hr.QSpec.from_dict(w.qspecs[0]), y_rot=y_rot)


@pytest.mark.parametrize("m", [256, 512, 1024])
@pytest.mark.parametrize("k", [12, 20, 28])
@pytest.mark.parametrize("mode", ["rotate", "sym", "asym", "asym+rot", "sym+rot"])
def test_kronecker_pieces(kernel_path, k, m, mode):
    """Widths K x M with K <= 32 and pieces of M = 256, 512, 1024 (the
    compiled Kronecker shapes, e.g. 20 x 256 = 5120, 28 x 512 = 14336,
    12 x 1024 = 12288) in every mode."""
    n = k * m
    x = synth.gaussian((9, n), seed=8000 + k + m, dtype=torch.bfloat16)
    x[2] *= 1e-3
    x[5, :700] = 0.0
    if mode == "rotate":
        say("hadamard_rotate (Kronecker)", 9, n)
        y = hr.rotate(x.to(DEV), 0)
        torch.cuda.synchronize()
        check_rotated(to_np64(y), oracle.rotate(x, n), "bf16")
        return
    sym = mode.startswith("sym")
    run_act(x, n, 0, hr.QSpec("int", 4, 128, sym, "bf16"), y_rot=mode.endswith("+rot"))


@pytest.mark.parametrize("rows", [1, 2, 3, 2501])
@pytest.mark.parametrize("m", [256, 512, 1024])
@pytest.mark.parametrize("mode", ["sym+rot", "asym+rot", "asym"])
def test_kronecker_small_order(kernel_path, rows, m, mode):
    """Base order 12.  Over pieces of 256 the kernel takes two rows per pass:
    one row, a full pair, a pair missing its second row, and enough rows that
    every workgroup handles several pairs and the last pair is again one
    short.  Over 512 and 1024 the row is taken as 24 pieces of half the size
    (H_12 (x) H_2 as the base matrix), on the same row counts."""
    n = 12 * m
    x = synth.gaussian((rows, n), seed=8200 + rows + m, dtype=torch.bfloat16)
    if rows > 2:
        x[rows - 1] *= 1e-3
        x[1, :300] = 0.0
    run_act(x, n, 0, hr.QSpec("int", 4, 128, mode.startswith("sym"), "bf16"), y_rot=mode.endswith("+rot"))


@pytest.mark.parametrize("k", [60, 108, 140])
@pytest.mark.parametrize("mode", ["rotate", "sym", "asym", "asym+rot", "sym+rot"])
def test_kronecker_128_pieces(kernel_path, k, mode):
    """Widths K x 128 with base orders above 32 (the compiled wide Kronecker
    shapes: 108 and 140, whose base matrices come from a prime q, and 60) in
    every mode, on a row count that is not a multiple of the grid."""
    n = k * 128
    x = synth.gaussian((11, n), seed=8100 + k, dtype=torch.bfloat16)
    x[2] *= 1e-3
    x[5, :500] = 0.0
    if mode == "rotate":
        say("hadamard_rotate (Kronecker)", 11, n)
        y = hr.rotate(x.to(DEV), 0)
        torch.cuda.synchronize()
        check_rotated(to_np64(y), oracle.rotate(x, n), "bf16")
        return
    sym = mode.startswith("sym")
    run_act(x, n, 0, hr.QSpec("int", 4, 128, sym, "bf16"), y_rot=mode.endswith("+rot"))


@pytest.mark.parametrize("y_rot", [False, True])
def test_r3_reduced_query_key(kernel_path, y_rot):
    w = synth.WORKLOADS["r3"]
    q, k = synth.make_inputs(w, batch=1, seq=75)
    say("hadamard_rotate Q", tuple(q.shape))
    qg = q.to(DEV)
    yq = hr.rotate(qg, 0)
    torch.cuda.synchronize()
    check_rotated(to_np64(yq).reshape(-1, 128), oracle.rotate(q, 128).reshape(-1, 128), "bf16")
    run_act(k, 128, 0, hr.QSpec.from_dict(w.qspecs[0]), y_rot=y_rot)


def test_weight_reduced_rows(kernel_path):
    w = synth.WORKLOADS["weight"]
    W = synth.make_inputs(w, out_features=300)
    specs = [hr.QSpec.from_dict(d) for d in w.qspecs]
    say("rotate_fuse_weight", tuple(W.shape), specs)
    out = hr.rotate_fuse_weight(W.to(DEV), 0, specs, w_rot=True)
    torch.cuda.synchronize()
    y = oracle.rotate(W, 4096)
    rep = Report()
    check_rotated(to_np64(out["w_rot"]), y, "bf16", rep)
    check_mxfp4(out["quant"][0], y, rep)
    check_int(out["quant"][1], y, 128, True, "bf16", rep)
    say("  ", rep)


# ------------------------------------------------------------------- sweeps

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("logn", list(range(1, 16)))
def test_full_width_pow2_rotate(dtype, logn):
    n = 1 << logn
    rows = max(3, min(515, (1 << 18) // n)) | 1      # odd row count: ragged tail
    x = synth.gaussian((rows, n), seed=1000 + logn, dtype=dtype)
    say("hadamard_rotate", rows, n, dtype)
    y = hr.rotate(x.to(DEV), 0)
    torch.cuda.synchronize()
    check_rotated(to_np64(y), oracle.rotate(x, n), dtname(x))


@pytest.mark.parametrize("block", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_block_diagonal_rotate_quant(block):
    n = 4096
    x = synth.gaussian((33, n), seed=2000 + block, dtype=torch.bfloat16)
    run_act(x, n, block, hr.QSpec("int", 4, 128, False, "bf16"), y_rot=True)


@pytest.mark.parametrize("case", [(32768, 8192, "int-asym"), (32768, 16384, "int-sym"), (16384, 0, "nvfp4"),
                                  (30720, 0, "int-asym"), (30720, 0, "mxfp4")],
                         ids=["b8192", "b16384", "full-16384-nvfp4", "kron60x512", "kron60x512-mxfp4"])
def test_maximum_widths(case):
    """The widest supported rows: n = 32768 with large blocks, NVFP4's widest
    block (1024 groups of 16), and the largest Kronecker width 60 x 512 (the
    generic kernel)."""
    n, block, q = case
    x = synth.gaussian((5, n), seed=5100 + n + block, dtype=torch.bfloat16)
    x[3] *= 1e-3
    spec = {"int-asym": hr.QSpec("int", 4, 128, False, "bf16"), "int-sym": hr.QSpec("int", 4, 64, True, "f32"),
            "nvfp4": hr.QSpec.nvfp4(), "mxfp4": hr.QSpec.mxfp4()}[q]
    run_act(x, n, block, spec, y_rot=True)


@pytest.mark.parametrize("case", [(32768, 0, hr.QSpec.nvfp4(0.5), "bf16"),
                                  (16384, 16384, hr.QSpec("int", 4, 8, True, "bf16"), "bf16"),
                                  (8192, 8192, hr.QSpec("int", 4, 4, False, "f32"), "bf16"),
                                  (32768, 32768, hr.QSpec("int", 4, 2, False, "bf16"), "bf16"),
                                  (4096, 4096, hr.QSpec("int", 4, 2, True, "f32"), "bf16"),
                                  (32768, 0, hr.QSpec("int", 4, 4, False, "f32"), "f32"),
                                  (30720, 0, hr.QSpec.nvfp4(), "bf16"),
                                  (30720, 0, hr.QSpec("int", 4, 8, True, "bf16"), "bf16"),
                                  (30720, 0, hr.QSpec("int", 4, 8, False, "f32"), "f32")],
                         ids=["full-32768-nvfp4", "b16384-int-g8", "b8192-asym-g4", "b32768-asym-g2", "b4096-g2",
                              "f32-full-32768-asym-g4", "kron60x512-nvfp4", "kron60x512-int-g8",
                              "f32-kron60x512-asym-g8"])
def test_more_than_1024_groups_per_block(case):
    """Blocks of more than 1024 groups: each thread of the generic kernel
    quantizes several whole groups (asymmetric zero points written per
    thread), on bfloat16 and float32 inputs and after the Kronecker mix."""
    n, block, spec, dt = case
    x = synth.gaussian((3, n), seed=5200 + n + spec.group_size, dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
    x[1, : n // 3] = 0.0
    run_act(x, n, block, spec, y_rot=True)


@pytest.mark.parametrize("case", [(16384, 0, 16384), (14336, 0, 2048), (12288, 0, 4096), (16384, 0, 8192)],
                         ids=["full-16384-one-group", "kron28x512-g2048", "kron12x1024-g4096", "full-16384-g8192"])
def test_wide_asymmetric_groups(case):
    """Asymmetric groups of 2048..16384 (an odd number of groups per chunk):
    the chunks are taken in pairs so that zero-point bytes are whole, with 32
    elements per thread where a pair would need more than 1024 threads."""
    n, block, g = case
    x = synth.gaussian((5, n), seed=5300 + n + g, dtype=torch.bfloat16)
    x[2] *= 1e-3
    run_act(x, n, block, hr.QSpec("int", 4, g, False, "bf16"), y_rot=True)


def test_weight_fusion_two_group_sizes_wide():
    """Two quantizers on a 32768-wide weight: groups of 128 spread over four
    threads and NVFP4 groups of 16, two per thread, from one read."""
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=6, in_features=32768)
    specs = [hr.QSpec("int", 4, 128, True, "bf16"), hr.QSpec.nvfp4()]
    say("rotate_fuse_weight 32768 wide, INT g128 + NVFP4")
    out = hr.rotate_fuse_weight(w.to(DEV), 0, specs)
    torch.cuda.synchronize()
    y = oracle.rotate(w, 32768)
    rep = Report()
    check_rotated(to_np64(out["w_rot"]), y, "bf16", rep)
    check_int(out["quant"][0], y, 128, True, "bf16", rep)
    check_nvfp4(out["quant"][1], y, rep)


@pytest.mark.parametrize("block", [64, 128, 256, 512, 1024, 2048, 4096, 8192])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("y_rot", [False, True])
def test_specialised_shapes(kernel_path, block, sym, y_rot):
    """Every compiled shape of the specialised kernels (INT g128 bf16 scales),
    on a row count that leaves the last wave partly empty: 13 rows of 3072
    hold 39 blocks of 1024 (the last wave has 3 of its 4) and 9.75 waves of
    blocks of 512, 256 or 64 (the last wave holds 3072 of its 4096
    elements), and 13 rows of 8192 are 13 blocks of 8192 (the last
    workgroup's second wave pair lies past the end)."""
    n = 3072 if block in (64, 256, 512, 1024) else 8192
    x = synth.gaussian((13, n), seed=2500 + block + sym, dtype=torch.bfloat16)
    x[3, :] *= 1e3
    x[4, 100:300] = 0.0
    run_act(x, n, block, hr.QSpec("int", 4, 128, sym, "bf16"), y_rot=y_rot)


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("sym", [True, False])
@pytest.mark.parametrize("block", [2048, 4096])
def test_int_group_sizes_bf16(kernel_path, g, sym, block):
    """INT groups of 32 (two per lane), 64 and 256 on the 2048- and 4096-block
    kernels: 13 rows of 6144 are 39 blocks of 2048 (the last wave holds one of
    its two), and 13 rows of 8192 are 26 blocks of 4096 (the last workgroup
    is half empty).  Rows of zeros and of large values exercise the scale's
    edge cases."""
    n = 6144 if block == 2048 else 8192
    x = synth.gaussian((13, n), seed=2900 + g + block + sym, dtype=torch.bfloat16)
    x[2] = 0.0
    x[5, :1000] *= 1e4
    run_act(x, n, block, hr.QSpec("int", 4, g, sym, "bf16"))


@pytest.mark.parametrize("head_dim", [64, 256])
@pytest.mark.parametrize("sym", [False, True])
def test_r3_other_head_dims(kernel_path, head_dim, sym):
    """R3 per head with one group per head vector for head_dim 64 and 256
    (a block of the head size, quantized as one group), on a head count that
    leaves the last wave partly filled."""
    heads = 4096 // head_dim * 3 + 5
    x = synth.gaussian((heads, head_dim), seed=3400 + head_dim + sym, dtype=torch.bfloat16)
    x[7] = 0.0
    x[9] *= 1e3
    run_act(x, head_dim, 0, hr.QSpec("int", 4, head_dim, sym, "bf16"))


@pytest.mark.parametrize("case", ["mxfp4-4096", "int-g32-asym-2048", "int-g32-sym-4096"])
def test_scale_buffers_at_minimum_alignment(kernel_path, case):
    """Scale and zero-point buffers at the smallest alignment the C ABI
    allows: E8M0 bytes at an odd address, bf16 scales at 2 mod 4 bytes, zero
    points at an odd address.  Kernels that store a lane's scales at once
    must fall back to naturally aligned pieces there."""
    fmt, rest = case.split("-", 1)
    if fmt == "mxfp4":
        spec, block, n = hr.QSpec.mxfp4(), 0, 4096
    else:
        sym = "-sym-" in case
        block = int(rest.rsplit("-", 1)[1])
        spec, n = hr.QSpec("int", 4, 32, sym, "bf16"), (6144 if block == 2048 else 8192)
    rows = 9
    x = synth.gaussian((rows, n), seed=3300 + n + block, dtype=torch.bfloat16)
    x[4] = 0.0
    o = hr.alloc_quant_outputs(rows, n, spec, DEV)
    gpr = n // spec.group_size
    sbuf = torch.full((rows * gpr + 8,), 0, dtype=o["scales"].dtype, device=DEV)
    o["scales"] = sbuf[1: 1 + rows * gpr].view(rows, gpr)
    assert o["scales"].data_ptr() % (2 if o["scales"].element_size() == 1 else 4) != 0
    if o["zeros"] is not None:
        zbuf = torch.zeros(o["zeros"].numel() + 8, dtype=torch.uint8, device=DEV)
        o["zeros"] = zbuf[1: 1 + o["zeros"].numel()]
    run_act(x, n, block, spec, out=o)
    torch.cuda.synchronize()
    # nothing written outside the views
    assert int(sbuf[0].view(torch.uint8 if sbuf.element_size() == 1 else torch.int16).item()) == 0
    assert not sbuf[1 + rows * gpr:].view(torch.uint8).any()
    if o["zeros"] is not None:
        assert int(zbuf[0].item()) == 0 and not zbuf[1 + o["zeros"].numel():].any()


@pytest.mark.parametrize("block", [64, 256, 512])
@pytest.mark.parametrize("shape", [(13, 3072), (3, 1024), (3, 512)], ids=["ragged-waves", "one-wave", "tiny"])
@pytest.mark.parametrize("spec", ["mxfp4", "int-asym", "rotate"])
def test_small_blocks(kernel_path, block, shape, spec):
    """Blocks of 64, 256 and 512, several to a wave: MXFP4, INT asym with
    groups spanning two 64-blocks, and rotation alone, on row counts that
    fill a wave only partly (3072 of its 4096 elements; 1536)."""
    rows, n = shape
    x = synth.gaussian((rows, n), seed=2700 + block + n, dtype=torch.bfloat16)
    x[rows - 1, : min(n, 300)] = 0.0
    if spec == "rotate":
        say("hadamard_rotate", rows, n, "block", block)
        y = hr.rotate(x.to(DEV), block)
        torch.cuda.synchronize()
        check_rotated(to_np64(y), oracle.rotate(x, n, block).reshape(-1, n), "bf16")
        return
    q = hr.QSpec.mxfp4() if spec == "mxfp4" else hr.QSpec("int", 4, 128, False, "bf16")
    run_act(x, n, block, q, y_rot=spec == "int-asym")


@pytest.mark.parametrize("w_rot", [False, True])
@pytest.mark.parametrize("nq", [1, 2])
def test_weight_variants(kernel_path, w_rot, nq):
    w = synth.WORKLOADS["weight"]
    W = synth.make_inputs(w, out_features=77)
    specs = [hr.QSpec.from_dict(d) for d in w.qspecs][:nq]
    say("rotate_fuse_weight", tuple(W.shape), specs, "w_rot", w_rot)
    out = hr.rotate_fuse_weight(W.to(DEV), 0, specs, w_rot=w_rot)
    torch.cuda.synchronize()
    y = oracle.rotate(W, 4096)
    rep = Report()
    if w_rot:
        check_rotated(to_np64(out["w_rot"]), y, "bf16", rep)
    check_mxfp4(out["quant"][0], y, rep)
    if nq == 2:
        check_int(out["quant"][1], y, 128, True, "bf16", rep)
    say("  ", rep)


@pytest.mark.parametrize("w_rot", [False, True])
@pytest.mark.parametrize("rows", [1, 6])
def test_weight_8192_wide(kernel_path, w_rot, rows):
    """The weight pass on in_features 8192 (a pair of waves per row): W.H,
    MXFP4 and int4 sym g128 from one read."""
    w = synth.WORKLOADS["weight"]
    W = synth.make_inputs(w, out_features=rows, in_features=8192)
    specs = [hr.QSpec.from_dict(d) for d in w.qspecs]
    say("rotate_fuse_weight", tuple(W.shape), specs, "w_rot", w_rot)
    out = hr.rotate_fuse_weight(W.to(DEV), 0, specs, w_rot=w_rot)
    torch.cuda.synchronize()
    y = oracle.rotate(W, 8192)
    rep = Report()
    if w_rot:
        check_rotated(to_np64(out["w_rot"]), y, "bf16", rep)
    check_mxfp4(out["quant"][0], y, rep)
    check_int(out["quant"][1], y, 128, True, "bf16", rep)
    say("  ", rep)


@pytest.mark.parametrize("g", [2, 4, 8, 16, 32, 64, 128, 256, 512, 2048, 8192])
@pytest.mark.parametrize("sym", [True, False])
def test_group_sizes(g, sym):
    n = 8192
    x = synth.gaussian((21, n), seed=3000 + g, dtype=torch.float32)
    block = 2048 if g <= 2048 else 0
    if g <= 4:
        block = 1024      # keeps the chunk within 1024 threads
    run_act(x, n, block, hr.QSpec("int", 4, g, sym, "f32"), y_rot=True)


@pytest.mark.parametrize("n", [96, 12 * 256, 20 * 64, 28 * 512, 60 * 64, 44 * 32, 28 * 8, 108 * 128, 140 * 128,
                               108 * 32, 140 * 64])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_kronecker_widths(n, dtype):
    x = synth.gaussian((19, n), seed=4000 + n, dtype=dtype)
    say("hadamard_rotate (Kronecker)", 19, n, dtype)
    y = hr.rotate(x.to(DEV), 0)
    torch.cuda.synchronize()
    check_rotated(to_np64(y), oracle.rotate(x, n), dtname(x))
    run_act(x, n, 0, hr.QSpec("int", 4, 32, True, "bf16"), y_rot=True)


@pytest.mark.parametrize("rows", [1, 7, 31, 32, 33, 1001])
def test_head_dim_rows_ragged_asym(kernel_path, rows):
    # n = 128 with one group per row: zero points pack two rows per byte and an
    # odd total leaves a padded high nibble
    x = synth.gaussian((rows, 128), seed=5000 + rows, dtype=torch.bfloat16)
    out, _ = run_act(x, 128, 0, hr.QSpec("int", 4, 128, False, "bf16"))
    if rows % 2:
        assert int(out["zeros"][-1].item()) >> 4 == 0


@pytest.mark.parametrize("rows", [1, 15, 17, 64, 1001])
def test_head_dim_rows_ragged_sym(kernel_path, rows):
    # n = 128, one symmetric group per row (the R3 key kernel handles 16 rows
    # per wave: partial waves at the end)
    x = synth.gaussian((rows, 128), seed=6000 + rows, dtype=torch.bfloat16)
    run_act(x, 128, 0, hr.QSpec("int", 4, 128, True, "bf16"))


@pytest.mark.parametrize("case", [(64, 14336, 2048), (64, 14336, 0), (4096, 128, 0), (48, 13824, 0),
                                  (96, 4096, 4096)],
                         ids=["r4-block2048", "kron-28x512", "r3-head128", "kron-108x128", "block4096"])
def test_asym_clamp_binds(kernel_path, case):
    # Asymmetric codes are clamp(rne(y / s) + z, 0, 15).  With a bf16 scale a
    # group's extreme values can round one step past 0 or 15, and the kernels
    # skip the clamp for waves where no lane's extremes do.  These inputs hold
    # groups of both kinds; the codes must still match the oracle exactly.
    rows, n, block = case
    x = synth.gaussian((rows, n), seed=7100 + n + block, dtype=torch.bfloat16)
    y = oracle.rotate(x, n, block).reshape(-1, n)
    ref = oracle.rtn_quant(y, 128, 4, False, "bf16")
    pre = ref.pre.reshape(rows, n // 128, 128)
    unclamped = np.rint(pre) + ref.zeros[..., None]
    binds = ((unclamped < 0) | (unclamped > 15)).any(axis=-1)
    say("groups where the clamp binds: %d of %d" % (int(binds.sum()), binds.size))
    assert 0 < binds.sum() < binds.size
    run_act(x, n, block, hr.QSpec("int", 4, 128, False, "bf16"), ref_y=y)


@pytest.mark.parametrize("block", [32, 0])
def test_mxfp4_activations(kernel_path, block):
    # block-32 rotation with MXFP4 activations (the pages' accuracy setting)
    w = synth.WORKLOADS["r1"]
    x = synth.make_inputs(w, tokens=45)
    run_act(x, 4096, block, hr.QSpec.mxfp4(), y_rot=True)


# ------------------------------------------- blocks of 32 (MXFP4 activations)

@pytest.mark.parametrize("shape", [(45, 4096), (5, 14336), (7, 1024), (3, 96)],
                         ids=["r1", "r4", "partial-wave", "not-1024-multiple"])
@pytest.mark.parametrize("y_rot", [False, True])
def test_block32_mxfp4(kernel_path, shape, y_rot):
    """rotation_size 32 (the MX block) fused with MXFP4 on R1/R4-shaped
    inputs; a row count that leaves a partial wave; and a width that is not a
    multiple of 1024 elements (served by the generic kernel)."""
    rows, n = shape
    if n == 4096:
        x = synth.make_inputs(synth.WORKLOADS["r1"], tokens=rows)
    elif n == 14336:
        x = synth.make_inputs(synth.WORKLOADS["r4"], tokens=rows)
    else:
        x = synth.gaussian((rows, n), seed=12000 + n, dtype=torch.bfloat16)
    run_act(x, n, 32, hr.QSpec.mxfp4(), y_rot=y_rot)


def test_block32_degenerate_blocks(kernel_path):
    n = 1024
    x = synth.gaussian((6, n), seed=12, dtype=torch.bfloat16)
    x[0] = 0.0                      # all-zero blocks: E8M0 byte 0, codes 0
    x[1, :32] = 0.0
    x[1, 64:96] *= 1e-30
    x[1, 96:128] *= 1e30
    x[2, 32:64] = 0.0
    x[2, 40] = 3.0                  # one-hot block: a flat rotated block
    out, _ = run_act(x, n, 32, hr.QSpec.mxfp4(), y_rot=True)
    s = out["scales"].cpu().numpy().reshape(6, n // 32)
    assert np.all(s[0] == 0) and s[1, 0] == 0


@pytest.mark.parametrize("rows", [1, 33, 512])
def test_block32_rotate(rows):
    x = synth.gaussian((rows, 2048), seed=13 + rows, dtype=torch.bfloat16)
    y = hr.rotate(x.to(DEV), 32)
    torch.cuda.synchronize()
    check_rotated(to_np64(y), oracle.rotate(x, 2048, 32), "bf16")


# ------------------------------------------- randomised rotations (hr_mix)

def _mix_cpu(n, seed, perm=False, si=False, so=False):
    m = {}
    if perm:
        m["perm"] = synth.permutation(n, seed)
    if si:
        m["in_signs"] = synth.rademacher(n, seed + 1)
    if so:
        m["out_signs"] = synth.rademacher(n, seed + 2)
    return m


def _oracle_mixed(x, n, block, m):
    return oracle.rotate_mixed(x, n, block, m.get("perm"), m.get("in_signs"), m.get("out_signs")).reshape(-1, n)


@pytest.mark.parametrize("case", [
    # (rows, n, block, dtype, perm, in_signs, out_signs, spec)
    (33, 4096, 0, torch.bfloat16, False, False, True, hr.QSpec("int", 4, 128, True, "bf16")),   # random Hadamard
    (17, 4096, 0, torch.float32, False, False, True, hr.QSpec("int", 4, 64, False, "f32")),
    (40, 4096, 256, torch.bfloat16, True, True, False, hr.QSpec("int", 4, 128, False, "bf16")),  # RPBH
    (40, 4096, 32, torch.bfloat16, True, True, False, hr.QSpec.mxfp4()),                         # RPBH + MX
    (25, 2048, 512, torch.bfloat16, True, True, True, hr.QSpec("int", 4, 32, True, "bf16")),
    (19, 96, 0, torch.float32, True, True, True, hr.QSpec("int", 4, 32, True, "f32")),           # Kronecker 12 x 8
    (9, 14336, 2048, torch.bfloat16, True, True, True, hr.QSpec("int", 4, 128, False, "bf16")),   # RPBH, R4 shape
    (12, 4096, 2048, torch.bfloat16, True, False, False, hr.QSpec("int", 4, 128, True, "bf16")),
    (7, 4096, 0, torch.bfloat16, True, True, True, hr.QSpec("int", 4, 128, False, "bf16")),
    (9, 14336, 2048, torch.bfloat16, False, True, True, hr.QSpec("int", 4, 128, False, "bf16")),  # signs, odd blocks
    (6, 4096, 0, torch.bfloat16, False, True, False, hr.QSpec("int", 4, 128, True, "bf16")),
    (40, 4096, 16, torch.bfloat16, True, True, False, hr.QSpec.nvfp4(0.02)),                    # RPBH + NV
    (33, 4096, 0, torch.bfloat16, False, False, True, hr.QSpec.nvfp4()),                        # random H + NV
], ids=["random-full-bf16", "random-full-f32", "rpbh-256", "rpbh-32-mxfp4", "all-512", "all-kron96",
        "rpbh-2048-r4", "perm-2048-sym", "all-4096-asym", "signs-2048-r4", "in-signs-4096",
        "rpbh-16-nvfp4", "random-full-nvfp4"])
def test_mixed_rotate_quantize(case):
    rows, n, block, dt, pm, si, so, spec = case
    x = synth.gaussian((rows, n), seed=14000 + n + block, dtype=dt)
    m = _mix_cpu(n, 77 + block, pm, si, so)
    say("rotate_quantize_act_mixed", rows, n, block, dt, sorted(m), spec)
    out = hr.rotate_quantize_act(x.to(DEV), block, spec, y_rot=True, mix={k: v.to(DEV) for k, v in m.items()})
    torch.cuda.synchronize()
    y = _oracle_mixed(x, n, block, m)
    rep = Report()
    kk = oracle.kron_factor(n)[0] if (block <= 0 and n & (n - 1)) else 0
    check_rotated(to_np64(out["y_rot"]).reshape(-1, n), y, dtname(x), rep)
    if spec.format == "mxfp4":
        check_mxfp4(out, y, rep, kron_k=kk)
    elif spec.format == "nvfp4":
        check_nvfp4(out, y, rep, spec.tensor_scale, kron_k=kk)
    else:
        check_int(out, y, spec.group_size, spec.sym, spec.scale_dtype, rep, kron_k=kk)
    say("  ", rep)


def test_mixed_rotate_only_and_in_place_signs():
    n = 1024
    x = synth.gaussian((65, n), seed=15, dtype=torch.bfloat16)
    m = _mix_cpu(n, 5, True, True, True)
    y = hr.rotate(x.to(DEV), 128, mix={k: v.to(DEV) for k, v in m.items()})
    torch.cuda.synchronize()
    check_rotated(to_np64(y).reshape(-1, n), _oracle_mixed(x, n, 128, m), "bf16")
    # signs alone may run in place
    ms = _mix_cpu(n, 9, False, True, True)
    xg = x.to(DEV)
    hr.rotate(xg, 0, out=xg, mix={k: v.to(DEV) for k, v in ms.items()})
    torch.cuda.synchronize()
    check_rotated(to_np64(xg).reshape(-1, n), _oracle_mixed(x, n, 0, ms), "bf16")


def test_mixed_rotate_4096_and_unaligned_signs():
    """Rotation only through the specialised kernel (4096 blocks), and sign
    vectors that are not 16-byte aligned (served by the generic kernel)."""
    n = 4096
    x = synth.gaussian((21, n), seed=16, dtype=torch.bfloat16)
    m = _mix_cpu(n, 31, True, True, True)
    y = hr.rotate(x.to(DEV), 0, mix={k: v.to(DEV) for k, v in m.items()})
    torch.cuda.synchronize()
    check_rotated(to_np64(y).reshape(-1, n), _oracle_mixed(x, n, 0, m), "bf16")
    big = torch.zeros(n + 16, dtype=torch.int8, device=DEV)
    signs = big[1:n + 1]                      # one byte past an aligned base
    signs.copy_(m["in_signs"].to(DEV))
    spec = hr.QSpec("int", 4, 128, True, "bf16")
    out = hr.rotate_quantize_act(x.to(DEV), 0, spec, mix={"in_signs": signs})
    torch.cuda.synchronize()
    check_int(out, _oracle_mixed(x, n, 0, {"in_signs": m["in_signs"]}), 128, True, "bf16", Report())


def test_mixed_weight_fusion():
    """Offline fusion of a random Hadamard, W . H . diag(+-1) / sqrt(N), with
    MXFP4 and int4 from one read."""
    rows, n = 96, 4096
    x = synth.make_inputs(synth.WORKLOADS["weight"], out_features=rows)
    m = _mix_cpu(n, 21, False, False, True)
    specs = [hr.QSpec.mxfp4(), hr.QSpec("int", 4, 128, True, "bf16")]
    out = hr.rotate_fuse_weight(x.to(DEV), 0, specs, mix={k: v.to(DEV) for k, v in m.items()})
    torch.cuda.synchronize()
    y = _oracle_mixed(x, n, 0, m)
    rep = Report()
    check_rotated(to_np64(out["w_rot"]).reshape(-1, n), y, "bf16", rep)
    check_mxfp4(out["quant"][0], y, rep)
    check_int(out["quant"][1], y, 128, True, "bf16", rep)


# ------------------------------------------------------------------ NVFP4

def _tensor_scale(x, n, block):
    """The two-level choice g = amax(tensor) / (448 * 6), from the oracle's
    rotation, rounded to float32 (what the C ABI carries)."""
    return float(np.float32(np.abs(oracle.rotate(x, n, block)).max() / (448.0 * 6.0)))


@pytest.mark.parametrize("shape", [(67, 4096, 16), (37, 14336, 16), (19, 4096, 0), (23, 2048, 128),
                                   (5, 32, 16), (9, 14336, 0)],
                         ids=["r1-b16", "r4-b16", "r1-full", "b128", "tiny", "r4-kron"])
@pytest.mark.parametrize("scale", ["unit", "two-level"])
def test_nvfp4_activations(kernel_path, shape, scale):
    rows, n, block = shape
    x = synth.gaussian((rows, n), seed=rows * 7 + n + block, dtype=torch.bfloat16)
    x[1] *= 50.0                     # one outlier row
    x[2, :] = 0.0
    ts = 1.0 if scale == "unit" else _tensor_scale(x, n, block)
    run_act(x, n, block, hr.QSpec.nvfp4(ts), y_rot=(scale == "unit"))


@pytest.mark.parametrize("rows", [64, 3])
def test_block16_rotate_and_weight(kernel_path, rows):
    """Rotation only and W . R + NVFP4 with blocks of 16 (the specialised
    path takes whole runs of 512 elements: 64 rows of 4096 do, 3 rows of 80
    do not)."""
    n = 4096 if rows == 64 else 80
    x = synth.gaussian((rows, n), seed=41 + rows, dtype=torch.bfloat16)
    say("hadamard_rotate block 16", rows, n)
    y = hr.rotate(x.to(DEV), 16)
    torch.cuda.synchronize()
    ref = oracle.rotate(x, n, 16)
    check_rotated(to_np64(y), ref, "bf16")
    say("rotate_fuse_weight block 16 NVFP4", rows, n)
    out = hr.rotate_fuse_weight(x.to(DEV), 16, [hr.QSpec.nvfp4(0.5)])
    torch.cuda.synchronize()
    rep = Report()
    check_rotated(to_np64(out["w_rot"]), ref, "bf16", rep)
    check_nvfp4(out["quant"][0], ref, rep, 0.5)


def test_nvfp4_float32_and_extremes():
    n = 1024
    x = synth.gaussian((12, n), seed=31, dtype=torch.float32)
    x[0] = 0.0                       # all-zero blocks: byte 0, codes 0
    x[1] *= 1e-5                     # block scales in the E4M3 subnormal range or 0
    x[2] *= 1e4                      # scales saturate at 448, codes at 6
    x[3, :16] = torch.tensor([6.0, 3.0, 1.75, 0.25] * 4)   # ties on the E2M1 grid
    for ts in (1.0, 0.03125, 3.0):
        run_act(x, n, 16, hr.QSpec.nvfp4(ts), y_rot=True)


def test_nvfp4_weight_fusion_and_dequant():
    """W . R with NVFP4 and int4 from one read; dequant_check of the NVFP4
    codes against the oracle's dequantization."""
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=96, in_features=4096)
    specs = [hr.QSpec.nvfp4(0.01), hr.QSpec("int", 4, 128, True, "bf16")]
    say("rotate_fuse_weight NVFP4 + INT", tuple(w.shape))
    out = hr.rotate_fuse_weight(w.to(DEV), 16, specs)
    torch.cuda.synchronize()
    y = oracle.rotate(w, 4096, 16)
    rep = Report()
    check_rotated(to_np64(out["w_rot"]), y, "bf16", rep)
    q = out["quant"][0]
    check_nvfp4(q, y, rep, 0.01)
    check_int(out["quant"][1], y, 128, True, "bf16", rep)
    deq, st = hr.dequant_check(q, specs[0], 96, 4096, ref=out["w_rot"])
    codes = oracle.unpack_nibbles(q["codes"].cpu().numpy(), 96 * 4096).reshape(96, 4096)
    ref_deq = oracle.dequant_nvfp4(codes, q["scales"].cpu().numpy().astype(np.int64), 16,
                                   float(np.float32(0.01)))
    assert np.allclose(to_np64(deq), ref_deq, rtol=2e-7, atol=0)
    # the E4M3 scale may round amax / 6 down by up to 1/16, so a block's
    # largest element can sit past 6 (clamped); never more than one per block
    assert st["n_clamped"] <= 96 * 4096 // 16 and 0 < st["rel_l2_err"] < 0.2
    say("  ", rep, st)


# ------------------------------------------- output-side weight fusion (R^T W)

@pytest.mark.parametrize("shape", [(4096, 4096, 0), (4096, 14336, 0), (4096, 4096, 128), (2048, 1024, 256),
                                   (64, 64, 32), (1024, 96, 64), (4096, 6184, 0), (2048, 2056, 1024)],
                         ids=["o_proj-R1", "down_proj-R1", "v_proj-R2", "b256", "b32-small", "f32-b64",
                              "tiles-not-8k", "b1024-ragged"])
def test_weight_out_fusion(shape):
    out_f, in_f, block = shape
    dt = torch.float32 if in_f == 96 else torch.bfloat16
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=out_f, in_features=in_f).to(dt)
    say("rotate_fuse_weight_out", out_f, in_f, block, dt)
    wr = hr.rotate_fuse_weight_out(w.to(DEV), block)
    torch.cuda.synchronize()
    cols = np.unique(np.random.default_rng(out_f + in_f).choice(in_f, size=min(in_f, 96), replace=False))
    ref = oracle.rotate_out(w[:, torch.as_tensor(cols)], out_f, block)
    got = to_np64(wr)[:, cols]
    check_rotated(got.T.copy(), ref.T.copy(), dtname(w))


@pytest.mark.parametrize("in_f,dt", [(6144, "bf16"), (8192, "bf16"), (10240, "bf16"), (12352, "bf16"),
                                     (3080, "f32")])
def test_weight_out_tiles_per_workgroup(in_f, dt):
    """4096 rows in tiles of 8 columns on a grid of one workgroup per CU:
    3, 4, 5, and 6 or 7 tiles per workgroup for bf16 (the two tiles before
    the pair loop, whole pairs, an odd last tile), and a float32 weight.
    Every column of a sample of 128 is compared."""
    out_f = 4096
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=out_f, in_features=in_f)
    w = w.float() if dt == "f32" else w
    say("rotate_fuse_weight_out", out_f, in_f, 0, dt)
    wr = hr.rotate_fuse_weight_out(w.to(DEV), 0)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(8), np.arange(in_f - 8, in_f),
                                     np.random.default_rng(in_f).choice(in_f, size=112, replace=False)]))
    ref = oracle.rotate_out(w[:, torch.as_tensor(cols)], out_f, 0)
    got = to_np64(wr)[:, cols]
    check_rotated(got.T.copy(), ref.T.copy(), dt)


@pytest.mark.parametrize("block", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_weight_out_every_block(block):
    """Every block size, with in_features three times the smallest tile width
    (so the smallest tile of that block is taken) and two row blocks (one for
    4096)."""
    out_f = block * (1 if block == 4096 else 2)
    in_f = 3 * max(8, 2048 // block)
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=out_f, in_features=in_f)
    say("rotate_fuse_weight_out", out_f, in_f, block)
    wr = hr.rotate_fuse_weight_out(w.to(DEV), block)
    torch.cuda.synchronize()
    ref = oracle.rotate_out(w, out_f, block)
    check_rotated(to_np64(wr).T.copy(), ref.T.copy(), "bf16")


@pytest.mark.parametrize("out_f,in_f,block,dt", [(8192, 200, 0, "bf16"), (8192, 60, 0, "f32"), (16384, 36, 8192, "bf16"),
                                                 (5120, 104, 0, "bf16"), (5120, 44, 0, "f32"), (1536, 100, 0, "bf16"),
                                                 (2560, 64, 0, "bf16"), (3072, 52, 0, "bf16"), (3584, 68, 0, "bf16"),
                                                 (6144, 36, 0, "bf16"), (7168, 40, 0, "bf16"), (7168, 12, 0, "f32")],
                         ids=lambda v: str(v))
def test_weight_out_tall_and_kronecker(out_f, in_f, block, dt):
    """Output-side fusion over 8192 rows (Sylvester) and over out_features
    that are not a power of two (the Kronecker form K x M: hidden 5120 =
    20 x 256 and others), every column compared; in_features leave a ragged
    number of 4-column tiles."""
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=out_f, in_features=in_f).to(dtype)
    w[:, 3] = 0.0
    say("rotate_fuse_weight_out", out_f, in_f, block, dt)
    wr = hr.rotate_fuse_weight_out(w.to(DEV), block)
    torch.cuda.synchronize()
    ref = oracle.rotate_out(w, out_f, block)
    rep = Report()
    check_rotated(to_np64(wr).T.copy(), ref.T.copy(), dt, rep)
    say("  ", rep)


@pytest.mark.parametrize("in_f,in_place", [(1032, False), (2400, False), (4096, False), (4096, True)])
def test_weight_out_8192_bf16(in_f, in_place):
    """bf16 over 8192 rows on wider weights: 258, 600 and 1024 tiles of 4
    columns (more than one per workgroup of the persistent grid; 258 is not a
    multiple of 8, so no XCD grouping), and in place.  The first 16 and last 8
    columns and a sample of others are compared with the oracle."""
    out_f = 8192
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=out_f, in_features=in_f)
    w[:, 9] = 0.0
    say("rotate_fuse_weight_out", out_f, in_f, 0, "bf16", "in place" if in_place else "")
    wg = w.to(DEV)
    wr = hr.rotate_fuse_weight_out(wg, 0, out=wg if in_place else None)
    torch.cuda.synchronize()
    if in_place:
        assert wr.data_ptr() == wg.data_ptr()
    cols = np.unique(np.concatenate([np.arange(16), np.arange(in_f - 8, in_f),
                                     np.random.default_rng(in_f).choice(in_f, size=48, replace=False)]))
    ref = oracle.rotate_out(w[:, torch.as_tensor(cols)], out_f, 0)
    rep = Report()
    check_rotated(to_np64(wr)[:, cols].T.copy(), ref.T.copy(), "bf16", rep)
    say("  ", rep)


def test_weight_out_in_place_and_layer_equivalence():
    """In place, and the fused weight reproduces the rotated layer output:
    x . W'^T against (x . W^T) . R on the GPU-rounded weight."""
    out_f, in_f = 1024, 512
    w = synth.gaussian((out_f, in_f), seed=17, dtype=torch.float32)
    wg = w.to(DEV)
    hr.rotate_fuse_weight_out(wg, 0, out=wg)
    torch.cuda.synchronize()
    x = np.random.default_rng(5).standard_normal((9, in_f))
    lhs = x @ to_np64(wg).T
    rhs = oracle.rotate(x @ to_np64(w).T, out_f)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-4 * np.abs(rhs).max())
    # W' then quantized along in_features with the identity rotation (block 1)
    spec = hr.QSpec("int", 4, 128, True, "f32")
    o = hr.rotate_fuse_weight(wg, 1, [spec], w_rot=False)["quant"][0]
    torch.cuda.synchronize()
    check_int(o, to_np64(wg), 128, True, "f32", Report())


# ------------------------------------------------------------- special cases

def test_in_place_rotation():
    x = synth.gaussian((65, 2048), seed=6, dtype=torch.bfloat16)
    ref = oracle.rotate(x, 2048, 256)
    xg = x.to(DEV)
    y = hr.rotate(xg, 256, out=xg)
    torch.cuda.synchronize()
    assert y.data_ptr() == xg.data_ptr()
    check_rotated(to_np64(xg), ref, "bf16")


def test_in_place_y_rot():
    x = synth.gaussian((40, 4096), seed=7, dtype=torch.float32)
    xg = x.to(DEV)
    spec = hr.QSpec("int", 4, 64, True, "f32")
    o = hr.alloc_quant_outputs(40, 4096, spec, DEV)
    o["y_rot"] = xg
    hr.rotate_quantize_act(xg, 0, spec, y_rot=True, out=o)
    torch.cuda.synchronize()
    y = oracle.rotate(x, 4096)
    check_rotated(to_np64(xg), y, "f32")
    check_int(o, y, 64, True, "f32", Report())


def test_degenerate_groups_and_magnitudes():
    n = 1024
    x = synth.gaussian((12, n), seed=8, dtype=torch.float32)
    x[0] = 0.0                      # all-zero row: scale 1, codes 0
    x[1] = 3.0                      # constant row: rotation is a single spike
    x[2] *= 1e-20
    x[3] *= 1e20
    x[4] = 0.0
    x[4, 17] = 5.0                  # one-hot
    x[5, :512] = 0.0
    for sym in (True, False):
        for sd in ("f32", "bf16"):
            out, _ = run_act(x, n, 0, hr.QSpec("int", 4, 32, sym, sd), y_rot=True)
            s = to_np64(out["scales"])
            assert np.all(s[0] == 1.0)
    out, _ = run_act(x, n, 0, hr.QSpec.mxfp4())
    assert np.all(out["scales"][0].cpu().numpy() == 0)


def test_empty_tensor():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    y = hr.rotate(x, 0)
    assert y.shape == (0, 256)
    o = hr.rotate_quantize_act(x, 0, hr.QSpec("int", 4, 128, False, "bf16"))
    assert o["codes"].shape == (0, 128)
    o = hr.rotate_quantize_act(x, 16, hr.QSpec.nvfp4(0.5))
    assert o["codes"].shape == (0, 128) and o["scales"].shape == (0, 16)
    w = hr.rotate_fuse_weight_out(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), 0)
    assert w.shape == (0, 64)
    torch.cuda.synchronize()


def test_weight_fusion_nvfp4_and_mxfp4():
    """Both FP4 forms of W . R from one read (the generic kernel takes two
    quantizers of different group sizes)."""
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=40, in_features=2048)
    specs = [hr.QSpec.nvfp4(), hr.QSpec.mxfp4()]
    say("rotate_fuse_weight NVFP4 + MXFP4", tuple(w.shape))
    out = hr.rotate_fuse_weight(w.to(DEV), 32, specs, w_rot=False)
    torch.cuda.synchronize()
    y = oracle.rotate(w, 2048, 32)
    rep = Report()
    check_nvfp4(out["quant"][0], y, rep)
    check_mxfp4(out["quant"][1], y, rep)


def test_errors_leave_outputs_untouched():
    n = 4096
    x = synth.gaussian((8, n), seed=9, dtype=torch.bfloat16).to(DEV)
    spec = hr.QSpec("int", 4, 128, True, "bf16")
    o = hr.alloc_quant_outputs(8, n, spec, DEV)
    o["codes"].fill_(0xA5)
    o["scales"].fill_(-7.0)
    with pytest.raises(hr.HadarotError):
        hr.rotate_quantize_act(x, 3, spec, out=o)           # block 3: not a power of two
    with pytest.raises(hr.HadarotError):
        hr.rotate_quantize_act(x, 0, hr.QSpec("int", 3, 128, True, "bf16"), out=o)
    torch.cuda.synchronize()
    assert bool((o["codes"] == 0xA5).all())
    assert bool((o["scales"] == -7.0).all())


def test_guard_bytes_around_outputs():
    """Outputs carved from larger buffers: the bytes just before and after
    each output keep their sentinel value (no out-of-bounds writes)."""
    rows, n = 37, 2048
    x = synth.gaussian((rows, n), seed=10, dtype=torch.bfloat16).to(DEV)
    spec = hr.QSpec("int", 4, 128, False, "bf16")
    pad = 256
    cbuf = torch.full((rows * n // 2 + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((rows * n // 128 + 2 * pad,), 1234.0, dtype=torch.bfloat16, device=DEV)
    zbuf = torch.full(((rows * n // 128 + 1) // 2 + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV)
    ybuf = torch.full((rows * n + 2 * pad,), 99.0, dtype=torch.bfloat16, device=DEV)
    o = {"codes": cbuf[pad:-pad].view(rows, n // 2), "scales": sbuf[pad:-pad].view(rows, n // 128),
         "zeros": zbuf[pad:-pad], "y_rot": ybuf[pad:-pad].view(rows, n)}
    hr.rotate_quantize_act(x, 512, spec, y_rot=True, out=o)
    torch.cuda.synchronize()
    for buf, val in ((cbuf, 0x5A), (zbuf, 0x5A), (sbuf, 1234.0), (ybuf, 99.0)):
        assert bool((buf[:pad] == val).all()) and bool((buf[-pad:] == val).all())
    y = oracle.rotate(x.cpu(), n, 512)
    check_int(o, y, 128, False, "bf16", Report())


# ------------------------------------------------------------ dequant_check

@pytest.mark.parametrize("spec", [hr.QSpec("int", 4, 128, True, "bf16"), hr.QSpec("int", 4, 64, False, "f32"),
                                  hr.QSpec.mxfp4()], ids=["sym-bf16", "asym-f32", "mxfp4"])
def test_dequant_check(spec):
    rows, n = 50, 4096
    x = synth.gaussian((rows, n), seed=11, dtype=torch.bfloat16)
    out = hr.rotate_quantize_act(x.to(DEV), 0, spec, y_rot=True)
    deq, st = hr.dequant_check(out, spec, rows, n, ref=out["y_rot"])
    torch.cuda.synchronize()
    # the oracle dequantizes the GPU's own codes and scales
    if spec.format == "mxfp4":
        codes = oracle.unpack_nibbles(out["codes"].cpu().numpy().reshape(-1), rows * n).reshape(rows, n)
        ref_deq = oracle.dequant_mxfp4(codes, out["scales"].cpu().numpy().astype(np.int64), 32)
    else:
        codes = oracle.unpack_nibbles(out["codes"].cpu().numpy().reshape(-1), rows * n,
                                      signed=spec.sym).reshape(rows, n)
        zeros = None
        if not spec.sym:
            zeros = oracle.unpack_nibbles(out["zeros"].cpu().numpy(), rows * n // spec.group_size)
            zeros = zeros.reshape(rows, n // spec.group_size)
        ref_deq = oracle.dequant_int(codes, to_np64(out["scales"]), zeros, spec.group_size)
    got = to_np64(deq)
    assert np.allclose(got, ref_deq, rtol=2.0 ** -23, atol=0)
    r = to_np64(out["y_rot"])
    rel = np.linalg.norm(r - ref_deq) / np.linalg.norm(r)
    assert abs(st["rel_l2_err"] - rel) <= 1e-6 + 1e-4 * rel
    assert st["max_err_steps"] >= 0
    if spec.format == "int":
        # nearest rounding of values inside the grid: within half a step, up
        # to the bf16 rounding of the reference (2^-8 relative on values of
        # at most 16 steps)
        assert st["max_err_steps"] < 0.5 + 16 * 2.0 ** -8


@pytest.mark.parametrize("n,block", [(128, 0), (4096, 0), (8192, 2048), (4096, 512)])
def test_bf16_outputs_round_to_nearest_even(kernel_path, n, block):
    """bfloat16 outputs are the round-to-nearest-even of the float32 result:
    nearly all of them equal the oracle's exact value rounded to bfloat16
    (differences only where the float32 result and the exact value straddle
    a rounding midpoint), which truncation or round-half-up would miss on
    about half or a quarter of the elements."""
    x = synth.gaussian((64, n), seed=7000 + n + block, dtype=torch.bfloat16)
    y = hr.rotate(x.to(DEV), block)
    torch.cuda.synchronize()
    ref = oracle.bf16_round(oracle.rotate(x, n, block))
    got = to_np64(y)
    frac = float(np.mean(got == ref))
    say("bf16 outputs equal to RNE(exact):", frac)
    assert frac > 0.999


E2M1_TIES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 0.125, 3.0, 7.0]


@pytest.mark.parametrize("path", ["act", "weight"])
def test_mxfp4_exact_ties(kernel_path, path):
    """Rows with two nonzero inputs x[0] = a, x[1] = b rotate (n = 4096,
    1/sqrt(n) = 2^-6) to the exact values (a + b)/64 at even and (a - b)/64 at
    odd positions, so the quantizer input is known exactly and the codes must
    equal the oracle's bit for bit: every E2M1 rounding tie (ties to the even
    mantissa), saturation above 6 and negative values (sign kept)."""
    n = 4096
    rows = []
    for e in (-3, 0, 4):
        for t in E2M1_TIES:
            for sgn in (1.0, -1.0):
                hi, lo = 6.0 * 2.0 ** e, sgn * t * 2.0 ** e   # amax = 6 2^e -> shared exponent e
                a, b = 32.0 * (hi + lo), 32.0 * (hi - lo)
                r = np.zeros(n)
                r[0], r[1] = a, b
                rows.append(r)
    x64 = np.array(rows)
    x = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float64).numpy(), x64), "inputs must be exact in bf16"
    y = oracle.rotate(x, n)
    assert np.array_equal(y[:, 0], (x64[:, 0] + x64[:, 1]) / 64)
    spec = hr.QSpec.mxfp4()
    if path == "act":
        out = hr.rotate_quantize_act(x.to(DEV), 0, spec)
    else:
        out = hr.rotate_fuse_weight(x.to(DEV), 0, [spec], w_rot=False)["quant"][0]
    torch.cuda.synchronize()
    ref = oracle.mxfp4_quant(y, 32)
    codes = oracle.unpack_nibbles(out["codes"].cpu().numpy().reshape(-1), y.size).reshape(y.shape)
    assert np.array_equal(out["scales"].cpu().numpy().astype(np.int64).reshape(ref.scales.shape), ref.scales)
    assert np.array_equal(codes, ref.codes)


def test_int4_exact_ties(kernel_path):
    """Two-nonzero rows as above with amax = 7 2^m (so s = 2^m exactly) and the
    other value at (k + 1/2) 2^m: every symmetric rounding tie, both signs."""
    n = 4096
    rows = []
    for m in (-5, 0, 3):
        for k in range(-7, 7):
            hi, lo = 7.0 * 2.0 ** m, (k + 0.5) * 2.0 ** m
            r = np.zeros(n)
            r[0], r[1] = 32.0 * (hi + lo), 32.0 * (hi - lo)
            rows.append(r)
    x64 = np.array(rows)
    x = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float64).numpy(), x64)
    y = oracle.rotate(x, n)
    spec = hr.QSpec("int", 4, 128, True, "bf16")
    out = hr.rotate_quantize_act(x.to(DEV), 0, spec)
    torch.cuda.synchronize()
    ref = oracle.rtn_quant(y, 128, 4, True, "bf16")
    codes = oracle.unpack_nibbles(out["codes"].cpu().numpy().reshape(-1), y.size, signed=True).reshape(y.shape)
    assert np.array_equal(to_np64(out["scales"]).reshape(ref.scales.shape), ref.scales)
    assert np.array_equal(codes, ref.codes)


# ------------------------------------------------------------ graph capture

@pytest.mark.parametrize("path", ["kwave-int4", "kkron", "kbsmall-nvfp4", "colrot", "weight-two-specs"])
def test_hip_graph_capture_replays_match_eager(path):
    """The entry points allocate nothing and enqueue only kernels, so they can
    be captured in a HIP graph: three replays, each after the input changed
    in place (eager work between the replays), match eager calls bit for bit."""
    torch.manual_seed(0)
    if path == "kwave-int4":
        x = synth.gaussian((64, 4096), seed=61, dtype=torch.bfloat16).to(DEV)
        spec = hr.QSpec("int", 4, 128, False, "bf16")
        out = hr.alloc_quant_outputs(64, 4096, spec, DEV)
        run = lambda: hr.rotate_quantize_act(x, 0, spec, out=out)
        snap = lambda: [out["codes"].clone(), out["scales"].clone(), out["zeros"].clone()]
    elif path == "kkron":
        x = synth.gaussian((16, 14336), seed=62, dtype=torch.bfloat16).to(DEV)
        spec = hr.QSpec("int", 4, 128, False, "bf16")
        out = hr.alloc_quant_outputs(16, 14336, spec, DEV)
        run = lambda: hr.rotate_quantize_act(x, 0, spec, out=out)
        snap = lambda: [out["codes"].clone(), out["scales"].clone(), out["zeros"].clone()]
    elif path == "kbsmall-nvfp4":
        x = synth.gaussian((64, 4096), seed=63, dtype=torch.bfloat16).to(DEV)
        spec = hr.QSpec.nvfp4(0.25)
        out = hr.alloc_quant_outputs(64, 4096, spec, DEV)
        run = lambda: hr.rotate_quantize_act(x, 16, spec, out=out)
        snap = lambda: [out["codes"].clone(), out["scales"].clone()]
    elif path == "colrot":
        x = synth.gaussian((4096, 256), seed=64, dtype=torch.bfloat16).to(DEV)
        y = torch.empty_like(x)
        run = lambda: hr.rotate_fuse_weight_out(x, 0, out=y)
        snap = lambda: [y.clone()]
    else:
        x = synth.gaussian((48, 4096), seed=65, dtype=torch.bfloat16).to(DEV)
        specs = [hr.QSpec.mxfp4(), hr.QSpec("int", 4, 128, True, "bf16")]
        wo = {"w_rot": torch.empty_like(x), "quant": [hr.alloc_quant_outputs(48, 4096, s, DEV) for s in specs]}
        run = lambda: hr.rotate_fuse_weight(x, 0, specs, out=wo)
        snap = lambda: [wo["w_rot"].clone()] + [t.clone() for q in wo["quant"] for t in (q["codes"], q["scales"])]
    say("graph capture", path)
    run()                                   # first call outside capture (one-time launch setup)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        x.mul_(-1.5 if i % 2 else 0.75)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        run()                               # eager reference on the same input
        torch.cuda.synchronize()
        want = snap()
        for a_, b_ in zip(got, want):
            assert torch.equal(a_, b_), (path, i)
