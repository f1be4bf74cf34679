"""GPU parity at the configs' full sizes, in the launch configuration
bench.py times: the whole tensor is rotated and quantized on the GPU in one
call, and then every row is compared with the oracle, chunk by chunk, with the
same tolerances as the reduced-size tests.  Every output is also checked for
properties that hold at any size (scales positive, E8M0 bytes below 255, E4M3
bytes at most 448, zero points in range).

On the five named workloads (tiny, R1, R4, R3 and the weight pass) no
acceptance may rest on the float32 rotation-error widening of tests/parity.py:
each test asserts that Report.widened is 0 and prints the report line."""
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


def to_host(out: dict) -> dict:
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}


def zeros_of_rows(zeros: np.ndarray, lo: int, hi: int, gpr: int) -> np.ndarray:
    """Unpack the uint4 zero points of the groups of rows [lo, hi)."""
    gi = np.arange(lo * gpr, hi * gpr, dtype=np.int64)
    b = zeros[gi >> 1]
    return np.where(gi & 1, b >> 4, b & 15).astype(np.int64).reshape(hi - lo, gpr)


def check_quant_chunk(out_h: dict, spec, y: np.ndarray, lo: int, hi: int, n: int, rep: Report, kron_k: int = 0):
    """Compare the quantized outputs of rows [lo, hi) (host tensors) with the
    oracle's rotated rows y."""
    sub = {"codes": out_h["codes"][lo:hi], "scales": out_h["scales"][lo:hi]}
    if spec.format == "mxfp4":
        check_mxfp4(sub, y, rep, kron_k=kron_k)
    elif spec.format == "nvfp4":
        check_nvfp4(sub, y, rep, spec.tensor_scale, kron_k=kron_k)
    else:
        zg = None
        if not spec.sym:
            zg = zeros_of_rows(out_h["zeros"].numpy(), lo, hi, n // spec.group_size)
        check_int(dict(sub, zeros=None), y, spec.group_size, spec.sym, spec.scale_dtype, rep, zeros_gpu=zg,
                  kron_k=kron_k)


def range_checks(out_h: dict, spec):
    s = out_h["scales"]
    if spec.format == "mxfp4":
        assert int(s.max()) < 255
    elif spec.format == "nvfp4":
        assert int(s.max()) <= 126                 # 448 at most, never the NaN byte
    else:
        sv = to_np64(s)
        assert np.all(sv > 0) and np.all(np.isfinite(sv))


def chunks(rows: int, size: int):
    for lo in range(0, rows, size):
        yield lo, min(rows, lo + size)


def run_rows(name, x2: torch.Tensor, n: int, block: int, quant, rot_h=None, kron_k=0, chunk=1024, rot=None):
    """Oracle comparison of every row of a full-size call: x2 [rows, n] on
    the host, quant = [(spec, host outputs)], rot_h the rotated output (host)
    or None; rot(x rows) overrides the oracle rotation (randomised rotations)."""
    rows = x2.shape[0]
    rep = Report()
    for lo, hi in chunks(rows, chunk):
        y = oracle.rotate(x2[lo:hi], n, block) if rot is None else rot(x2[lo:hi])
        y = y.reshape(hi - lo, n)
        if rot_h is not None:
            check_rotated(to_np64(rot_h[lo:hi]).reshape(hi - lo, n), y, "bf16", rep)
        for spec, out_h in quant:
            check_quant_chunk(out_h, spec, y, lo, hi, n, rep, kron_k=kron_k)
    for spec, out_h in quant:
        range_checks(out_h, spec)
    say("  %s: every row of %d compared: %s" % (name, rows, rep))
    return rep


@pytest.mark.parametrize("name,block", [("r1", 0), ("r4", 2048), ("r4_kron", 0)])
def test_activation_configs_full_size(name, block):
    w = synth.WORKLOADS["r4" if name == "r4_kron" else name]
    x = synth.make_inputs(w)
    spec = hr.QSpec.from_dict(w.qspecs[0])
    rows, n = x.shape
    say(name, "full size", rows, n, "block", block, spec)
    out = hr.alloc_quant_outputs(rows, n, spec, DEV)
    hr.rotate_quantize_act(x.to(DEV), block, spec, out=out)
    torch.cuda.synchronize()
    kk = oracle.kron_factor(n)[0] if name == "r4_kron" else 0
    rep = run_rows(name, x, n, block, [(spec, to_host(out))], kron_k=kk, chunk=2048)
    if name != "r4_kron":
        assert rep.widened == 0, rep


@pytest.mark.parametrize("part", ["q", "k"])
def test_r3_full_size(part):
    w = synth.WORKLOADS["r3"]
    q, k = synth.make_inputs(w)
    spec = hr.QSpec.from_dict(w.qspecs[0])
    rows = q.numel() // 128
    say("r3 full size", part, tuple(q.shape))
    if part == "q":
        yq = hr.rotate(q.to(DEV), 0).reshape(rows, 128).cpu()
        rep = run_rows("r3_q", q.reshape(rows, 128), 128, 0, [], rot_h=yq, chunk=1 << 17)
    else:
        out = hr.alloc_quant_outputs(rows, 128, spec, DEV)
        hr.rotate_quantize_act(k.to(DEV), 0, spec, out=out)
        torch.cuda.synchronize()
        rep = run_rows("r3_k", k.reshape(rows, 128), 128, 0, [(spec, to_host(out))], chunk=1 << 17)
    assert rep.widened == 0, rep


def test_weight_full_size():
    w = synth.WORKLOADS["weight"]
    x = synth.make_inputs(w)
    specs = [hr.QSpec.from_dict(d) for d in w.qspecs]
    rows, n = x.shape
    say("weight full size", rows, n)
    out = hr.rotate_fuse_weight(x.to(DEV), 0, specs)
    torch.cuda.synchronize()
    rep = run_rows("weight", x, n, 0, [(s, to_host(o)) for s, o in zip(specs, out["quant"])],
                   rot_h=out["w_rot"].cpu(), chunk=2048)
    assert rep.widened == 0, rep


def test_tiny_full_size():
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w)
    spec = hr.QSpec.from_dict(w.qspecs[0])
    out = hr.rotate_quantize_act(x.to(DEV), 0, spec, y_rot=True)
    torch.cuda.synchronize()
    y = oracle.rotate(x, 128)
    rep = Report()
    check_rotated(to_np64(out["y_rot"]), y, "f32", rep)
    check_int(out, y, 32, True, "f32", rep)
    say("  tiny: every row of %d compared: %s" % (x.shape[0], rep))
    assert rep.widened == 0, rep


@pytest.mark.parametrize("name", ["r1", "r4"])
def test_block32_mxfp4_full_size(name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    spec = hr.QSpec.mxfp4()
    rows, n = x.shape
    out = hr.alloc_quant_outputs(rows, n, spec, DEV)
    hr.rotate_quantize_act(x.to(DEV), 32, spec, out=out)
    torch.cuda.synchronize()
    run_rows(name + " block 32 MXFP4", x, n, 32, [(spec, to_host(out))], chunk=2048)


@pytest.mark.parametrize("name,block,pm,si,so", [("r1", 0, False, False, True), ("r4", 2048, True, True, False)],
                         ids=["r1-random-hadamard", "r4-rpbh"])
def test_randomised_full_size(name, block, pm, si, so):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    spec = hr.QSpec.from_dict(w.qspecs[0])
    rows, n = x.shape
    m = {}
    if pm:
        m["perm"] = synth.permutation(n, 101)
    if si:
        m["in_signs"] = synth.rademacher(n, 102)
    if so:
        m["out_signs"] = synth.rademacher(n, 103)
    out = hr.alloc_quant_outputs(rows, n, spec, DEV)
    hr.rotate_quantize_act(x.to(DEV), block, spec, out=out, mix={k: v.to(DEV) for k, v in m.items()})
    torch.cuda.synchronize()

    def rot(xs):
        return oracle.rotate_mixed(xs, n, block, m.get("perm"), m.get("in_signs"), m.get("out_signs"))

    run_rows(name + " randomised", x, n, block, [(spec, to_host(out))], chunk=2048, rot=rot)


@pytest.mark.parametrize("name", ["r1", "r4"])
def test_block16_nvfp4_full_size(name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    spec = hr.QSpec.nvfp4()
    rows, n = x.shape
    say(name, "full size, block 16, NVFP4", rows, n)
    out = hr.alloc_quant_outputs(rows, n, spec, DEV)
    hr.rotate_quantize_act(x.to(DEV), 16, spec, out=out)
    torch.cuda.synchronize()
    run_rows(name + " block 16 NVFP4", x, n, 16, [(spec, to_host(out))], chunk=2048)


def test_down_proj_output_fusion_full_size():
    """rotate_fuse_weight_out on down_proj [4096, 14336] as bench.py times it,
    every column (each a full-length transform) compared."""
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=4096, in_features=14336)
    say("down_proj output fusion full size")
    wr = hr.rotate_fuse_weight_out(w.to(DEV), 0).cpu()
    rep = Report()
    for lo, hi in chunks(14336, 2048):
        ref = oracle.rotate_out(w[:, lo:hi], 4096, 0)
        check_rotated(to_np64(wr[:, lo:hi]).T.copy(), ref.T.copy(), "bf16", rep)
    say("  down_out: every column compared: %s" % rep)
