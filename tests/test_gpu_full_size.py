"""GPU parity at the configs' full sizes, in the launch configuration
bench.py times: the whole tensor is rotated and quantized on the GPU, and a
seeded sample of rows (the first, the last and random ones) is compared with
the oracle row by row, with the same tolerances as the reduced-size tests.
Every output is also checked for properties that hold at any size (scales
positive, E8M0 bytes below 255, E4M3 bytes at most 448, zero points in range)."""
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


def sample_rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, rows - 8), size=k, replace=False)
    return np.unique(np.concatenate([np.arange(8), mid, np.arange(rows - 8, rows)]))


def zeros_of_rows(zeros, idx, gpr):
    """Unpack the uint4 zero points of the groups of the sampled rows."""
    z = zeros.cpu().numpy()
    gi = idx[:, None] * gpr + np.arange(gpr)[None, :]
    b = z[gi >> 1]
    return np.where(gi & 1, b >> 4, b & 15).astype(np.int64)


def check_quant_rows(out, spec, y, idx, n, rep, kron_k=0):
    ti = torch.as_tensor(idx, device=out["codes"].device)
    sub = {"codes": out["codes"][ti], "scales": out["scales"][ti]}
    if spec.format == "mxfp4":
        check_mxfp4(sub, y, rep, kron_k=kron_k)
        e = out["scales"].cpu().numpy()
        assert e.max() < 255
    elif spec.format == "nvfp4":
        check_nvfp4(sub, y, rep, spec.tensor_scale, kron_k=kron_k)
        b = out["scales"].cpu().numpy()
        assert b.max() <= 126                      # 448 at most, never the NaN byte
    else:
        zg = None
        if not spec.sym:
            zg = zeros_of_rows(out["zeros"], idx, n // spec.group_size)
        check_int(dict(sub, zeros=None), y, spec.group_size, spec.sym, spec.scale_dtype, rep, zeros_gpu=zg,
                  kron_k=kron_k)
        s = to_np64(out["scales"])
        assert np.all(s > 0) and np.all(np.isfinite(s))


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
    idx = sample_rows(rows, 48, 1)
    y = oracle.rotate(x[torch.as_tensor(idx)], n, block)
    rep = Report()
    kk = oracle.kron_factor(n)[0] if name == "r4_kron" else 0
    check_quant_rows(out, spec, y, idx, n, rep, kron_k=kk)
    say("  ", rep)


def test_r3_full_size():
    w = synth.WORKLOADS["r3"]
    q, k = synth.make_inputs(w)
    spec = hr.QSpec.from_dict(w.qspecs[0])
    rows = q.numel() // 128
    say("r3 full size", tuple(q.shape))
    yq = hr.rotate(q.to(DEV), 0)
    out = hr.alloc_quant_outputs(rows, 128, spec, DEV)
    hr.rotate_quantize_act(k.to(DEV), 0, spec, out=out)
    torch.cuda.synchronize()
    idx = sample_rows(rows, 512, 2)
    q2, k2 = q.reshape(rows, 128), k.reshape(rows, 128)
    rep = Report()
    ti = torch.as_tensor(idx)
    check_rotated(to_np64(yq.reshape(rows, 128)[ti.to(DEV)]), oracle.rotate(q2[ti], 128), "bf16", rep)
    check_quant_rows(out, spec, oracle.rotate(k2[ti], 128), idx, 128, rep)
    say("  ", rep)


def test_weight_full_size():
    w = synth.WORKLOADS["weight"]
    x = synth.make_inputs(w)
    specs = [hr.QSpec.from_dict(d) for d in w.qspecs]
    rows, n = x.shape
    say("weight full size", rows, n)
    out = hr.rotate_fuse_weight(x.to(DEV), 0, specs)
    torch.cuda.synchronize()
    idx = sample_rows(rows, 48, 3)
    ti = torch.as_tensor(idx)
    y = oracle.rotate(x[ti], n)
    rep = Report()
    check_rotated(to_np64(out["w_rot"][ti.to(DEV)]), y, "bf16", rep)
    for spec, o in zip(specs, out["quant"]):
        check_quant_rows(o, spec, y, idx, n, rep)
    say("  ", rep)


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


@pytest.mark.parametrize("name", ["r1", "r4"])
def test_block32_mxfp4_full_size(name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    spec = hr.QSpec.mxfp4()
    rows, n = x.shape
    out = hr.alloc_quant_outputs(rows, n, spec, DEV)
    hr.rotate_quantize_act(x.to(DEV), 32, spec, out=out)
    torch.cuda.synchronize()
    idx = sample_rows(rows, 48, 4)
    rep = Report()
    check_quant_rows(out, spec, oracle.rotate(x[torch.as_tensor(idx)], n, 32), idx, n, rep)
    say("  ", rep)


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
    idx = sample_rows(rows, 16, 5)
    y = oracle.rotate_mixed(x[torch.as_tensor(idx)], n, block, m.get("perm"), m.get("in_signs"),
                            m.get("out_signs")).reshape(-1, n)
    rep = Report()
    check_quant_rows(out, spec, y, idx, n, rep)
    say("  ", rep)


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
    idx = sample_rows(rows, 48, 6)
    rep = Report()
    check_quant_rows(out, spec, oracle.rotate(x[torch.as_tensor(idx)], n, 16), idx, n, rep)
    say("  ", rep)


def test_down_proj_output_fusion_full_size():
    """rotate_fuse_weight_out on down_proj [4096, 14336] as bench.py times it,
    checked on sampled columns (each a full-length transform)."""
    w = synth.make_inputs(synth.WORKLOADS["weight"], out_features=4096, in_features=14336)
    say("down_proj output fusion full size")
    wr = hr.rotate_fuse_weight_out(w.to(DEV), 0)
    torch.cuda.synchronize()
    cols = sample_rows(14336, 48, 7)
    ref = oracle.rotate_out(w[:, torch.as_tensor(cols)], 4096, 0)
    check_rotated(to_np64(wr[:, torch.as_tensor(cols, device=DEV)]).T.copy(), ref.T.copy(), "bf16")
