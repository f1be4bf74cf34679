#!/usr/bin/env python3
"""Throughput of the fused Hadamard rotate + quantize path on one MI355X.

One step is one pass over every stage of the hot path, each on its own
seeded synthetic input already resident in HBM:

  r1       R1 residual stream: 4096 x 4096 bf16, full FWHT 4096, int4 sym g128
  r4       R4 down_proj input: 8192 x 14336 bf16, block-diagonal 7 x 2048,
           int4 asym g128 + uint4 zeros
  r4_kron  the same input at full width 14336 = 28 x 512 (Kronecker)
  r3_q     R3 queries 16 x 2048 x 32 x 128 bf16: per-head FWHT 128 -> bf16
  r3_k     R3 keys (same shape): FWHT 128 + int4 asym per head vector
  weight   W 14336 x 4096 bf16 -> W.H bf16 + MXFP4 + int4 sym g128, one read

Reported beside the step (not part of it): tiny, 256 x 128 float32 with
FWHT 128, int4 sym g32 and the rotated float32 output; its 282,624 bytes take
35 ns at HBM peak, so its launch time measures latency, not bandwidth.

Measured when named in --only (not part of the step): r1_mx32 and
r4_mx32, the R1 and R4 inputs with a block-32 rotation fused with MXFP4
(E2M1 codes, one E8M0 scale per block of 32); r1_nv16 and r4_nv16, the same
inputs with a block-16 rotation fused with NVFP4 (one E4M3 scale per block
of 16); r1_random, the R1 part with a
random Hadamard H diag(+-1); r4_rpbh, the R4 part with RPBH (permutation,
signs, blocks of 2048); down_out, the output-side fusion R1^T W on down_proj
[4096, 14336]; r1_5120, R1 at hidden 5120 (Kronecker 20 x 256); r4_12288,
r4_13824 and r4_17920, R4 at full intermediate widths 12 x 1024, 108 x 128
and 140 x 128; out_5120 and out_8192, output-side fusion of square weights
over 5120 (20 x 256) and 8192 rows; r1_8192, R1 at hidden 8192; r4_b1024,
r4_b256 and r4_b64, the R4 input with blocks of 1024, 256 and 64.  A default
run (no --only) also times r1_mx32, r1_nv16, r1_random, r4_rpbh, down_out,
r4_13824 and r4_17920 alone after the step and reports them under
config.next_rows (not in the value).

The step touches about 2 GB, eight times the 256 MB Infinity Cache, and no
two launches read the same tensor, so every launch reads its input from HBM.
Warm-up runs at least --warmup steps and at least --min-warmup-s seconds
(both reported).  Timing uses HIP events on the stream the
kernels are launched on (torch's current stream).  The value is algorithmic
bytes (one read of each input plus every mandatory output write) per second
over K whole steps with no event between launches.  The per-part durations
(and the roofline) time each part alone: at least K launches back to back,
each on the next of n copies of the part's input (n copies span at least
640 MiB), one event pair around them all.  The same is timed for a plain
streaming kernel (libhrstream.so: 16-byte streaming loads and stores, no
arithmetic) that reads the part's input from the same copies and writes the
rest of its algorithmic bytes: stream_floor_ms is what a launch of that shape
takes here with no computation, and of_stream_floor = stream_floor_ms / ms.
Each part's single-launch time
inside K more steps, an event pair around every launch, is reported too
(ms_single, the mean, with ms_single_median and ms_single_min: it adds the
events' few microseconds, which matter for the 42 MB R1 launch).  copy_reference times the runtime's 256 MiB device copy the same
way, as a reference point.  valu_clock_mhz is the shader clock measured
right before and right after the timed steps (an FMA issue-rate probe in
libhrstream.so): boxes of this model run at different clocks, which moves the
parts that are bound by their instruction stream.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, AMD published peak
METRIC = "rotate+quantize GB/s and rows/s on 1 MI355X; fraction of HBM peak"
PARTS = ("r1", "r4", "r4_kron", "r3_q", "r3_k", "weight")
EXTRA_PARTS = ("r1_mx32", "r4_mx32", "r1_nv16", "r4_nv16", "r1_random", "r4_rpbh",
               "down_out", "r1_5120", "r4_12288", "r4_13824", "r4_17920", "out_5120",
               "out_8192", "r1_8192", "r4_b1024", "r4_b256", "r4_b64")   # measured only when named in --only
# one part per row beside the step (block-32 MXFP4, randomised rotations,
# output-side fusion, NVFP4) and the widest Kronecker base orders: timed alone
# after the step in a default run, reported under config.next_rows
NEXT_DEFAULT = ("r1_mx32", "r1_nv16", "r1_random", "r4_rpbh", "down_out", "r4_13824", "r4_17920")
COPY_BYTES = 256 * 1024 * 1024
CYCLE_BYTES = 640 * 1024 * 1024   # input copies cycled per part when timing it alone


def sources_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "hadamard_rotation_preprocessing_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def qbytes(rows, n, spec):
    groups = rows * n // spec.group_size
    sb = {"f32": 4, "bf16": 2, "e8m0": 1}[spec.scale_dtype]
    zb = (groups + 1) // 2 if (spec.format == "int" and not spec.sym) else 0
    return rows * n // 2 + groups * sb + zb


def build_parts(hr, synth, torch, only):
    """Inputs (CPU and device), launches and algorithmic bytes per kernel."""
    W = synth.WORKLOADS
    dev = "cuda:0"
    parts = {}
    host = {}

    def want(name):
        return only is None or name in only

    if want("r1"):
        w = W["r1"]
        x = synth.make_inputs(w)
        spec = hr.QSpec.from_dict(w.qspecs[0])
        xg = x.to(dev)
        out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
        parts["r1"] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec: hr.rotate_quantize_act(xg, 0, spec, out=out),
                           bytes=x.numel() * 2 + qbytes(x.shape[0], w.n, spec), rows=x.shape[0])
        host["r1"] = (x, w.n, 0, [spec], False)
    # block-32 rotation fused with MXFP4 on the R1 and R4 inputs: measured
    # only when named in --only (not part of the hot-path step)
    for name, wn in (("r1_mx32", "r1"), ("r4_mx32", "r4")):
        if only is not None and name in only:
            w = W[wn]
            x = synth.make_inputs(w)
            spec = hr.QSpec.mxfp4()
            xg = x.to(dev)
            out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
            parts[name] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec: hr.rotate_quantize_act(xg, 32, spec, out=out),
                               bytes=x.numel() * 2 + qbytes(x.shape[0], w.n, spec), rows=x.shape[0])
            host[name] = (x, w.n, 32, [spec], False)
    # block-16 rotation fused with NVFP4 (E4M3 block scales, unit tensor
    # scale) on the R1 and R4 inputs
    for name, wn in (("r1_nv16", "r1"), ("r4_nv16", "r4")):
        if only is not None and name in only:
            w = W[wn]
            x = synth.make_inputs(w)
            spec = hr.QSpec.nvfp4()
            xg = x.to(dev)
            out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
            parts[name] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec: hr.rotate_quantize_act(xg, 16, spec, out=out),
                               bytes=x.numel() * 2 + x.numel() // 2 + x.numel() // 16, rows=x.shape[0])
    # randomised rotations (hr_mix): the random Hadamard H diag(+-1) on the R1
    # input, and RPBH (permutation, signs, blocks of 2048) on the R4 input
    for name, wn, block, pm, si, so in (("r1_random", "r1", 0, False, False, True),
                                         ("r4_rpbh", "r4", 2048, True, True, False)):
        if only is not None and name in only:
            w = W[wn]
            x = synth.make_inputs(w)
            spec = hr.QSpec.from_dict(w.qspecs[0])
            xg = x.to(dev)
            mix = {}
            if pm:
                mix["perm"] = synth.permutation(w.n, 101).to(dev)
            if si:
                mix["in_signs"] = synth.rademacher(w.n, 102).to(dev)
            if so:
                mix["out_signs"] = synth.rademacher(w.n, 103).to(dev)
            out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
            parts[name] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec, block=block, mix=mix:
                               hr.rotate_quantize_act(xg, block, spec, out=out, mix=mix),
                               bytes=x.numel() * 2 + qbytes(x.shape[0], w.n, spec), rows=x.shape[0])
    # output-side fusion W' = R1^T W on down_proj [4096, 14336] (full width
    # along out_features)
    if only is not None and "down_out" in only:
        wd = synth.make_inputs(W["weight"], out_features=4096, in_features=14336).to(dev)
        yd = torch.empty_like(wd)
        parts["down_out"] = dict(x=wd, fn=lambda wd=wd, yd=yd: hr.rotate_fuse_weight_out(wd, 0, out=yd),
                                 bytes=wd.numel() * 4, rows=wd.shape[0])
    # Kronecker widths of other model sizes: R1 at hidden 5120 (20 x 256),
    # R4 at full intermediate widths 12288 (12 x 1024), 13824 (108 x 128) and
    # 17920 (140 x 128); output-side fusion over 5120 (20 x 256) and 8192 rows
    # and R1 at hidden 8192 (blocks of 8192), R4 with blocks of 1024
    for name, wn, kw, block in (("r1_5120", "r1", dict(hidden=5120), 0), ("r4_12288", "r4", dict(inter=12288), 0),
                                ("r4_13824", "r4", dict(inter=13824), 0), ("r4_17920", "r4", dict(inter=17920), 0),
                                ("r1_8192", "r1", dict(hidden=8192), 0), ("r4_b1024", "r4", {}, 1024),
                                ("r4_b256", "r4", {}, 256), ("r4_b64", "r4", {}, 64)):
        if only is not None and name in only:
            w = W[wn]
            x = synth.make_inputs(w, **kw)
            n = x.shape[1]
            spec = hr.QSpec.from_dict(w.qspecs[0])
            xg = x.to(dev)
            out = hr.alloc_quant_outputs(x.shape[0], n, spec, dev)
            parts[name] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec, block=block:
                               hr.rotate_quantize_act(xg, block, spec, out=out),
                               bytes=x.numel() * 2 + qbytes(x.shape[0], n, spec), rows=x.shape[0])
    for name, rows_out in (("out_5120", 5120), ("out_8192", 8192)):
        if only is not None and name in only:
            wo = synth.make_inputs(W["weight"], out_features=rows_out, in_features=rows_out).to(dev)
            yo = torch.empty_like(wo)
            parts[name] = dict(x=wo, fn=lambda wo=wo, yo=yo: hr.rotate_fuse_weight_out(wo, 0, out=yo),
                               bytes=wo.numel() * 4, rows=wo.shape[0])
    if want("r4") or want("r4_kron"):
        w = W["r4"]
        x = synth.make_inputs(w)
        spec = hr.QSpec.from_dict(w.qspecs[0])
        xg = x.to(dev)
        b = x.numel() * 2 + qbytes(x.shape[0], w.n, spec)
        if want("r4"):
            out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
            parts["r4"] = dict(x=xg, fn=lambda xg=xg, out=out, spec=spec: hr.rotate_quantize_act(xg, 2048, spec, out=out),
                               bytes=b, rows=x.shape[0])
            host["r4"] = (x, w.n, 2048, [spec], False)
        if want("r4_kron"):
            # its own copy of the input: right after r4, reads of r4's tensor
            # could still hit the 256 MB Infinity Cache
            xk = xg.clone()
            out2 = hr.alloc_quant_outputs(x.shape[0], w.n, spec, dev)
            parts["r4_kron"] = dict(x=xk, fn=lambda xk=xk, out=out2, spec=spec: hr.rotate_quantize_act(xk, 0, spec, out=out2),
                                    bytes=b, rows=x.shape[0])
            host["r4_kron"] = (x, w.n, 0, [spec], False)
    if want("r3_q") or want("r3_k"):
        w = W["r3"]
        q, k = synth.make_inputs(w)
        spec = hr.QSpec.from_dict(w.qspecs[0])
        rows = q.numel() // 128
        if want("r3_q"):
            qg = q.to(dev)
            yq = torch.empty_like(qg)
            parts["r3_q"] = dict(x=qg, fn=lambda qg=qg, yq=yq: hr.rotate(qg, 0, out=yq), bytes=q.numel() * 4, rows=rows)
            host["r3_q"] = (q.reshape(rows, 128), 128, 0, [], True)
        if want("r3_k"):
            kg = k.to(dev)
            out = hr.alloc_quant_outputs(rows, 128, spec, dev)
            parts["r3_k"] = dict(x=kg, fn=lambda kg=kg, out=out, spec=spec: hr.rotate_quantize_act(kg, 0, spec, out=out),
                                 bytes=k.numel() * 2 + qbytes(rows, 128, spec), rows=rows)
            host["r3_k"] = (k.reshape(rows, 128), 128, 0, [spec], False)
        del q, k
    if want("weight"):
        w = W["weight"]
        x = synth.make_inputs(w)
        specs = [hr.QSpec.from_dict(d) for d in w.qspecs]
        xg = x.to(dev)
        rows = x.shape[0]
        out = {"w_rot": torch.empty_like(xg), "quant": [hr.alloc_quant_outputs(rows, w.n, s, dev) for s in specs]}
        parts["weight"] = dict(x=xg, fn=lambda xg=xg, out=out, specs=specs: hr.rotate_fuse_weight(xg, 0, specs, out=out),
                               bytes=x.numel() * 4 + sum(qbytes(rows, w.n, s) for s in specs), rows=rows)
        host["weight"] = (x, w.n, 0, specs, True)
    return parts, host


def cpu_baseline(host, fraction):
    """Time the oracle (as it stands) on the first rows of every part: the
    same fraction of each part's rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    total_bytes = 0
    t0 = time.perf_counter()
    for name, (x, n, block, specs, write_rot) in host.items():
        rows = max(2, int(x.shape[0] * fraction)) // 2 * 2
        xs = x.reshape(-1, n)[:rows]
        y = oracle.rotate(xs, n, block)
        for s in specs:
            if s.format == "mxfp4":
                r = oracle.mxfp4_quant(y, 32)
            else:
                r = oracle.rtn_quant(y, s.group_size, 4, s.sym, s.scale_dtype)
            oracle.pack_nibbles(r.codes)
            if r.zeros is not None:
                oracle.pack_nibbles(r.zeros)
        if write_rot:
            oracle.bf16_round(y)
        es = 2
        total_bytes += rows * n * es + (rows * n * es if write_rot else 0) + sum(
            rows * n // 2 + rows * n // s.group_size * {"f32": 4, "bf16": 2, "e8m0": 1}[s.scale_dtype]
            + ((rows * n // s.group_size + 1) // 2 if (s.format == "int" and not s.sym) else 0) for s in specs)
        del y
    dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "first %.4g of the rows of every part (%d bytes of the step's workload), "
                      "float64 dense-matrix oracle, %.1f s wall" % (fraction, total_bytes, dt)}


def time_tiny(hr, synth, torch, stream, launches):
    """The tiny workload (256 x 128 float32, FWHT 128, int4 sym g32, rotated
    float32 written), timed alone with an event pair per launch.  It moves
    282,624 bytes, which HBM would carry in 35 ns: a launch takes microseconds,
    so the figure measures launch latency, not bandwidth (reported outside
    the step)."""
    w = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(w).to("cuda:0")
    spec = hr.QSpec.from_dict(w.qspecs[0])
    out = hr.alloc_quant_outputs(x.shape[0], w.n, spec, "cuda:0")
    out["y_rot"] = torch.empty_like(x)
    for _ in range(5):
        hr.rotate_quantize_act(x, 0, spec, y_rot=True, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record(stream)
        hr.rotate_quantize_act(x, 0, spec, y_rot=True, out=out)
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    nbytes = x.numel() * 4 * 2 + qbytes(x.shape[0], w.n, spec)
    return {"ms_median": round(med, 5), "ms_min": round(ms[0], 5), "bytes": nbytes,
            "GB_s": round(nbytes / (med * 1e-3) / 1e9, 1), "frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
            "rows_per_s": round(x.shape[0] / (med * 1e-3), 1), "latency_bound": True,
            "dispatches": 5 + launches}


def stream_lib():
    """ctypes handle of libhrstream.so (the streaming reference), or None."""
    import ctypes
    path = os.path.join(ROOT, "hadamard_rotation_preprocessing_amd", "lib", "libhrstream.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.hr_stream_ref.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hr_stream_ref.restype = ctypes.c_int
    lib.hr_clock_ref.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hr_clock_ref.restype = ctypes.c_int
    return lib


def valu_clock_mhz(torch, stream, sref, iters=20000):
    """Shader clock from libhrstream's FMA issue probe: four waves per SIMD,
    each issuing iters * 8 independent wave64 FMAs (4 cycles each), so every
    SIMD is busy 4 * iters * 8 * 4 cycles.  The GPU's clock under power
    management differs between boxes, and the parts bound by their
    instruction stream (r4_kron, and r1, r4 and weight in part) follow it."""
    if sref is None:
        return None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 4 * cus
    out = torch.empty(blocks, dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream
    for _ in range(2):
        if sref.hr_clock_ref(out.data_ptr(), blocks, iters // 10, sp) != 0:
            raise RuntimeError("clock probe launch failed")
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    if sref.hr_clock_ref(out.data_ptr(), blocks, iters, sp) != 0:
        raise RuntimeError("clock probe launch failed")
    b.record(stream)
    torch.cuda.synchronize()
    cycles = 4 * iters * 8 * 4
    return round(cycles / (a.elapsed_time(b) * 1e-3) / 1e6, 1)


def time_back_to_back(torch, stream, part, launches, sref=None):
    """Average duration of one part's launches run back to back, each on the
    next of n copies of its input (n copies span at least CYCLE_BYTES, 2.5
    times the 256 MB Infinity Cache, so no launch finds its input there): one
    event pair around at least `launches` launches (k, after n untimed
    ones).  With sref (the streaming reference library), the same is timed
    for a plain streaming kernel that reads the part's input bytes from the
    same copies and writes the rest of its algorithmic bytes: the floor of
    that shape.  Returns (ms, n, k, floor_ms or None)."""
    x = part["x"]
    nbytes = x.numel() * x.element_size()
    n = max(1, -(-CYCLE_BYTES // nbytes))
    xs = [x] + [x.clone() for _ in range(n - 1)]
    k = -(-max(launches, 2 * n) // n) * n
    for i in range(n):
        part["fn"](xs[i])
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(k):
        part["fn"](xs[i % n])
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / k
    floor_ms = None
    if sref is not None:
        wbytes = (part["bytes"] - nbytes) // 16 * 16
        dst = torch.empty(max(wbytes, 16), dtype=torch.uint8, device=x.device)
        sp = stream.cuda_stream

        def ref(i):
            if sref.hr_stream_ref(xs[i].data_ptr(), nbytes // 16 * 16, dst.data_ptr(), wbytes, sp) != 0:
                raise RuntimeError("streaming reference launch failed")
        for i in range(n):
            ref(i)
        a.record(stream)
        for i in range(k):
            ref(i % n)
        b.record(stream)
        torch.cuda.synchronize()
        floor_ms = a.elapsed_time(b) / k
        del dst
    del xs
    return ms, n, k, floor_ms


def copy_reference(torch, stream, pairs=3, launches=12):
    """The runtime's device copy (torch's copy_, a device-to-device memcpy)
    of 256 MiB into 256 MiB, back to back over `pairs` buffer pairs, timed
    like the parts: a reference point for a plain read + write stream (it is
    not a ceiling: the parts that stream whole lines run faster)."""
    bufs = [(torch.full((COPY_BYTES,), 1, dtype=torch.uint8, device="cuda"),
             torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")) for _ in range(pairs)]
    for src, dst in bufs:
        dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(launches):
        src, dst = bufs[i % pairs]
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / launches
    del bufs
    gbs = 2 * COPY_BYTES / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 5), "bytes": 2 * COPY_BYTES, "GB_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "kind": "torch copy_, 256 MiB -> 256 MiB, back to back over %d buffer pairs" % pairs}


def traffic_for(kernel: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("sources_digest") != digest or kernel not in d.get("kernels", {}):
        return None
    return d["kernels"][kernel].get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep warming up (untimed steps) until this much wall time has passed")
    ap.add_argument("--only", default=None, help="comma-separated subset of %s (for profiling), or of %s (block-32 MXFP4 "
                         "on the R1 / R4 inputs)" % (",".join(PARTS), ",".join(EXTRA_PARTS)))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the parts timed beside the step in a default run (%s)" % ",".join(NEXT_DEFAULT))
    ap.add_argument("--cpu-fraction", type=float, default=1.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 256 MiB device copy three times "
                         "(reference for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path shards rows across GPUs with no communication, "
              "so it runs and reports a single MI355X (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import hadamard_rotation_preprocessing_amd as hr
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    only = set(args.only.split(",")) if args.only else None
    t_gen = time.perf_counter()
    parts, host = build_parts(hr, synth, torch, only)
    torch.cuda.synchronize()
    print("inputs ready in %.1f s: %s" % (time.perf_counter() - t_gen, ", ".join(parts)), file=sys.stderr, flush=True)
    names = [p for p in PARTS + EXTRA_PARTS if p in parts]

    # warm-up: the W steps asked for, then more untimed steps until at least
    # MIN_WARMUP_S of wall time has passed.  Right after idle the first ~10 ms
    # of steps ran about 12 % slower (measured: 0.40 ms/step over 20 steps
    # after a 2 ms warm-up, 0.36 ms/step after a longer one), so a short
    # step-count warm-up alone would time that ramp, not the kernels.
    t_w = time.perf_counter()
    warm_steps = 0
    while warm_steps < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        for nm in names:
            parts[nm]["fn"]()
        warm_steps += 1
        if warm_steps >= args.warmup and warm_steps % 8 == 0:
            torch.cuda.synchronize()   # at most 8 steps queued ahead of the GPU
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    # the timed region: K whole steps, nothing recorded between launches
    stream = torch.cuda.current_stream()
    sref = stream_lib()
    clock_before = valu_clock_mhz(torch, stream, sref)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for nm in names:
            parts[nm]["fn"]()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # per-launch durations (parts, roofline): each part alone, K launches back
    # to back over copies of its input, one event pair around them all
    clock_after = valu_clock_mhz(torch, stream, sref)
    b2b = {nm: time_back_to_back(torch, stream, parts[nm], args.steps, sref) for nm in names}
    # and single launches inside K more steps, an event pair around each (the
    # events add a few microseconds per launch, so they stay out of the timed
    # region)
    ev = {nm: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for nm in names}
    for s in range(args.steps):
        for nm in names:
            a, b = ev[nm][s]
            a.record(stream)
            parts[nm]["fn"]()
            b.record(stream)
    torch.cuda.synchronize()
    tiny = None
    copy_ref = None
    if only is None:
        tiny = time_tiny(hr, synth, torch, stream, max(args.steps, 20))
        copy_ref = copy_reference(torch, stream)
    next_rows = None
    if only is None and not args.no_next_rows:
        # beside the step, not part of it: each part alone, back to back over
        # copies of its input, as the step's parts are timed (before the copy
        # calibration, whose copies must be the run's last)
        # optional: a failure here is reported in the line, not fatal to it
        next_rows = {}
        try:
            nparts, _ = build_parts(hr, synth, torch, set(NEXT_DEFAULT))
            for nm in NEXT_DEFAULT:
                ms, copies, launches, floor_ms = time_back_to_back(torch, stream, nparts[nm], min(args.steps, 100),
                                                                   sref)
                gbs = nparts[nm]["bytes"] / (ms * 1e-3) / 1e9
                next_rows[nm] = {"ms": round(ms, 5), "bytes": nparts[nm]["bytes"], "GB_s": round(gbs, 1),
                                 "frac": round(gbs / HBM_PEAK_GBS, 4), "input_copies": copies, "launches": launches}
                if floor_ms is not None:
                    next_rows[nm]["stream_floor_ms"] = round(floor_ms, 5)
                    next_rows[nm]["of_stream_floor"] = round(floor_ms / ms, 4)
            del nparts
            torch.cuda.synchronize()
        except Exception as e:   # noqa: BLE001
            next_rows["error"] = "%s: %s" % (type(e).__name__, e)
            print("parts beside the step not measured: %s" % next_rows["error"], file=sys.stderr, flush=True)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_per_step = total_ms / args.steps

    step_bytes = sum(parts[nm]["bytes"] for nm in names)
    step_rows = sum(parts[nm]["rows"] for nm in names)
    per = {}
    for nm in names:
        ms, copies, launches, floor_ms = b2b[nm]
        singles = sorted(a.elapsed_time(b) for a, b in ev[nm])
        ms_single = sum(singles) / args.steps
        gbs = parts[nm]["bytes"] / (ms * 1e-3) / 1e9
        per[nm] = {"ms": round(ms, 5), "bytes": parts[nm]["bytes"], "GB_s": round(gbs, 1),
                   "frac": round(gbs / HBM_PEAK_GBS, 4), "rows_per_s": round(parts[nm]["rows"] / (ms * 1e-3), 1),
                   "input_copies": copies, "launches": launches, "ms_single": round(ms_single, 5),
                   "frac_single": round(parts[nm]["bytes"] / (ms_single * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "ms_single_median": round(singles[len(singles) // 2], 5), "ms_single_min": round(singles[0], 5)}
        if floor_ms is not None:
            per[nm]["stream_floor_ms"] = round(floor_ms, 5)
            per[nm]["stream_floor_frac"] = round(parts[nm]["bytes"] / (floor_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            per[nm]["of_stream_floor"] = round(floor_ms / ms, 4)
    dom = max(names, key=lambda nm: per[nm]["ms"])
    digest = sources_digest()
    roofline = {"bound": "hbm", "kernel": dom, "achieved": per[dom]["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": per[dom]["frac"], "traffic": traffic_for(dom, digest),
                "algorithmic_bytes_per_launch": parts[dom]["bytes"], "launch_ms": per[dom]["ms"]}
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": warm_steps, "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded tensors shaped like 8B-class layers (no real activations or weights)",
        "config": {"workload": "hot-path step: " + " + ".join(names), "bytes_per_step": step_bytes,
                   "rows_per_step": step_rows, "io": "bf16 in; int4/MXFP4 codes, bf16 scales/outputs",
                   "parts": per, "sum_of_parts_ms": round(sum(per[nm]["ms"] for nm in names), 5),
                   "tiny": tiny, "copy_reference": copy_ref, "next_rows": next_rows,
                   "valu_clock_mhz": {"before_timed_steps": clock_before, "after_timed_steps": clock_after}},
        "rows_per_s": round(step_rows / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "sources_digest": digest,
    }
    if not args.no_cpu_baseline and only is None:
        out["cpu_baseline"] = cpu_baseline(host, args.cpu_fraction)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
