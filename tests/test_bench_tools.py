"""Host-side checks of the measurement tooling (no GPU).

bench_profiles.py attributes the launches of a rocprofv3 kernel trace of
bench.py to its parts by launch order, from the bench JSON line of the same
run.  A synthetic trace with known durations per phase checks that order:
warm-up, timed steps, each part alone (untimed copies first), the event
pass, the tiny workload, then the parts timed beside the step.  Runtime and
torch kernels and the streaming reference interleaved with them are skipped.
bench.py refuses more than one GPU before touching one.
"""
import contextlib
import csv
import io
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench_profiles  # noqa: E402


def _bench_line(parts, next_rows, steps=2, warm=3, tiny_dispatches=4):
    per = {n: {"ms": 0.01, "ms_single": 0.012, "input_copies": c, "launches": k} for n, (c, k) in parts.items()}
    nxt = {n: {"ms": 0.02, "input_copies": c, "launches": k} for n, (c, k) in next_rows.items()}
    return {"value": 1.0, "ms_per_step": 0.1, "steps": steps, "warmup_steps_run": warm,
            "config": {"parts": per, "sum_of_parts_ms": 0.02, "tiny": {"dispatches": tiny_dispatches},
                       "next_rows": nxt}, "warmup_s": 0.3}


def _trace(tmp_path, parts, next_rows, steps=2, warm=3, tiny_dispatches=4):
    """Launch sequence of a bench run; durations encode (phase, part)."""
    names = list(parts)
    code = {"warm": 1000, "step": 2000, "b2b_warm": 3000, "b2b": 4000, "event": 5000, "tiny": 6000,
            "next_warm": 7000, "next": 8000}
    seq = []
    for _ in range(warm):
        seq += [("warm", n) for n in names]
    for _ in range(steps):
        seq += [("step", n) for n in names]
    for n in names:
        c, k = parts[n]
        seq += [("b2b_warm", n)] * c + [("b2b", n)] * k
        seq += [("stream", n)] * (c + k)          # the streaming reference: not a library kernel
    for _ in range(steps):
        seq += [("event", n) for n in names]
    seq += [("tiny", "tiny")] * tiny_dispatches
    seq += [("copy", "-")] * 2                     # the runtime's copy: skipped
    for n, (c, k) in next_rows.items():
        seq += [("clone", n)] * (c - 1)            # torch clones of the input copies: skipped
        seq += [("next_warm", n)] * c + [("next", n)] * k
    rows = []
    t = 0
    for i, (phase, n) in enumerate(seq):
        if phase == "stream":
            kname = "void hr_stream_kernel(...)"
            dur = 1
        elif phase == "copy":
            kname = "__amd_rocclr_copyBuffer"
            dur = 1
        elif phase == "clone":
            kname = "void at::native::elementwise_kernel<...>"
            dur = 1
        else:
            kname = "void hr::kernel_%s(...)" % n
            base = code[phase]
            idx = names.index(n) if n in names else list(next_rows).index(n) if n in next_rows else 0
            dur = base + 10 * idx
        rows.append({"Kernel_Name": kname, "Start_Timestamp": str(t), "End_Timestamp": str(t + 1000 * dur)})
        t += 1000 * dur + 5
    path = os.path.join(str(tmp_path), "trace.csv")
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows[::-1])                    # the summary sorts by start time
    return path


def test_trace_summary_attributes_every_phase(tmp_path):
    parts = {"r1": (2, 3), "r4": (1, 4)}
    next_rows = {"down_out": (3, 2), "r4_rpbh": (1, 5)}
    trace = _trace(tmp_path, parts, next_rows)
    bench = os.path.join(str(tmp_path), "bench.json")
    with open(bench, "w") as fh:
        fh.write("inputs ready\n" + json.dumps(_bench_line(parts, next_rows)) + "\n")
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        bench_profiles.cmd_trace([trace, bench])
    got = {}
    for line in out.getvalue().splitlines():
        f = line.split()
        if f and f[0] in ("r1", "r4", "tiny", "down_out", "r4_rpbh"):
            got[f[0]] = f
    # per part: calls (steps + timed alone + events), step avg, alone avg,
    # event avg (us); durations encode the phase
    assert got["r1"][1:5] == ["7", "2000.00", "4000.00", "5000.00"]
    assert got["r4"][1:5] == ["8", "2010.00", "4010.00", "5010.00"]
    assert got["tiny"][1] == "4" and got["tiny"][3] == "6000.00"
    # parts beside the step: timed launches only, after the untimed copies
    assert got["down_out"][1] == "2" and got["down_out"][3] == "8000.00"
    assert got["r4_rpbh"][1] == "5" and got["r4_rpbh"][3] == "8010.00"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr
