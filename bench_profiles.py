#!/usr/bin/env python3
"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/.

  python bench_profiles.py trace <kernel_trace.csv> <bench JSON line file>
      per-part kernel durations, split by phase: the timed steps (launches
      back to back, so neighbouring kernels overlap) and the event pass that
      gives bench.py's per-part times; then the tiny workload's launches.
  python bench_profiles.py traffic <fetch counter_collection.csv>
      <write counter_collection.csv> <bench JSON line of the fetch run>
      <out.txt> [traffic.json]
      HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE run (KiB per
      dispatch), scaled by what the same counters read for the runtime's
      256 MiB device copy (bench.py --copy-calibration); appends the summary
      to out.txt and writes traffic.json (stamped with the kernel sources'
      digest, which bench.py checks before reporting roofline.traffic).
  python bench_profiles.py mem <SQ counter_collection.csv> <its bench JSON line file>
      <TD/TA/TCP counter_collection.csv> <its bench JSON line file>
      per-part memory-pipeline figures: vector memory instructions per wave;
      TD busy and TD stalled by the L2 (TD_TD_BUSY, TD_TC_STALL) and TA
      address stalls by the L2 (TA_ADDR_STALLED_BY_TC_CYCLES) as fractions
      of 256 CUs x GRBM_GUI_ACTIVE / 8 cycles; L2 request latency in cycles
      (TCP_TCC_*_REQ_LATENCY / TCP_TCC_*_REQ).
  python bench_profiles.py sq <counter_collection.csv> <bench JSON line file>
      per-part SQ counter averages with derived figures:
        VALU instructions per wave = SQ_INSTS_VALU / SQ_WAVES;
        VALU busy = SQ_ACTIVE_INST_VALU * 4 / (4 SIMDs * 256 CUs *
          GRBM_GUI_ACTIVE / 8) (a wave64 instruction occupies its SIMD for 4
          cycles; GRBM_GUI_ACTIVE is summed over the 8 XCDs);
        wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.

Launches are matched to bench.py's parts by order: the bench JSON line gives
the parts, the steps and the warm-up steps run.  bench.py launches the
warm-up steps and the timed steps (every part once per step), then each part
alone back to back (input_copies untimed launches, then `launches` timed
ones, and the streaming reference for its shape), then the event pass
(every part once per step).  Kernels of the runtime, of torch (clones,
copies, fills) and the streaming reference are skipped.
"""
import csv
import hashlib
import json
import os
import statistics
import sys


def is_lib(name):
    """A launch of the rotate + quantize library (not the runtime's copies,
    torch's kernels or bench.py's streaming and clock references)."""
    return not name.startswith(("__amd", "void at::")) and "stream_kernel" not in name and "clock_kernel" not in name


def lib_rows(rows, name_of):
    return [r for r in rows if is_lib(name_of(r))]


def phase_of(d):
    """Phase and part of each library launch, in launch order:
    [(phase, part)] with phase warm / step / b2b / event."""
    names = list(d["config"]["parts"].keys())
    steps, warm = d["steps"], d["warmup_steps_run"]
    seq = [("warm", n) for _ in range(warm) for n in names]
    seq += [("step", n) for _ in range(steps) for n in names]
    for n in names:
        p = d["config"]["parts"][n]
        seq += [("b2b_warm", n)] * p.get("input_copies", 0) + [("b2b", n)] * p.get("launches", 0)
    seq += [("event", n) for _ in range(steps) for n in names]
    return seq

def cmd_trace(argv):
    trace, bench = argv[0], argv[1]
    d = json.loads(open(bench).read().strip().splitlines()[-1])
    names = list(d["config"]["parts"].keys())
    rows = lib_rows(list(csv.DictReader(open(trace))), lambda r: r["Kernel_Name"])
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    seq = phase_of(d)
    per = {n: {"step": [], "b2b": [], "event": [], "kernel": ""} for n in names}
    for (phase, n), r in zip(seq, rows):
        if phase in per[n]:
            per[n][phase].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
            per[n]["kernel"] = r["Kernel_Name"]
    print("%-8s %6s %12s %12s %12s %10s  %s" % ("part", "calls", "step_avg_us", "alone_avg_us", "event_avg_us",
                                                "alone_min", "kernel"))
    for n in names:
        p = per[n]
        print("%-8s %6d %12.2f %12.2f %12.2f %10.2f  %s" % (
            n, len(p["step"]) + len(p["b2b"]) + len(p["event"]), statistics.mean(p["step"]), statistics.mean(p["b2b"]),
            statistics.mean(p["event"]), min(p["b2b"]), p["kernel"][:110]))
    tail = rows[len(seq):]
    tiny = d["config"].get("tiny") or {}
    ntiny = tiny.get("dispatches", len(tail))
    if tail:
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in tail[:ntiny]]
        print("tiny     %6d %12s %12.2f %12s %10.2f  %s" % (len(durs), "-", statistics.median(durs), "-", min(durs),
                                                           tail[0]["Kernel_Name"][:110]))
    # parts timed beside the step (config.next_rows): each alone, back to
    # back over copies of its input (the first input_copies launches untimed)
    rest = tail[ntiny:]
    for n, p in (d["config"].get("next_rows") or {}).items():
        if not isinstance(p, dict):
            continue   # "error": those parts were not measured
        k0, k = p["input_copies"], p["launches"]
        mine, rest = rest[:k0 + k], rest[k0 + k:]
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in mine[k0:]]
        if durs:
            print("%-8s %6d %12s %12.2f %12s %10.2f  %s" % (n, len(durs), "-", statistics.mean(durs), "-", min(durs),
                                                            mine[-1]["Kernel_Name"][:110]))
    print("bench: value %.1f GB/s, ms_per_step %.5f, sum of parts (alone, back to back) %.5f ms, warm-up %d steps "
          "in %.2f s" % (d["value"], d["ms_per_step"], d["config"]["sum_of_parts_ms"], d["warmup_steps_run"],
                         d["warmup_s"]))
    print("bench per part (us): " + ", ".join("%s %.2f alone / %.2f single" % (
        n, 1e3 * d["config"]["parts"][n]["ms"], 1e3 * d["config"]["parts"][n]["ms_single"]) for n in names))


COPY_KIB = 256 * 1024


def sources_digest(root):
    h = hashlib.sha256()
    d = os.path.join(root, "hadamard_rotation_preprocessing_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def per_dispatch(path, counter):
    vals = {}
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        vals[k] = vals.get(k, 0.0) + float(r["Counter_Value"])
        names[k] = r["Kernel_Name"]
    return [(names[k], vals[k]) for k in sorted(vals)]


def split(disp, d):
    """Per-part counter values of the timed steps and the event pass, and
    the values of the last three runtime copies (bench.py's
    --copy-calibration: 256 MiB each, after every other launch)."""
    names = list(d["config"]["parts"].keys())
    hot = [x for x in disp if is_lib(x[0])]
    copies = [v for n, v in disp if n.startswith("__amd_rocclr_copyBuffer")][-3:]
    out = {n: [] for n in names}
    for (phase, n), (kn, v) in zip(phase_of(d), hot):
        if phase in ("step", "event"):
            out[n].append(v)
    return out, copies


def cmd_traffic(argv):
    fetch, write, bench, out_txt = argv[0:4]
    out_json = argv[4] if len(argv) > 4 else None
    d = json.loads(open(bench).read().strip().splitlines()[-1])
    names = list(d["config"]["parts"].keys())
    fr, fc = split(per_dispatch(fetch, "FETCH_SIZE"), d)
    wr, wc = split(per_dispatch(write, "WRITE_SIZE"), d)
    rf = COPY_KIB / statistics.median(fc)
    wf = COPY_KIB / statistics.median(wc)
    root = os.path.dirname(os.path.abspath(__file__))
    digest = sources_digest(root)
    lines = ["copy calibration: FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB for %d KiB read and written -> "
             "factors %.4f (read), %.4f (write)" % (statistics.median(fc), statistics.median(wc), COPY_KIB, rf, wf),
             "kernel sources digest: %s" % digest, "",
             "%-10s %14s %14s %14s %8s" % ("part", "read_bytes", "write_bytes", "alg_bytes", "ratio")]
    kern = {}
    for n in names:
        rb = statistics.mean(fr[n]) * rf * 1024
        wb = statistics.mean(wr[n]) * wf * 1024
        alg = d["config"]["parts"][n]["bytes"]
        lines.append("%-10s %14.0f %14.0f %14d %8.4f" % (n, rb, wb, alg, (rb + wb) / alg))
        kern[n] = {"bytes_per_launch": int(round(rb + wb)), "read_bytes": int(round(rb)), "write_bytes": int(round(wb))}
    open(out_txt, "a").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if out_json:
        old = json.load(open(out_json)) if os.path.exists(out_json) else {}
        if old.get("sources_digest") != digest:
            old = {"kernels": {}}
        old["sources_digest"] = digest
        old.setdefault("kernels", {}).update(kern)
        old["source"] = "profiles/traffic_hot_path_step.txt"
        json.dump(old, open(out_json, "w"), indent=1)


def per_part_counters(path, bench):
    """Counter values summed per dispatch, grouped by bench part (timed
    steps and event pass; warm-up dispatches dropped): {part: [dict]}."""
    d = json.loads(open(bench).read().strip().splitlines()[-1])
    names = list(d["config"]["parts"].keys())
    disp = {}
    kname = {}
    for r in csv.DictReader(open(path)):
        k = int(r["Dispatch_Id"])
        disp.setdefault(k, {})
        disp[k][r["Counter_Name"]] = disp[k].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        kname[k] = r["Kernel_Name"]
    order = [k for k in sorted(disp) if is_lib(kname[k])]
    per = {n: [] for n in names}
    for (phase, n), k in zip(phase_of(d), order):
        if phase in ("step", "event"):
            per[n].append(disp[k])
    return per


def cmd_sq(argv):
    path, bench = argv[0], argv[1]
    per = per_part_counters(path, bench)
    names = list(per)
    cu, simd = 256, 4
    print("%-8s %9s %13s %10s %10s %9s %8s  %s" % ("part", "waves", "VALU/wave", "LDS/wave", "VALUbusy", "wait", "cycles",
                                                  "counters (averages per dispatch)"))
    for n in names:
        avg = {c: statistics.mean(x[c] for x in per[n]) for c in per[n][0]}
        w = avg.get("SQ_WAVES", 0.0)
        busy = 100.0 * avg.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (simd * cu * avg["GRBM_GUI_ACTIVE"] / 8)
        wait = 100.0 * avg.get("SQ_WAIT_INST_ANY", 0.0) / avg["SQ_WAVE_CYCLES"]
        print("%-8s %9.0f %13.1f %10.1f %9.1f%% %8.1f%% %8.0f  %s" % (
            n, w, avg["SQ_INSTS_VALU"] / w, avg.get("SQ_INSTS_LDS", 0.0) / w, busy, wait, avg["GRBM_GUI_ACTIVE"] / 8,
            ", ".join("%s=%.0f" % (c, v) for c, v in sorted(avg.items()))))


def cmd_mem(argv):
    sq_path, sq_bench, t_path, t_bench = argv[:4]
    a = {n: {c: statistics.mean(x[c] for x in v) for c in v[0]} for n, v in per_part_counters(sq_path, sq_bench).items()}
    b = {n: {c: statistics.mean(x[c] for x in v) for c in v[0]} for n, v in per_part_counters(t_path, t_bench).items()}
    cu = 256
    print("%-8s %10s %10s %9s %9s %9s %9s %9s" % ("part", "VMEM_RD/wv", "VMEM_WR/wv", "TD busy", "TD<-TC", "TA<-TC",
                                                   "L2 rd lat", "L2 wr lat"))
    for n in a:
        w = a[n]["SQ_WAVES"]
        cyc = b[n]["GRBM_GUI_ACTIVE"] / 8
        print("%-8s %10.2f %10.2f %8.1f%% %8.1f%% %8.1f%% %9.0f %9.0f" % (
            n, a[n]["SQ_INSTS_VMEM_RD"] / w, a[n]["SQ_INSTS_VMEM_WR"] / w,
            100.0 * b[n]["TD_TD_BUSY"] / (cu * cyc), 100.0 * b[n]["TD_TC_STALL"] / (cu * cyc),
            100.0 * b[n]["TA_ADDR_STALLED_BY_TC_CYCLES"] / (cu * cyc),
            b[n]["TCP_TCC_READ_REQ_LATENCY"] / max(b[n]["TCP_TCC_READ_REQ"], 1.0),
            b[n]["TCP_TCC_WRITE_REQ_LATENCY"] / max(b[n]["TCP_TCC_WRITE_REQ"], 1.0)))


def main():
    cmds = {"trace": cmd_trace, "traffic": cmd_traffic, "sq": cmd_sq, "mem": cmd_mem}
    if len(sys.argv) < 2 or sys.argv[1] not in cmds:
        sys.exit(__doc__)
    cmds[sys.argv[1]](sys.argv[2:])


if __name__ == "__main__":
    main()
