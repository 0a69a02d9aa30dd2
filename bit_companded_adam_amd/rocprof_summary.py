"""Summaries of rocprofv3 output for the measurement notes (profiles/).

    python -m bit_companded_adam_amd.rocprof_summary trace DIR [--title T] [--cmd C]
        [--bytes REGEX=BYTES_PER_LAUNCH ...] [--order REGEX] [--skip K]
    python -m bit_companded_adam_amd.rocprof_summary counters --fetch DIR --write DIR
        --cal-fetch DIR --cal-write DIR --params N --alg-read B --alg-write B
        [--kernel REGEX] [--json OUT] [--sha SHA] [--cmds JSON]

trace: per-kernel calls, total, average, minimum and maximum duration from a
--kernel-trace run (DIR/run_kernel_trace.csv); with --bytes, the GB/s and
fraction of 8 TB/s of each matching kernel from its algorithmic bytes per
launch; with --order, the durations of the matching kernel in dispatch order
(and their average after the first K).

counters: per-dispatch counter values of the step kernel from --pmc runs
(DIR/run_counter_collection.csv), the HBM bytes per launch from FETCH_SIZE and
WRITE_SIZE scaled by what the same counters read for a plain copy of 2 GiB
each way (bench.py --calibrate-copy), the VALU instructions per element and
lane, and the shader clock during the step (GRBM_GUI_ACTIVE over the
dispatch's duration, per XCD).  Reads rocprofv3's CSV files only; runs on a
host without a GPU.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import re
import statistics
import sys
from collections import defaultdict

PEAK_HBM_GBS = 8000.0
XCDS = 8                # MI355X: 8 accelerator complex dies
SIMDS = 256 * 4         # 256 CUs x 4 SIMDs


def short_name(name: str) -> str:
    """'void flashopt::(anonymous namespace)::k<24, 1>(args...)' -> 'flashopt::k<24, 1>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for i, ch in enumerate(n):        # cut the argument list: the first '(' at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            break
        out.append(ch)
    return "".join(out).strip()


def _csv(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def trace(args) -> None:
    rows = _csv(_find(args.dir, "kernel_trace.csv"))
    per = defaultdict(list)
    order = []
    for r in rows:
        name = short_name(r["Kernel_Name"])
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per[name].append(us)
        order.append((int(r["Start_Timestamp"]), name, us))
    total = sum(sum(v) for v in per.values())
    nbytes = []
    for spec in args.bytes or []:
        rx, b = spec.rsplit("=", 1)
        nbytes.append((re.compile(rx), float(b)))
    if args.title:
        print(f"# rocprofv3 kernel-trace summary: {args.title}")
    if args.cmd:
        print(f"# command (run from /tmp; $R = repository root): {args.cmd}")
    for line in args.note or []:
        print(f"# {line}")
    print("#")
    head = "# calls   total_ms      avg_us   min_us   max_us   pct"
    print(head + ("    GB/s  of 8 TB/s" if nbytes else "") + "  kernel")
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))[: args.top]:
        line = (f"{len(v):7d} {sum(v) / 1e3:10.2f} {statistics.mean(v):11.1f} {min(v):8.1f} "
                f"{max(v):8.1f} {100 * sum(v) / total:5.1f}")
        if nbytes:
            b = next((b for rx, b in nbytes if rx.search(name)), None)
            if b is None:
                line += " " * 20
            else:
                gbs = b / (statistics.mean(v) * 1e-6) / 1e9
                line += f" {gbs:8.0f}  {gbs / PEAK_HBM_GBS:7.1%}  "
        print(line + "  " + name[:90])
    if args.order:
        rx = re.compile(args.order)
        seq = [us for _, name, us in sorted(order) if rx.search(name)]
        if seq:
            print("#")
            print(f"# durations of the kernels matching '{args.order}' in dispatch order (ms):")
            for i in range(0, len(seq), 12):
                print("#   " + " ".join(f"{x / 1e3:.3f}" for x in seq[i:i + 12]))
            k = args.skip
            if len(seq) > k:
                print(f"# average over launches {k + 1}..{len(seq)}: {statistics.mean(seq[k:]) / 1e3:.3f} ms; "
                      f"over all {len(seq)}: {statistics.mean(seq) / 1e3:.3f} ms")


def _dispatches(d: str, kernel: str):
    """{dispatch id: {counter: value}} and durations (ms) of the matching kernel."""
    rx = re.compile(kernel)
    vals, dur = defaultdict(dict), {}
    for r in _csv(_find(d, "counter_collection.csv")):
        if not rx.search(r["Kernel_Name"]):
            continue
        k = int(r["Dispatch_Id"])
        vals[k][r["Counter_Name"]] = vals[k].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        dur[k] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
    return dict(sorted(vals.items())), dur


def counters(args) -> None:
    cal_f, _ = _dispatches(args.cal_fetch, args.cal_kernel)
    cal_w, _ = _dispatches(args.cal_write, args.cal_kernel)
    copy_bytes = float(args.cal_bytes)
    # FETCH_SIZE / WRITE_SIZE are in KiB; the copy reads and writes copy_bytes
    f_cal = [v["FETCH_SIZE"] * 1024 for v in cal_f.values() if "FETCH_SIZE" in v]
    w_cal = [v["WRITE_SIZE"] * 1024 for v in cal_w.values() if "WRITE_SIZE" in v]
    f_factor = copy_bytes / statistics.median(f_cal)
    w_factor = copy_bytes / statistics.median(w_cal)
    fetch, _ = _dispatches(args.fetch, args.kernel)
    write, wdur = _dispatches(args.write, args.kernel)
    fl = [v["FETCH_SIZE"] * 1024 * f_factor for v in fetch.values()]
    wl = list(write.values())
    n = float(args.params)
    rec = {"kernel": args.kernel_label or args.kernel, "workload": args.workload,
           "kernel_sha": args.sha, "fetch_factor": f_factor, "write_factor": w_factor}
    # the last dispatch of each run is a steady step (the first starts from zero moments)
    r_last = fl[-1]
    w_last = wl[-1]["WRITE_SIZE"] * 1024 * w_factor
    rec.update(fetch_bytes_per_launch=r_last, write_bytes_per_launch=w_last,
               hbm_bytes_per_launch=r_last + w_last)
    last_id = list(write)[-1]
    v = write[last_id]
    if "SQ_INSTS_VALU" in v:
        rec["valu_insts_per_launch"] = v["SQ_INSTS_VALU"]
        rec["valu_per_element_lane"] = v["SQ_INSTS_VALU"] * 64 / n
        if len(wl) > 1:
            rec["valu_first_step"] = wl[0]["SQ_INSTS_VALU"]
    if "GRBM_GUI_ACTIVE" in v and wdur.get(last_id):
        per_xcd = v["GRBM_GUI_ACTIVE"] / XCDS
        rec["launch_ms_in_counter_run"] = wdur[last_id]
        rec["sclk_mhz_during_step"] = per_xcd / (wdur[last_id] * 1e-3) / 1e6
        if "SQ_INSTS_VALU" in v:
            # VALU wavefront instructions per SIMD per 4 cycles of the step
            rec["valu_insts_per_simd_quad_cycle"] = v["SQ_INSTS_VALU"] / SIMDS / (per_xcd / 4)
    if "SQ_ACTIVE_INST_VALU2" in v and "SQ_ACTIVE_INST_VALU" in v:
        rec["sq_active_inst_valu"] = v["SQ_ACTIVE_INST_VALU"]
        rec["sq_active_inst_valu2"] = v["SQ_ACTIVE_INST_VALU2"]
    if args.cmds:
        rec["commands"] = json.loads(args.cmds)
    alg_r, alg_w = float(args.alg_read), float(args.alg_write)
    print(f"# HBM read  per launch (scaled)  {r_last / 1e9:.3f} GB = {r_last / n:.4f} B/param (algorithmic {alg_r:g})")
    print(f"# HBM write per launch (scaled)  {w_last / 1e9:.3f} GB = {w_last / n:.4f} B/param (algorithmic {alg_w:g})")
    print(f"# calibration factors: FETCH_SIZE x {f_factor:.4f}, WRITE_SIZE x {w_factor:.4f}")
    for k in ("valu_per_element_lane", "sclk_mhz_during_step", "valu_insts_per_simd_quad_cycle"):
        if k in rec:
            print(f"# {k}: {rec[k]:.4f}")
    for i, (k, vv) in enumerate(write.items()):
        print(f"# dispatch {k}: " + ", ".join(f"{c} {x:.6g}" for c, x in sorted(vv.items())))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title")
    t.add_argument("--cmd")
    t.add_argument("--note", action="append")
    t.add_argument("--bytes", action="append")
    t.add_argument("--order")
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--top", type=int, default=8)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--cal-fetch", required=True)
    c.add_argument("--cal-write", required=True)
    c.add_argument("--cal-kernel", default="neg")
    c.add_argument("--cal-bytes", default=str(2 << 30))
    c.add_argument("--kernel", default="adamw_step")
    c.add_argument("--kernel-label")
    c.add_argument("--workload", default="")
    c.add_argument("--params", required=True)
    c.add_argument("--alg-read", required=True)
    c.add_argument("--alg-write", required=True)
    c.add_argument("--sha", default="")
    c.add_argument("--json")
    c.add_argument("--cmds")
    a = ap.parse_args(argv)
    if a.cmd_name == "trace":
        trace(a)
    else:
        counters(a)


if __name__ == "__main__":
    main(sys.argv[1:])
