#!/usr/bin/env python3
"""rocprofv3 evidence behind the numbers bench.py prints.

Two sub-commands:

``collect --out DIR [--bench-args ...]``
    Runs, each in its own process and under its own time limit:
      1. ``rocprofv3 --kernel-trace --stats -f csv`` around the bench command
         (by default exactly ``python3 bench.py --gpus 1 --steps 20 --warmup 5``,
         the command the bench line is quoted from), keeping that run's JSON line;
      2. one ``rocprofv3 --pmc`` pass per counter group below around the same bench
         command without the CPU-oracle leg (which launches no GPU work), counters
         restricted to this library's kernels;
      3. two ``--pmc`` passes (FETCH_SIZE, then WRITE_SIZE) around a plain 1 GiB
         device copy, the calibration that turns the cache-side byte counters into
         bytes.
    Raw rocprofv3 output stays under DIR.

``summarize --in DIR --out PROFILES``
    Reads DIR and writes, per kernel launch group (kernel name, grid size), a text
    summary ``PROFILES/<kernel>_<workload>.txt``: dispatch count, mean duration over
    all dispatches and over the timed window (the last ``--window`` dispatches of the
    group, the launches bench.py times), the bench line's own figure for comparison,
    and the counters of the timed window turned into rates (MFMA busy, clock, waves
    per CU, VALU and LDS issue, HBM bytes against the algorithmic bytes).  It also
    rewrites ``PROFILES/hbm_traffic.json``, the measured bytes per launch that
    bench.py reports as ``roofline.traffic`` while the library source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DRIVER_ARGS = ["--gpus", "1", "--steps", "20", "--warmup", "5"]
KERNEL_REGEX = "dg_gemm_kernel|quant_1x128_kernel|quant_128x128_kernel"
COPY_MIB = 1024

# Counter groups, one rocprofv3 pass each (at most 8 SQ and 2 GRBM counters a pass).
PMC_PASSES = {
    "sq_core": ["SQ_WAVES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_SALU",
                "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
    "sq_stall": ["SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT",
                 "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_VMEM", "GRBM_GUI_ACTIVE"],
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "lds": ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "SQ_INSTS_LDS_STORE_BANDWIDTH",
            "SQ_WAIT_ANY", "TA_BUSY_avr", "GRBM_GUI_ACTIVE"],
}
OPTIONAL_PASSES = ("lds",)


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------- collect
def run_step(name: str, cmd: list, limit: int, log: str) -> int:
    say(f"profile: {name}: {' '.join(cmd)}")
    t0 = time.time()
    with open(log, "w") as f:
        try:
            rc = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, stdout=f, stderr=subprocess.STDOUT,
                                cwd=ROOT).returncode
        except OSError as e:
            f.write(f"{e}\n")
            rc = 127
    say(f"profile: {name}: rc {rc} after {time.time() - t0:.0f} s")
    return rc


def collect(args) -> int:
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    bench = [sys.executable, "bench.py"] + (args.bench_args or DRIVER_ARGS)
    meta = {"bench_cmd": ["python3", "bench.py"] + (args.bench_args or DRIVER_ARGS), "passes": {}}
    # 1. kernel trace around the bench command; its JSON line is kept beside the trace
    tdir = os.path.join(out, "trace")
    rc = run_step("trace", ["rocprofv3", "--kernel-trace", "--stats", "-f", "csv", "-d", tdir, "-o", "run", "--"]
                  + bench, args.limit, os.path.join(out, "trace.log"))
    meta["trace_rc"] = rc
    if rc != 0:
        json.dump(meta, open(os.path.join(out, "meta.json"), "w"), indent=1)
        return rc
    # 2. counter passes (no CPU-oracle leg: it launches nothing)
    pbench = bench + (["--no-cpu-baseline"] if "--no-cpu-baseline" not in bench else [])
    for pname, ctrs in PMC_PASSES.items():
        pdir = os.path.join(out, "pmc_" + pname)
        # a counter pass over the bench takes seconds; a refused counter set can hang
        rc = run_step(f"pmc {pname}", ["rocprofv3", "--pmc"] + ctrs + ["--kernel-include-regex", KERNEL_REGEX,
                                                                        "-f", "csv", "-d", pdir, "-o", "run", "--"]
                      + pbench, min(args.limit, 150), os.path.join(out, f"pmc_{pname}.log"))
        meta["passes"][pname] = {"counters": ctrs, "rc": rc}
        if rc != 0 and pname in OPTIONAL_PASSES:
            say(f"profile: optional pass {pname} failed (rc {rc}); its counters are left out")
            rc = 0
            continue
        if rc != 0:
            break
    # 3. copy calibration of the byte counters
    if rc == 0:
        for pname in ("fetch", "write"):
            pdir = os.path.join(out, "copy_" + pname)
            rc = run_step(f"copy {pname}", ["rocprofv3", "--pmc"] + PMC_PASSES[pname] + ["-f", "csv", "-d", pdir,
                                                                                        "-o", "run", "--",
                                                                                        sys.executable, "bench.py",
                                                                                        "--copy-calibration-mib",
                                                                                        str(COPY_MIB)],
                          120, os.path.join(out, f"copy_{pname}.log"))
            meta["passes"]["copy_" + pname] = {"rc": rc}
            if rc != 0:
                break
    json.dump(meta, open(os.path.join(out, "meta.json"), "w"), indent=1)
    return rc


# ---------------------------------------------------------------------------- summarize
def read_csv(pattern: str) -> list:
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return None


def total_size(row: dict, base: str) -> int:
    """Work-items of a dispatch's grid or workgroup: the kernel trace gives one column
    per dimension, the counter collection the product."""
    dims = [col(row, f"{base}_{d}") for d in "XYZ"]
    if dims[0] is not None:
        n = 1
        for d in dims:
            n *= int(float(d or 1))
        return n
    return int(float(col(row, base, base + "s") or 0))


def group_key(row: dict) -> tuple:
    return (col(row, "Kernel_Name"), total_size(row, "Grid_Size"), total_size(row, "Workgroup_Size"))


def short_name(kernel: str) -> str:
    m = re.match(r"(?:void )?(?:dg::)?(?:\(anonymous namespace\)::)?(\w+)(<[^()]*>)?", kernel or "")
    if not m:
        return "kernel"
    base = m.group(1)
    targs = (m.group(2) or "").strip("<>")
    targs = re.sub(r"unsigned short|float|true|false", lambda x: {"true": "1", "false": "0"}.get(x.group(0), "t"),
                   targs)
    targs = re.sub(r"[^0-9,]", "", targs)
    return base + ("_" + "x".join(t for t in targs.split(",") if t) if targs else "")


def trace_groups(tdir: str) -> dict:
    """(kernel, grid, wg) -> list of durations in ns, in dispatch order."""
    rows = read_csv(os.path.join(tdir, "**", "*kernel_trace.csv"))
    rows.sort(key=lambda r: int(col(r, "Dispatch_Id", "Correlation_Id") or 0))
    groups = {}
    for r in rows:
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault(group_key(r), []).append(d)
    return groups


def counter_groups(pdir: str) -> dict:
    """(kernel, grid, wg) -> list (dispatch order) of {counter: value}."""
    rows = read_csv(os.path.join(pdir, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        did = int(col(r, "Dispatch_Id", "Correlation_Id") or 0)
        key = group_key(r)
        name = r.get("Counter_Name")
        val = float(r.get("Counter_Value") or 0.0)
        per.setdefault(key, {}).setdefault(did, {})
        per[key][did][name] = per[key][did].get(name, 0.0) + val
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            per[key][did]["_dur_ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: [v[d] for d in sorted(v)] for k, v in per.items()}


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def bench_line(path: str):
    try:
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.startswith("{") and '"metric"' in line:
                    return json.loads(line)
    except OSError:
        pass
    return None


def workload_of(key: tuple, bench: dict, order: list) -> tuple:
    """Which bench workload a launch group belongs to, from the bench line's own launch
    configurations (kernel template arguments and grid), in bench order."""
    return order.get(key, ("unmatched", None))


def summarize(args) -> int:
    src = os.path.abspath(args.inp)
    meta = json.load(open(os.path.join(src, "meta.json")))
    tgroups = trace_groups(os.path.join(src, "trace"))
    bench = bench_line(os.path.join(src, "trace.log"))
    if bench is None:
        print("no bench JSON line in the trace run's output", file=sys.stderr)
        return 1
    counters = {}
    for pname in PMC_PASSES:
        pdir = os.path.join(src, "pmc_" + pname)
        if os.path.isdir(pdir):
            for key, lst in counter_groups(pdir).items():
                counters.setdefault(key, {})[pname] = lst
    # copy calibration: counter KiB per byte copied
    calib = {}
    for pname, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        rows = counter_groups(os.path.join(src, "copy_" + pname))
        best = None
        for key, lst in rows.items():
            vals = [d.get(ctr, 0.0) for d in lst]
            if vals and (best is None or max(vals) > best):
                best = max(vals)
        if best:
            calib[ctr] = (COPY_MIB << 20) / (best * 1024.0)   # bytes per counted byte
    # Which group is which workload: the bench line names each workload's measured
    # launch (headline: roofline.launch_us; secondaries: us).  Groups are matched by
    # the order in which the bench runs them: headline first, then secondaries in
    # the line's order, each capped masked run after its workload, then the casts.
    seq = [("headline", bench["config"]["workload"], bench["roofline"]["launch_us"])]
    for name, s in (bench.get("secondary") or {}).items():
        seq.append(("secondary", name, s["us"]))
        for cap, cs in (s.get("cu_capped") or {}).items():
            seq.append(("capped", f"{name}_cu{cap}", cs["us"]))
    # dispatch order of first appearance of each group
    first = {}
    rows = read_csv(os.path.join(src, "trace", "**", "*kernel_trace.csv"))
    rows.sort(key=lambda r: int(col(r, "Dispatch_Id", "Correlation_Id") or 0))
    for r in rows:
        k = group_key(r)
        if k[0] and ("dg_gemm_kernel" in k[0] or "quant_" in k[0]):
            first.setdefault(k, len(first))
    ordered = sorted(first, key=first.get)
    # a group that reappears (the masked kernel at full width and again at a cap that
    # picks the same configuration) differs in grid size, so groups map one to one
    if len(ordered) != len(seq):
        print(f"warning: {len(ordered)} launch groups vs {len(seq)} bench entries", file=sys.stderr)
    os.makedirs(args.out, exist_ok=True)
    traffic = {}
    cmd = " ".join(meta["bench_cmd"])
    for i, key in enumerate(ordered):
        kind, wname, bench_us = seq[i] if i < len(seq) else ("unmatched", f"group{i}", None)
        durs = tgroups.get(key, [])
        win = durs[-args.window:]
        lines = []
        lines.append(f"# {short_name(key[0])} -- {wname}")
        lines.append("")
        lines.append(f"kernel: {key[0]}")
        lines.append(f"grid: {key[1]} work-items, workgroup {key[2]}")
        lines.append(f"workload: {wname} ({kind} in the bench line)")
        lines.append("")
        lines.append("made by (from the repository root, on one MI355X):")
        lines.append(f"  python3 bench_profile.py collect --out gpurun_out/prof   # runs: rocprofv3 --kernel-trace "
                     f"--stats -f csv -- {cmd}")
        lines.append("  python3 bench_profile.py summarize --in gpurun_out/prof --out profiles")
        lines.append("")
        lines.append("## kernel trace (rocprofv3 --kernel-trace --stats)")
        lines.append(f"dispatches: {len(durs)}")
        lines.append(f"mean duration, all dispatches: {mean(durs) / 1e3:.2f} us")
        lines.append(f"mean duration, timed window (last {len(win)} dispatches): {mean(win) / 1e3:.2f} us "
                     f"(min {min(win) / 1e3:.2f}, max {max(win) / 1e3:.2f})" if win else "timed window: none")
        if durs:
            # in dispatch order: the chip's clock changes show as steps within the run
            lines.append("durations in dispatch order (us): " + " ".join(f"{d / 1e3:.1f}" for d in durs))
        if bench_us is not None:
            lines.append(f"bench line of the traced run (one HIP event pair over its timed launches): {bench_us:.2f} us")
            lines.append("  (the trace adds a few us of dispatch overhead between launches, which the bench line "
                         "counts and the kernel durations do not: it matters only for kernels of a few tens of us)")
        c = counters.get(key, {})
        if c:
            lines.append("")
            lines.append(f"## counters (rocprofv3 --pmc, one pass per group, mean over the last {args.window} "
                         "dispatches of each pass)")

            def cmean(pname, ctr):
                lst = c.get(pname, [])[-args.window:]
                vals = [d[ctr] for d in lst if ctr in d]
                return mean(vals) if vals else None

            for pname, ctrs in PMC_PASSES.items():
                for ctr in ctrs:
                    if ctr.startswith("_"):
                        continue
                    v = cmean(pname, ctr)
                    if v is not None:
                        lines.append(f"{pname:9s} {ctr:32s} {v:18.1f}")
            gui = cmean("sq_core", "GRBM_GUI_ACTIVE")
            dur = cmean("sq_core", "_dur_ns")
            derived = []
            if gui and dur:
                # GRBM_GUI_ACTIVE is summed over the 8 XCDs; the duration is the same
                # dispatch's, from the counter run.  For kernels of a few tens of us the
                # counter window is wider than the kernel and this overstates the clock.
                note = "" if dur >= 100e3 else " (upper bound: the counter window is wider than this short kernel)"
                derived.append(("clock (GRBM_GUI_ACTIVE / 8 / duration of the same dispatch)",
                                f"{gui / 8 / dur:.3f} GHz{note}"))
                derived.append(("mean duration in the counter run", f"{dur / 1e3:.2f} us"))
            mf = cmean("sq_core", "SQ_VALU_MFMA_BUSY_CYCLES")
            if mf is not None and gui:
                derived.append(("MFMA busy (MFMA_BUSY / (GUI_ACTIVE/8 * 1024 SIMDs))",
                                f"{100 * mf / (gui / 8 * 1024):.1f} %"))
            wc = cmean("sq_core", "SQ_WAVE_CYCLES")
            if wc is not None and gui:
                derived.append(("resident waves per CU (WAVE_CYCLES / (GUI_ACTIVE/8 * 256))",
                                f"{wc / (gui / 8 * 256):.2f}"))
            va = cmean("sq_stall", "SQ_ACTIVE_INST_VALU")
            g2 = cmean("sq_stall", "GRBM_GUI_ACTIVE")
            if va is not None and g2:
                derived.append(("VALU busy (ACTIVE_INST_VALU / (GUI_ACTIVE/8 * 256 CUs))",
                                f"{100 * va / (g2 / 8 * 256):.1f} %"))
            lb = cmean("sq_stall", "SQ_INSTS_LDS_LOAD_BANDWIDTH")
            if lb is not None and g2:
                derived.append(("LDS load bytes per CU per clock (LDS_LOAD_BANDWIDTH*64 / ...)",
                                f"{lb * 64 / (g2 / 8 * 256):.1f}"))
            bc = cmean("sq_stall", "SQ_LDS_BANK_CONFLICT")
            if bc is not None:
                derived.append(("LDS bank-conflict cycles", f"{bc:.0f}"))
            # LDS pass: indexed-access cycles (fragment reads; the copies' direct-to-LDS
            # writes are not indexed accesses), full command/data queues, the texture
            # address unit's busy cycles averaged over its instances
            g3 = cmean("lds", "GRBM_GUI_ACTIVE")
            if g3:
                cyc = g3 / 8 * 256
                for ctr, label in (("SQ_LDS_IDX_ACTIVE", "LDS busy, indexed accesses (LDS_IDX_ACTIVE / (GUI_ACTIVE/8 * 256 CUs))"),
                                   ("SQ_LDS_CMD_FIFO_FULL", "LDS command queue full (LDS_CMD_FIFO_FULL / (GUI_ACTIVE/8 * 256 CUs))"),
                                   ("SQ_LDS_DATA_FIFO_FULL", "LDS data queue full (LDS_DATA_FIFO_FULL / (GUI_ACTIVE/8 * 256 CUs))")):
                    v = cmean("lds", ctr)
                    if v is not None:
                        derived.append((label, f"{100 * v / cyc:.1f} %"))
                sb = cmean("lds", "SQ_INSTS_LDS_STORE_BANDWIDTH")
                if sb is not None:
                    derived.append(("LDS store bytes per CU per clock (LDS_STORE_BANDWIDTH*64 / ...)", f"{sb * 64 / cyc:.1f}"))
                ta = cmean("lds", "TA_BUSY_avr")
                if ta is not None:
                    derived.append(("texture address unit busy (TA_BUSY_avr / (GUI_ACTIVE/8))", f"{100 * ta / (g3 / 8):.1f} %"))
            fs, ws = cmean("fetch", "FETCH_SIZE"), cmean("write", "WRITE_SIZE")
            alg = None
            if kind == "headline":
                alg = bench["roofline"].get("algorithmic_bytes")
            elif kind == "secondary":
                alg = bench["secondary"][wname].get("algorithmic_bytes")
            if fs is not None and ws is not None and calib.get("FETCH_SIZE") and calib.get("WRITE_SIZE"):
                fb = fs * 1024 * calib["FETCH_SIZE"]
                wb = ws * 1024 * calib["WRITE_SIZE"]
                derived.append(("HBM bytes read (FETCH_SIZE KiB x 1024 x copy factor "
                                f"{calib['FETCH_SIZE']:.3f})", f"{fb / 1e6:.1f} MB"))
                derived.append(("HBM bytes written (WRITE_SIZE KiB x 1024 x copy factor "
                                f"{calib['WRITE_SIZE']:.3f})", f"{wb / 1e6:.1f} MB"))
                if alg:
                    derived.append(("traffic / algorithmic bytes", f"{(fb + wb) / alg:.2f} x ({alg / 1e6:.1f} MB)"))
                if kind in ("headline", "secondary"):
                    traffic[wname] = {"bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
                                      "write_bytes": int(round(wb)), "kernel": short_name(key[0])}
            if derived:
                lines.append("")
                lines.append("## derived (timed window)")
                for k_, v_ in derived:
                    lines.append(f"{k_}: {v_}")
        fname = os.path.join(args.out, f"{short_name(key[0])}__{wname}.txt")
        with open(fname, "w") as f:
            f.write("\n".join(lines) + "\n")
        say(f"wrote {fname}")
    if traffic and calib:
        from bench import kernel_source_hash
        with open(os.path.join(args.out, "hbm_traffic.json"), "w") as f:
            json.dump({"kernel_source_hash": kernel_source_hash(),
                       "calibration": {"copy_bytes": COPY_MIB << 20,
                                       "fetch_factor": calib.get("FETCH_SIZE"),
                                       "write_factor": calib.get("WRITE_SIZE")},
                       "command": " ".join(meta["bench_cmd"]), "workloads": traffic}, f, indent=1)
        say("wrote hbm_traffic.json")
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect")
    c.add_argument("--out", required=True)
    c.add_argument("--limit", type=int, default=240, help="seconds per rocprofv3 run")
    c.add_argument("bench_args", nargs=argparse.REMAINDER, help="bench.py arguments after --")
    s = sub.add_parser("summarize")
    s.add_argument("--in", dest="inp", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--window", type=int, default=20)
    args = ap.parse_args()
    if args.cmd == "collect":
        if args.bench_args and args.bench_args[0] == "--":
            args.bench_args = args.bench_args[1:]
        sys.exit(collect(args))
    sys.exit(summarize(args))


if __name__ == "__main__":
    main()
