#!/usr/bin/env python3
"""Throughput of the fine-grained-scaled FP8 E4M3 NT GEMM on one MI355X.

A step is one call of the GEMM on the prefill-like dense workload
(M=4096, N=7168, K=7168; seeded synthetic E4M3 data with per-1x128 / per-128x128
fp32 scales, BF16 out) with every input resident in HBM.  Prints ONE JSON line:
whole-job FP8 TFLOPS, the kernel's roofline position (achieved TFLOP/s from one
pair of HIP events around the timed steps on the launch stream, against the
5.0 PFLOP/s dense FP8 MFMA peak), the CPU oracle timed on a bounded sample of the
same workload, and -- under "secondary" -- the other workloads (small-M dense,
skewed contiguous MoE, masked decode, the two FP8 casts) each timed the same way,
HBM-bound ones with cold caches (every launch reads input copies that the
launches before it have evicted from L2 and the Infinity Cache).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 TFLOPS (% of MI355X FP8 MFMA peak); GB/s (% HBM) for masked decode"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
HEADLINE = "dense_m4096_n7168_k7168"
CU_CAPS = (224, 192, 128)       # CU caps the masked decode call is also timed under
KERNEL_SRC = os.path.join(ROOT, "fp8_block_scaled_e4m3_amd", "csrc", "dg_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_hash() -> str:
    """Hash of the library sources with comments and blank space removed, and of the
    code-generation flags, so that the stored traffic counters stay valid across comment
    edits and lapse on code or code-generation changes."""
    import re
    from fp8_block_scaled_e4m3_amd.build import CODEGEN_FLAGS
    h = hashlib.sha256()
    h.update(" ".join(CODEGEN_FLAGS).encode())
    for name in ("dg_gemm.hip", "dg_quant.hip", "dg_internal.h", "dg_api.cpp"):
        with open(os.path.join(ROOT, "fp8_block_scaled_e4m3_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def ceil_div(a, b):
    return -(-a // b)


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def upload(data: dict) -> dict:
    """The workload's arrays as GPU tensors (inputs resident in HBM before timing)."""
    import numpy as np
    import torch
    return {key: torch.from_numpy(np.ascontiguousarray(data[key])).to("cuda:0")
            for key in ("a", "sa", "b", "sb", "m_indices", "masked_m") if key in data}


def output_buffer(shape):
    """BF16 output (as int16 bits), pre-filled with the masked layout's sentinel."""
    import torch
    import workloads as W
    return torch.full(shape, W.SENTINEL_BF16, dtype=torch.int16, device="cuda:0")


def algorithmic(w, data):
    """(FLOPs, HBM bytes) that the method must do / move for one call: each input byte
    read once, each output element of a valid row written once (BF16)."""
    import numpy as np
    n, k = w.n, w.k
    kb, nb = ceil_div(k, 128), ceil_div(n, 128)
    if w.kind == "dense":
        m = w.m
        flops = 2 * m * n * k
        byts = m * k + n * k + 4 * m * kb + 4 * nb * kb + 2 * m * n
    elif w.kind == "contiguous":
        valid = int(sum(data["counts"]))
        mt, g = data["m_total"], data["groups"]
        flops = 2 * valid * n * k
        byts = mt * k + 4 * mt * kb + g * (n * k + 4 * nb * kb) + 4 * mt + 2 * valid * n
    else:
        mm = np.clip(data["masked_m"], 0, w.max_m)
        tot, active = int(mm.sum()), int((mm > 0).sum())
        flops = 2 * tot * n * k
        byts = active * (n * k + 4 * nb * kb) + tot * (k + 4 * kb + 2 * n) + 4 * w.groups
    return flops, byts


def make_call(w, dv, out):
    import fp8_block_scaled_e4m3_amd as dg
    if w.kind == "dense":
        return lambda: dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], out)
    if w.kind == "contiguous":
        return lambda: dg.dg_m_grouped_gemm_fp8_contiguous(dv["a"], dv["sa"], dv["b"], dv["sb"], out,
                                                           dv["m_indices"])
    return lambda: dg.dg_m_grouped_gemm_fp8_masked(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"])


def out_shape(w, data):
    if w.kind == "dense":
        return (w.m, w.n)
    if w.kind == "contiguous":
        return (data["m_total"], w.n)
    return (w.groups, w.max_m, w.n)


# Input copies an HBM-bound workload cycles through, so that every timed launch reads
# operands that are in neither the L2 (8 x 4 MB) nor the Infinity Cache (256 MB): each
# launch's inputs were last touched at least this many bytes of other inputs ago.
COLD_BYTES = 640 << 20


def input_sets(dv: dict, set_bytes: int, cold: bool) -> list:
    """[dv] for warm-cache timing; else dv plus enough device copies of it that cycling
    through them evicts each one from the caches before it is read again."""
    if not cold:
        return [dv]
    n = max(2, ceil_div(COLD_BYTES, max(set_bytes, 1)))
    return [dv] + [{k: v.clone() for k, v in dv.items()} for _ in range(n - 1)]


def run_timed(calls: list, warmup: int, steps: int, graph: bool = False):
    """`warmup` untimed launches, then `steps` launches back to back between one pair of
    HIP events recorded on the launch stream (no event between launches: event records
    there would idle the GPU for ~10 us each).  Launch i runs calls[i % len(calls)].
    graph=True captures the timed launches into one HIP graph first and times its
    replay: a kernel of ~10 us finishes faster than Python can issue the next call, so
    eagerly issued launches would time the host, not the GPU.
    Returns (mean seconds per launch from the events, wall seconds of the timed steps)."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)]()
    g = None
    if graph:
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                calls[(warmup + i) % len(calls)]()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            calls[(warmup + i) % len(calls)]()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3 / steps, wall


def traffic_for(workload: str):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration) if the committed counters were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = t.get("workloads", {}).get(workload)
    return None if entry is None else int(entry["bytes_per_launch"])


def cpu_baseline(w, data, target_s: float):
    """The oracle, as it stands, on a bounded row sample of the dense workload."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    cores = oracle.available_cores()
    a, sa, b, sb = data["a"], data["sa"], data["b"], data["sb"]
    # a call costs a fixed part (decoding B) plus a part per row: two probes (one and
    # two rows per thread) separate them, then the sample is sized to about target_s
    # (the whole workload when it fits), a whole number of rows per thread
    def probe_s(nrows):
        t0 = time.perf_counter()
        oracle.gemm_fp8_nt(a[:nrows], sa[:, :nrows], b, sb, nthreads=cores)
        return time.perf_counter() - t0
    p1 = min(cores, w.m)
    p2 = min(2 * p1, w.m)
    t1, t2 = probe_s(p1), probe_s(p2)
    per_row = max((t2 - t1) / max(p2 - p1, 1), t2 / p2 / 4, 1e-6)
    fixed = max(t1 - per_row * p1, 0.0)
    rows = int(min(w.m, max(p1, (target_s - fixed) / per_row)))
    if rows < w.m:
        rows = max(p1, rows - rows % cores)
    sel = np.linspace(0, w.m - 1, rows).astype(np.int64)
    t0 = time.perf_counter()
    oracle.gemm_fp8_nt(a[sel], sa[:, sel], b, sb, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = 2 * rows * w.n * w.k
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {w.m} rows (evenly spaced) x all {w.n} columns, K={w.k}; {dt:.1f} s fp64 C "
                      f"on {cores} host threads"}


CASTS = (("cast_1x128_m4096_k7168_f32", 4096, 7168, 1),
         ("cast_128x128_n7168_k7168_f32", 7168, 7168, 128))


def time_casts(warmup, iters):
    """The FP8 casts that feed the GEMM (fp32 in, E4M3 + scales out): HBM-bound, timed
    with cold caches (each launch reads an input copy not read recently)."""
    import torch

    import fp8_block_scaled_e4m3_amd as dg
    import workloads as W

    out = {}
    for cname, rows, k, gran in CASTS:
        say(f"bench: cast {cname}")
        x0 = torch.from_numpy(W.make_fp32_operand(rows, k, gran, seed=0)).to("cuda:0")
        xs = [t["x"] for t in input_sets({"x": x0}, rows * k * 4, True)]
        q = torch.empty((rows, k), dtype=torch.uint8, device="cuda:0")
        if gran == 1:
            s_ = torch.empty((k // 128, dg.dg_get_aligned_ld_sa(rows)), device="cuda:0")
            calls = [lambda x=x: dg.dg_quantize_fp8_1x128(x, q, s_) for x in xs]
            nsc = (k // 128) * rows
        else:
            s_ = torch.empty((ceil_div(rows, 128), k // 128), device="cuda:0")
            calls = [lambda x=x: dg.dg_quantize_fp8_128x128(x, q, s_) for x in xs]
            nsc = ceil_div(rows, 128) * (k // 128)
        b3 = rows * k * 4 + rows * k + 4 * nsc
        mean_s, _ = run_timed(calls, warmup, iters, graph=True)
        out[cname] = {"us": round(mean_s * 1e6, 2), "gbps": round(b3 / mean_s / 1e9, 1),
                      "frac_hbm": round(b3 / mean_s / 1e9 / PEAK_HBM_GBS, 4), "bound": "hbm",
                      "cold_caches": True, "input_copies": len(xs), "warmup": warmup, "steps": iters,
                      "launch": "hip graph replay",
                      "algorithmic_bytes": b3, "traffic": traffic_for(cname)}
        del x0, xs, q, s_, calls
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # From an idle GPU the chip's power management runs through a transient: a few fast
    # launches, a throttled stretch ~20-30% slower, then a slow return to the sustained
    # rate over ~50 ms.  The defaults time steps 6-25, inside that transient (what a
    # short run sees); --warmup 400 --steps 200 times the sustained state.
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--secondary-iters", type=int, default=20)
    ap.add_argument("--only-casts", action="store_true",
                    help="only time the two FP8 cast kernels (used for their profiles)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the GEMM library is single-GPU and runs no "
              "multi-GPU configuration; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_block_scaled_e4m3_amd as dg
    import workloads as W

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dg.load_library()
    if args.only_casts:
        print(json.dumps({"casts": time_casts(args.warmup, args.secondary_iters)}), flush=True)
        return
    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes, "launches": 5}))
        return
    w = W.WORKLOADS[args.workload]

    say(f"bench: generating {w.name}")
    data = W.make(w)
    dv = upload(data)
    out = output_buffer(out_shape(w, data))
    call = make_call(w, dv, out)
    flops, byts = algorithmic(w, data)
    plan = dg.dg_describe_launch({"dense": 0, "contiguous": 1, "masked": 2}[w.kind],
                                 w.m if w.kind == "dense" else (data.get("m_total") or w.max_m),
                                 w.n, w.k, w.groups)
    say(f"bench: plan {plan}; warmup {args.warmup}, timed steps {args.steps}")

    # ---- `warmup` untimed steps, then the timed region: exactly `steps` steps back to
    # back, synchronised on both sides, one HIP event pair around them on the launch stream
    launch_s, wall = run_timed([call], args.warmup, args.steps)
    ms_per_step = wall / args.steps * 1e3
    say(f"bench: {ms_per_step:.4f} ms/step wall, {launch_s * 1e6:.1f} us/launch (events over the timed region)")

    if w.kind == "masked":
        value, unit = byts / (ms_per_step / 1e3) / 1e9, "GB/s"
        achieved, peak, runit, bound = byts / launch_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        value, unit = flops / (ms_per_step / 1e3) / 1e12, "TFLOPS"
        achieved, peak, runit, bound = flops / launch_s / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s", "mfma"

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": w.kind, "m": w.m, "n": w.n, "k": w.k,
                   "block_m": plan["block_m"], "block_n": plan["block_n"], "tiles": plan["tiles"],
                   "grid": plan["grid"], "parallelism": "single-gpu"},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
                     "frac": round(achieved / peak, 4), "traffic": traffic_for(w.name),
                     "algorithmic_flops": flops, "algorithmic_bytes": byts,
                     "kernel": f"dg_gemm_kernel<{plan['block_m']},{plan['block_n']}>",
                     "launch_us": round(launch_s * 1e6, 2)},
    }
    del dv, out, call
    torch.cuda.empty_cache()

    if not args.no_secondary:
        # The other workloads, each after the same number of untimed launches as the
        # headline, timed as one HIP graph replay of their timed launches; HBM-bound ones
        # cycle through input copies so that every timed launch reads from HBM (cold L2
        # and Infinity Cache), MFMA-bound ones reuse one set.
        sec = {}
        for name, ww in W.WORKLOADS.items():
            if name == w.name or name.startswith("dense_m128"):
                continue
            say(f"bench: secondary {name}")
            d2 = W.make(ww)
            v2 = upload(d2)
            o2 = output_buffer(out_shape(ww, d2))
            f2, b2 = algorithmic(ww, d2)
            hbm_bound = f2 / b2 < PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
            sets = input_sets(v2, b2, hbm_bound)
            calls = [make_call(ww, v, o2) for v in sets]
            mean_s, _ = run_timed(calls, args.warmup, args.secondary_iters, graph=True)
            sec[name] = {"us": round(mean_s * 1e6, 2), "tflops": round(f2 / mean_s / 1e12, 2),
                         "gbps": round(b2 / mean_s / 1e9, 1),
                         "frac_mfma": round(f2 / mean_s / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "frac_hbm": round(b2 / mean_s / 1e9 / PEAK_HBM_GBS, 4),
                         "bound": "hbm" if hbm_bound else "mfma", "cold_caches": hbm_bound,
                         "input_copies": len(sets), "warmup": args.warmup, "steps": args.secondary_iters,
                         "launch": "hip graph replay",
                         "algorithmic_flops": f2, "algorithmic_bytes": b2,
                         "traffic": traffic_for(name)}
            if ww.kind == "masked":
                sec[name]["sum_masked_m"] = int(np.clip(d2["masked_m"], 0, ww.max_m).sum())
                # the decode GEMM sharing the GPU with a communication kernel: the same
                # call restricted to fewer CUs (dg_set_num_cus), the rest left free
                capped = {}
                for cap in CU_CAPS:
                    dg.dg_set_num_cus(cap)
                    try:
                        cs, _ = run_timed(calls, args.warmup, args.secondary_iters, graph=True)
                    finally:
                        dg.dg_set_num_cus(0)
                    capped[str(cap)] = {"us": round(cs * 1e6, 2), "gbps": round(b2 / cs / 1e9, 1)}
                sec[name]["cu_capped"] = capped
            del d2, v2, o2, sets, calls
            torch.cuda.empty_cache()
        sec.update(time_casts(args.warmup, args.secondary_iters))
        result["secondary"] = sec

    if not args.no_cpu_baseline and w.kind == "dense":
        say("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, data, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
