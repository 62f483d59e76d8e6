#!/usr/bin/env python3
"""Throughput of the fine-grained-scaled FP8 E4M3 NT GEMM on one MI355X.

A step is one call of the GEMM on the prefill-like dense workload
(M=4096, N=7168, K=7168; seeded synthetic E4M3 data with per-1x128 / per-128x128
fp32 scales, BF16 out) with every input resident in HBM.  Prints ONE JSON line:
whole-job FP8 TFLOPS, the kernel's roofline position (achieved TFLOP/s from HIP
events around each launch on the launch stream, against the 5.0 PFLOP/s dense
FP8 MFMA peak), the CPU oracle timed on a bounded sample of the same workload,
and -- under "secondary" -- the other workloads (small-M dense, skewed
contiguous MoE, masked decode) each timed the same way, HBM-bound ones with the
caches flushed between launches.
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
    """Hash of the library sources with comments and blank space removed, so that the
    stored traffic counters stay valid across comment edits and lapse on code edits."""
    import re
    h = hashlib.sha256()
    for name in ("dg_gemm.hip", "dg_quant.hip", "dg_internal.h", "dg_api.cpp"):
        with open(os.path.join(ROOT, "fp8_block_scaled_e4m3_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def ceil_div(a, b):
    return -(-a // b)


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


def warm_up(call, seconds: float = 0.06, cap: int = 400) -> None:
    """Run `call` back to back for about `seconds` of GPU time (at least 3 times), so the
    timed launches that follow see the power management settled (see --warmup)."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    call()
    e.record()
    torch.cuda.synchronize()
    one = max(s.elapsed_time(e) / 1e3, 1e-6)
    for _ in range(max(3, min(cap, int(seconds / one)))):
        call()
    torch.cuda.synchronize()


def time_launches(call, iters, flush=None):
    """Mean kernel time (s) from HIP events recorded around each launch on the
    stream the kernel is launched on (torch's current stream)."""
    import torch
    stream = torch.cuda.current_stream()
    pairs = []
    for _ in range(iters):
        if flush is not None:
            # evict L2 and the Infinity Cache by reading 512 MB: a read leaves the
            # caches clean, so the timed kernel pays for no write-back of the flush
            flush.amax()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        call()
        e.record(stream)
        pairs.append((s, e))
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in pairs]
    return sum(ms) / len(ms) / 1e3, min(ms) / 1e3


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
    probe = 8
    t0 = time.perf_counter()
    oracle.gemm_fp8_nt(a[:probe], sa[:, :probe], b, sb, nthreads=cores)
    dt = max(time.perf_counter() - t0, 1e-3)
    rows = int(min(w.m, max(cores, probe * target_s / dt)))
    rows = max(cores, rows - rows % cores)
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


def time_casts(iters, flush):
    """The FP8 casts that feed the GEMM (fp32 in, E4M3 + scales out): HBM-bound."""
    import torch

    import fp8_block_scaled_e4m3_amd as dg
    import workloads as W
    from tests.gpu_support import say

    out = {}
    for cname, rows, k, gran in CASTS:
        say(f"bench: cast {cname}")
        x = torch.from_numpy(W.make_fp32_operand(rows, k, gran, seed=0)).to("cuda:0")
        q = torch.empty((rows, k), dtype=torch.uint8, device="cuda:0")
        if gran == 1:
            s_ = torch.empty((k // 128, W.ld_sa_for(rows)), device="cuda:0")
            c3 = lambda: dg.dg_quantize_fp8_1x128(x, q, s_)
            nsc = (k // 128) * rows
        else:
            s_ = torch.empty((ceil_div(rows, 128), k // 128), device="cuda:0")
            c3 = lambda: dg.dg_quantize_fp8_128x128(x, q, s_)
            nsc = ceil_div(rows, 128) * (k // 128)
        b3 = rows * k * 4 + rows * k + 4 * nsc
        for _ in range(3):      # HBM-bound and timed with cold caches: a short warm-up
            c3()
        mean_s, _ = time_launches(c3, iters, flush)
        out[cname] = {"us": round(mean_s * 1e6, 2), "gbps": round(b3 / mean_s / 1e9, 1),
                      "frac_hbm": round(b3 / mean_s / 1e9 / PEAK_HBM_GBS, 4), "bound": "hbm",
                      "caches_flushed": True, "algorithmic_bytes": b3, "traffic": traffic_for(cname)}
        del x, q, s_, c3
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # Under a sustained FP8 load the chip's power management runs through a transient for
    # its first ~30 ms (per-launch time up 20-30%, then back down) before it settles; 400
    # warm-up steps (~70 ms for the headline GEMM) put the timed steps in the settled state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
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
    from tests.gpu_support import say, sentinel_like, upload

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dg.load_library()
    if args.only_casts:
        flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
        print(json.dumps({"casts": time_casts(args.secondary_iters, flush)}), flush=True)
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
    out = sentinel_like(out_shape(w, data))
    call = make_call(w, dv, out)
    flops, byts = algorithmic(w, data)
    plan = dg.dg_describe_launch({"dense": 0, "contiguous": 1, "masked": 2}[w.kind],
                                 w.m if w.kind == "dense" else (data.get("m_total") or w.max_m),
                                 w.n, w.k, w.groups)
    say(f"bench: plan {plan}; warmup {args.warmup}, timed steps {args.steps}")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronised on both sides ----
    stream = torch.cuda.current_stream()
    pairs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        call()
        e.record(stream)
        pairs.append((s, e))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_s = sum(s.elapsed_time(e) for s, e in pairs) / len(pairs) / 1e3
    ms_per_step = wall / args.steps * 1e3
    say(f"bench: {ms_per_step:.4f} ms/step wall, {launch_s * 1e6:.1f} us/launch (events)")

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
        sec = {}
        flush = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
        for name, ww in W.WORKLOADS.items():
            if name == w.name or name.startswith("dense_m128"):
                continue
            say(f"bench: secondary {name}")
            d2 = W.make(ww)
            v2 = upload(d2)
            o2 = sentinel_like(out_shape(ww, d2))
            c2 = make_call(ww, v2, o2)
            f2, b2 = algorithmic(ww, d2)
            warm_up(c2)
            hbm_bound = f2 / b2 < PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
            mean_s, best_s = time_launches(c2, args.secondary_iters, flush if hbm_bound else None)
            sec[name] = {"us": round(mean_s * 1e6, 2), "tflops": round(f2 / mean_s / 1e12, 2),
                         "gbps": round(b2 / mean_s / 1e9, 1),
                         "frac_mfma": round(f2 / mean_s / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "frac_hbm": round(b2 / mean_s / 1e9 / PEAK_HBM_GBS, 4),
                         "bound": "hbm" if hbm_bound else "mfma", "caches_flushed": hbm_bound,
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
                        c2()
                        cs, _ = time_launches(c2, args.secondary_iters, flush)
                    finally:
                        dg.dg_set_num_cus(0)
                    capped[str(cap)] = {"us": round(cs * 1e6, 2), "gbps": round(b2 / cs / 1e9, 1)}
                sec[name]["cu_capped"] = capped
            del d2, v2, o2, c2
            torch.cuda.empty_cache()
        sec.update(time_casts(args.secondary_iters, flush))
        result["secondary"] = sec

    if not args.no_cpu_baseline and w.kind == "dense":
        say("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, data, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
