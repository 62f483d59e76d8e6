"""The measurement harness on the CPU: bench.py's refusals, and bench_profile.py's
summary of a synthetic rocprofv3 run (dispatch matching, counter means, the derived
clock and MFMA busy, the copy calibration and the traffic record bench.py reads)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HEADLINE = "void dg::dg_gemm_kernel<256, 256, 4, 2, 0, 16, 2, true, 0, 7168, 56>(dg::GemmParams, unsigned char const*)"
CAST = "void dg::(anonymous namespace)::quant_128x128_kernel<float, 0>(float const*, long, int, int)"


def _run(args, **kw):
    return subprocess.run([sys.executable, *args], cwd=ROOT, capture_output=True, text=True, timeout=300, **kw)


def test_bench_refuses_more_than_one_gpu():
    r = _run(["bench.py", "--gpus", "2"])
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr


def test_bench_fails_loudly_without_a_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this checks the CPU-only failure")
    r = _run(["bench.py", "--steps", "1", "--warmup", "0", "--no-secondary", "--no-cpu-baseline"])
    assert r.returncode != 0
    assert not r.stdout.strip().startswith("{"), "no JSON line may be printed without a GPU"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    keys = sorted({k for r in rows for k in r})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        w.writerows(rows)


def _trace_row(did, name, t0, dur_ns, grid_xyz, wg):
    return {"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t0 + dur_ns,
            "Grid_Size_X": grid_xyz[0], "Grid_Size_Y": grid_xyz[1], "Grid_Size_Z": grid_xyz[2],
            "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1}


def _counter_rows(did, name, t0, dur_ns, grid, wg, values):
    return [{"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": wg,
             "Counter_Name": k, "Counter_Value": v, "Start_Timestamp": t0, "End_Timestamp": t0 + dur_ns}
            for k, v in values.items()]


def _synthetic_run(d, n=25):
    """Headline: 131072 x 512, 200 us, 2.0 GHz, MFMA busy 50 %, 100000 KiB fetched and 50000 KiB
    written per dispatch.  Cast: a two-dimensional grid (14336 x 56) in the trace, the same
    802816 work-items as one number in the counters.  Copy calibration: 1 GiB copied reads
    as 524288 KiB fetched (factor 2) and 1048576 KiB written (factor 1).  LDS pass: 40 % indexed-busy,
    queues full 10 % and 5 % of the cycles, 20 store bytes per clock, texture unit 30 % busy."""
    with open(os.path.join(d, "meta.json"), "w") as f:
        json.dump({"bench_cmd": ["python3", "bench.py", "--gpus", "1", "--steps", "20", "--warmup", "5"]}, f)
    line = {"metric": "m", "config": {"workload": "dense_m4096_n7168_k7168"},
            "roofline": {"launch_us": 201.0, "algorithmic_bytes": 140390656},
            "secondary": {"cast_128x128_n7168_k7168_f32": {"us": 43.0, "algorithmic_bytes": 256913664}}}
    with open(os.path.join(d, "trace.log"), "w") as f:
        f.write("some log line\n" + json.dumps(line) + "\n")
    trace, did, t = [], 1, 1_000_000
    for _ in range(n):
        trace.append(_trace_row(did, HEADLINE, t, 200_000, (131072, 1, 1), 512))
        did, t = did + 1, t + 210_000
    for _ in range(n):
        trace.append(_trace_row(did, CAST, t, 42_000, (14336, 56, 1), 256))
        did, t = did + 1, t + 50_000
    _write_csv(os.path.join(d, "trace", "run_kernel_trace.csv"), trace)
    gui = 8 * 2.0 * 200_000                      # 2.0 GHz over 200 us, summed over 8 XCDs
    passes = {
        "sq_core": {"GRBM_GUI_ACTIVE": gui, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * gui / 8 * 1024},
        "sq_stall": {"GRBM_GUI_ACTIVE": gui, "SQ_ACTIVE_INST_VALU": 0.25 * gui / 8 * 256},
        "fetch": {"FETCH_SIZE": 100000.0},
        "write": {"WRITE_SIZE": 50000.0},
        "lds": {"GRBM_GUI_ACTIVE": gui, "SQ_LDS_IDX_ACTIVE": 0.4 * gui / 8 * 256,
                "SQ_LDS_CMD_FIFO_FULL": 0.1 * gui / 8 * 256, "SQ_LDS_DATA_FIFO_FULL": 0.05 * gui / 8 * 256,
                "SQ_INSTS_LDS_STORE_BANDWIDTH": 20.0 * gui / 8 * 256 / 64, "TA_BUSY_avr": 0.3 * gui / 8},
    }
    for pname, vals in passes.items():
        rows, did, t = [], 1, 1_000_000
        for _ in range(n):
            rows += _counter_rows(did, HEADLINE, t, 200_000, 131072, 512, vals)
            did, t = did + 1, t + 210_000
        for _ in range(n):
            rows += _counter_rows(did, CAST, t, 42_000, 802816, 256,
                                  {k: v / 10 for k, v in vals.items() if not k.startswith("GRBM")})
            did, t = did + 1, t + 50_000
        _write_csv(os.path.join(d, "pmc_" + pname, "run_counter_collection.csv"), rows)
    _write_csv(os.path.join(d, "copy_fetch", "run_counter_collection.csv"),
               _counter_rows(1, "copy_kernel", 0, 100, 1 << 20, 256, {"FETCH_SIZE": 524288.0}))
    _write_csv(os.path.join(d, "copy_write", "run_counter_collection.csv"),
               _counter_rows(1, "copy_kernel", 0, 100, 1 << 20, 256, {"WRITE_SIZE": 1048576.0}))


def test_profile_summary_of_a_synthetic_run(tmp_path):
    src, out = tmp_path / "prof", tmp_path / "profiles"
    src.mkdir()
    _synthetic_run(str(src))
    r = _run(["bench_profile.py", "summarize", "--in", str(src), "--out", str(out)])
    assert r.returncode == 0, r.stderr
    assert "warning" not in r.stderr
    head = (out / "dg_gemm_kernel_256x256x4x2x0x16x2x1x0x7168x56__dense_m4096_n7168_k7168.txt").read_text()
    assert "dispatches: 25" in head
    assert "timed window (last 20 dispatches): 200.00 us" in head
    assert "bench line of the traced run (one HIP event pair over its timed launches): 201.00 us" in head
    assert "clock (GRBM_GUI_ACTIVE / 8 / duration of the same dispatch): 2.000 GHz" in head
    assert "MFMA busy (MFMA_BUSY / (GUI_ACTIVE/8 * 1024 SIMDs)): 50.0 %" in head
    assert "VALU busy (ACTIVE_INST_VALU / (GUI_ACTIVE/8 * 256 CUs)): 25.0 %" in head
    # 100000 KiB x 1024 x 2 read, 50000 KiB x 1024 x 1 written
    assert "HBM bytes read (FETCH_SIZE KiB x 1024 x copy factor 2.000): 204.8 MB" in head
    assert "HBM bytes written (WRITE_SIZE KiB x 1024 x copy factor 1.000): 51.2 MB" in head
    cast = (out / "quant_128x128_kernel_0__cast_128x128_n7168_k7168_f32.txt").read_text()
    assert "grid: 802816 work-items, workgroup 256" in cast
    assert "HBM bytes read (FETCH_SIZE KiB x 1024 x copy factor 2.000): 20.5 MB" in cast
    assert "upper bound" not in head
    assert "LDS busy, indexed accesses (LDS_IDX_ACTIVE / (GUI_ACTIVE/8 * 256 CUs)): 40.0 %" in head
    assert "LDS command queue full (LDS_CMD_FIFO_FULL / (GUI_ACTIVE/8 * 256 CUs)): 10.0 %" in head
    assert "LDS data queue full (LDS_DATA_FIFO_FULL / (GUI_ACTIVE/8 * 256 CUs)): 5.0 %" in head
    assert "LDS store bytes per CU per clock (LDS_STORE_BANDWIDTH*64 / ...): 20.0" in head
    assert "texture address unit busy (TA_BUSY_avr / (GUI_ACTIVE/8)): 30.0 %" in head
    rec = json.loads((out / "hbm_traffic.json").read_text())
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["workloads"]["dense_m4096_n7168_k7168"]["bytes_per_launch"] == 100000 * 1024 * 2 + 50000 * 1024
    assert rec["workloads"]["cast_128x128_n7168_k7168_f32"]["bytes_per_launch"] == 10000 * 1024 * 2 + 5000 * 1024
    sys.path.insert(0, ROOT)
    import bench
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
