"""bench.py's command-line contract that needs no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = run_bench(env=env)
    assert r.returncode == 2
    assert "WORLD_SIZE=4" in r.stderr


def test_committed_default_bench_line_keeps_the_contract():
    with open(os.path.join(ROOT, "profiles", "bench.bf16_8192.json")) as fh:
        line = json.loads(fh.read())
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["data"] == "synthetic"
    assert line["config"]["workload"] == "bf16_8192"
    roof = line["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0


def test_vendor_comparison_is_opt_in():
    r = run_bench("--help")
    assert r.returncode == 0 and "--vendor" in r.stdout
    with open(os.path.join(ROOT, "profiles", "bench.bf16_8192.json")) as fh:
        assert "vendor_blas" not in json.loads(fh.read())


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_takes_the_timed_dispatches(tmp_path):
    """--summarize-trace averages dispatches warmup .. warmup+steps-1 of each
    kernel of the call (in start order), not the warm-up ones."""
    name = "void tdm::(anonymous namespace)::skinny_bf16_kernel(...)"
    red = "void tdm::(anonymous namespace)::skinny_reduce_kernel(...)"
    rows, t = [], 0
    for i in range(8):  # 3 warm-up calls at 100 us, then 5 timed at 20 us
        dur = 100_000 if i < 3 else 20_000
        rows.append([i * 2, name, t, t + dur])
        rows.append([i * 2 + 1, red, t + dur, t + dur + 3_000])
        t += dur + 10_000
    _write_csv(str(tmp_path / "host" / "1_run_kernel_trace.csv"),
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    line = tmp_path / "line.json"
    line.write_text(json.dumps({"ms_per_step": 0.025, "value": 1.0, "unit": "TFLOP/s",
                                "roofline": {"achieved": 5000, "unit": "GB/s", "peak": 8000,
                                             "frac": 0.625}}) + "\n")
    r = run_bench("--summarize-trace", str(tmp_path), "--workload", "bf16_skinny", "--steps", "5",
                  "--warmup", "3", "--bench-line", str(line))
    assert r.returncode == 0, r.stderr
    assert "| skinny_bf16_kernel | 8 | 50.0 | 5 | 20.0 |" in r.stdout
    assert "| skinny_reduce_kernel | 8 | 3.0 | 5 | 3.0 |" in r.stdout
    assert "Timed kernel time per step 23.0 us = 0.920 of the step" in r.stdout


def test_trace_summary_skips_the_prewarm_calls(tmp_path):
    """The calls the run made before its warm-up (config.prewarm_calls in its
    line) are skipped too: 4 pre-warm calls at 300 us, 2 warm-up at 100 us,
    then 3 timed at 40 us."""
    name = "void tdm::(anonymous namespace)::mfma_bf16_kernel<...>(...)"
    rows, t = [], 0
    for i in range(9):
        dur = 300_000 if i < 4 else 100_000 if i < 6 else 40_000
        rows.append([i, name, t, t + dur])
        t += dur + 5_000
    _write_csv(str(tmp_path / "host" / "1_run_kernel_trace.csv"),
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    line = tmp_path / "line.json"
    line.write_text(json.dumps({"ms_per_step": 0.041, "value": 1.0, "unit": "TFLOP/s",
                                "config": {"prewarm_calls": 4},
                                "roofline": {"achieved": 1.0, "unit": "TFLOP/s", "peak": 2516.6,
                                             "frac": 0.0004}}) + "\n")
    r = run_bench("--summarize-trace", str(tmp_path), "--workload", "bf16_8192", "--steps", "3",
                  "--warmup", "2", "--bench-line", str(line))
    assert r.returncode == 0, r.stderr
    assert "| mfma_bf16_kernel | 9 | " in r.stdout and "| 3 | 40.0 | 40.0 | 40.0 | 40.0 |" in r.stdout


def test_prewarm_option_is_documented():
    r = run_bench("--help")
    assert r.returncode == 0 and "--prewarm-s" in r.stdout


def test_counter_summary_normalizes_to_the_measured_clock(tmp_path):
    name = "void tdm::(anonymous namespace)::mfma_bf16_kernel<...>(...)"
    rows = []
    for d in range(2):  # 1000 us at 1.5 GHz: 8 XCDs x 1.5e6 cycles
        for c, v in (("GRBM_GUI_ACTIVE", 12e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1.2e6)):
            rows.append([d, name, c, v / 2, 0, 1_000_000])
            rows.append([d, name, c, v / 2, 0, 1_000_000])  # two rows per dispatch, summed
    _write_csv(str(tmp_path / "p" / "run_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                "Start_Timestamp", "End_Timestamp"], rows)
    r = run_bench("--summarize-counters", str(tmp_path / "p"), "--workload", "bf16_8192")
    assert r.returncode == 0, r.stderr
    assert "| engine clock from GRBM_GUI_ACTIVE (GHz) | 1.500 |" in r.stdout
    assert "| MFMA busy / SIMD cycles at the measured clock | 0.800 |" in r.stdout


def test_counter_summary_rates_short_dispatches_at_the_peak_clock(tmp_path):
    """A 20 us dispatch: its counter window is longer than the dispatch, so no
    clock is derived and the rates use 2.4 GHz over the duration."""
    name = "void tdm::(anonymous namespace)::skinny_nk_bf16_kernel(...)"
    rows = [[0, name, "GRBM_GUI_ACTIVE", 8 * 60e3, 0, 20_000],
            [0, name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 4.8e3, 0, 20_000]]
    _write_csv(str(tmp_path / "p" / "run_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                "Start_Timestamp", "End_Timestamp"], rows)
    r = run_bench("--summarize-counters", str(tmp_path / "p"), "--workload", "bf16_skinny_nk")
    assert r.returncode == 0, r.stderr
    assert "engine clock" not in r.stdout
    assert "| MFMA busy / SIMD cycles at 2.4 GHz over the dispatch (too short to measure " \
           "the clock) | 0.100 |" in r.stdout


def test_traffic_record_from_byte_counters(tmp_path):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch, from two runs) scaled by
    the copy calibration give the record bench.py reads as roofline.traffic."""
    name = "void tdm::(anonymous namespace)::mfma_bf16_kernel<...>(...)"
    for c, v in (("FETCH_SIZE", 1000.0), ("WRITE_SIZE", 300.0)):
        _write_csv(str(tmp_path / c / "run_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"],
                   [[d, name, c, v, 0, 500_000] for d in range(3)])
    out = tmp_path / "t.json"
    r = run_bench("--summarize-counters", str(tmp_path / "FETCH_SIZE"),
                  str(tmp_path / "WRITE_SIZE"), "--workload", "bf16_8192", "--fetch-scale", "2.0",
                  "--write-scale", "1.0", "--traffic-json", str(out))
    assert r.returncode == 0, r.stderr
    rec = json.loads(out.read_text())
    assert rec["kernel"] == "mfma_bf16_kernel" and rec["workload"] == "bf16_8192"
    assert rec["hbm_bytes_per_launch"] == (1000.0 * 2.0 + 300.0) * 1024
    assert rec["source"] == "gemm_mfma_bf16.hip" and len(rec["source_sha"]) == 16


def test_power_sampler_reads_socket_power_and_the_first_engine_clock(monkeypatch):
    """--sample-power parses amd-smi's socket power and the first GFX clock
    (not MIN_CLK / MAX_CLK) and reports medians over its samples."""
    sys.path.insert(0, ROOT)
    import bench

    out = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1401 W\n    CLOCK:\n        GFX_0:\n"
           "            CLK: 1687 MHz\n            MIN_CLK: 500 MHz\n            MAX_CLK: 2400 MHz\n"
           "        GFX_1:\n            CLK: 1690 MHz\n")

    class R:
        stdout = out

    monkeypatch.setattr(subprocess, "run", lambda *a, **k: R())
    p = bench.PowerSampler(interval_s=0.01)
    assert p._one() == (1401.0, 1687.0)
    p.samples = [(1400.0, 1690.0), (1390.0, 1700.0), (1401.0, 1680.0)]
    s = p.summary()
    assert s["samples"] == 3 and s["socket_w_median"] == 1400.0 and s["sclk_mhz_median"] == 1690.0
    assert s["socket_w_min"] == 1390.0 and s["sclk_mhz_max"] == 1700.0
