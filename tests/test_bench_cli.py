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
    with open(os.path.join(ROOT, "profiles", "bench.f32_4096.json")) as fh:
        line = json.loads(fh.read())
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["data"] == "synthetic"
    assert line["config"]["workload"] == "f32_4096"
    roof = line["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0


def test_vendor_comparison_is_opt_in():
    r = run_bench("--help")
    assert r.returncode == 0 and "--vendor" in r.stdout
    with open(os.path.join(ROOT, "profiles", "bench.f32_4096.json")) as fh:
        assert "vendor_blas" not in json.loads(fh.read())
