"""bench.py end to end on the GPU, in a subprocess, at small workloads: one JSON
line with the fields the measurement contract names, a roofline below 100% of
peak, and the per-step statistics."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline"}


def run_bench(*args):
    print(f"\n[bench] {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--no-cpu-baseline", "--steps", "5",
                        "--warmup", "2", *args], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_common(d, workload):
    assert KEYS <= set(d), sorted(KEYS - set(d))
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == workload
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu")
    assert 0 < rf["achieved"] and 0 < rf["frac"] <= 1.0, rf
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_bench_training_step():
    d = run_bench("--workload", "gpt12m_bf16")
    check_common(d, "gpt12m_bf16")
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16"
    for k in ("step_ms", "step_ms_cache_cold"):
        st = d[k]
        assert st["n"] == 5 and st["min"] <= st["median"] <= st["p95"]
        assert st["ci95_median"][0] <= st["median"] <= st["ci95_median"][1]
    assert set(d["kernel_ms"]) == {"fwd", "bwd_dq", "bwd_dkdv"}


def test_bench_decode():
    d = run_bench("--workload", "decode_gpt205m_bf16")
    check_common(d, "decode_gpt205m_bf16")
    assert d["roofline"]["bound"] == "hbm"


def test_bench_fp8qk():
    d = run_bench("--workload", "gpt205m_fp8qk")
    check_common(d, "gpt205m_fp8qk")
