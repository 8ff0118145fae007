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
    # this grid's backward runs as one launch (dQ and dK/dV blocks side by side)
    assert set(d["kernel_ms"]) == {"fwd", "bwd"}
    st = d["step_ms_bwd_first"]
    assert st["n"] == 5 and st["min"] <= st["median"] <= st["p95"]
    assert 0.3 < d["clock_ghz"]["mean"] < 3.0, d["clock_ghz"]
    assert d["clock_warm"]["steps"] >= 10
    rf = d["roofline"]
    assert rf["peak_at_clock"] > 0 and abs(rf["frac_at_clock"] - rf["achieved"] / rf["peak_at_clock"]) < 1e-3
    # the second, fresh session reproduced this session's outputs bit for bit
    assert len(d["sessions"]) == 2 and d["sessions"][1]["receipt"] == "PASS", d["sessions"]


def test_bench_headline_passes_timed_apart():
    """At the headline workload attn_bwd runs the dQ and dK/dV passes one after the
    other, and the bench times each (the roofline's dominant kernel is one of them)."""
    d = run_bench("--workload", "gpt205m_bf16", "--sessions", "1")
    check_common(d, "gpt205m_bf16")
    assert set(d["kernel_ms"]) == {"fwd", "bwd_dq", "bwd_dkdv"}
    assert d["roofline"]["kernel"] in d["kernel_ms"]


def test_bench_receipt_against_the_oracle():
    """With the CPU baseline on, the session's outputs pass the oracle check on the
    heads the baseline ran (the tiny fp32 workload: every head)."""
    print("\n[bench] --workload tiny_f32 with the receipt", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--workload", "tiny_f32", "--cpu-seconds", "2", "--sessions", "1"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][0])
    rc = d["receipt"]
    assert rc["status"] == "PASS" and rc["heads"] == 4 and rc["kv_heads"] == 4, rc
    assert max(rc["max_err"].values()) <= 1e-4
    assert d["cpu_baseline"]["host_cores"] >= 1 and d["cpu_baseline"]["cores"] >= 1


def test_bench_decode():
    d = run_bench("--workload", "decode_gpt205m_bf16")
    check_common(d, "decode_gpt205m_bf16")
    assert d["roofline"]["bound"] == "hbm"


def test_bench_fp8qk():
    d = run_bench("--workload", "gpt205m_fp8qk")
    check_common(d, "gpt205m_fp8qk")


@pytest.mark.parametrize("workload", ["decode_gpt205m_bf16", "gpt205m_fp8qk"])
def test_bench_receipt_and_clock_other_modes(workload):
    """The decode and fp8-QK modes check their first step against the oracle heads
    the CPU baseline computes (a PASS receipt before any timing) and report the
    shader clock over the timed region."""
    print(f"\n[bench] --workload {workload} with the receipt", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--workload", workload, "--cpu-seconds", "2"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
    check_common(d, workload)
    rc = d["receipt"]
    assert rc["status"] == "PASS" and set(rc["max_err"]) == {"o", "lse"}, rc
    assert 0.3 < d["clock_ghz"]["mean"] < 3.0, d["clock_ghz"]
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["host_cores"] >= 1
