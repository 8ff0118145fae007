"""Host logic of bench.py (no GPU): the one-GPU refusal, the warm-up count, the
per-step statistics, the roofline bookkeeping and the traffic lookup."""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import seeded_inputs as si  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


class FakeEvent:
    """Stands in for torch.cuda.Event: elapsed times come from a fixed list."""
    clock = 0.0
    times = []

    def __init__(self, enable_timing=True):
        self.t = None

    def record(self):
        self.t = FakeEvent.clock

    def elapsed_time(self, other):
        return other.t - self.t

    def query(self):
        return True


def fake_torch():
    cuda = types.SimpleNamespace(Event=FakeEvent, synchronize=lambda: None)
    return types.SimpleNamespace(cuda=cuda)


def test_warm_up_runs_exactly_w_steps():
    calls = []
    args = types.SimpleNamespace(warmup=7)
    assert bench.warm_up(lambda: calls.append(1), args, fake_torch()) == 7
    assert len(calls) == 7


def test_warm_up_default_count():
    calls = []
    n = bench.warm_up(lambda: calls.append(1), types.SimpleNamespace(warmup=None), fake_torch())
    assert n == len(calls) == bench.DEFAULT_WARMUP


def test_clock_warm_fills_the_time():
    calls = []
    n = bench.clock_warm(lambda: calls.append(1), fake_torch(), seconds=0.02)
    assert n == len(calls) and n >= 10 and n % 10 == 0


def test_clock_from_two_samples():
    """Per XCC the median of the workgroups' cycles / seconds; workgroups that ran
    on another XCC in the second sample are left out; the mean over XCCs."""
    n = 16
    before = np.zeros((n, 4), dtype=np.uint64)
    after = np.zeros((n, 4), dtype=np.uint64)
    for i in range(n):
        x = i % 8
        ghz = 2.0 + 0.01 * x
        before[i] = (1_000_000 + 7 * i, 5_000 + i, x, 0)
        ticks = 10_000  # 100 us at 100 MHz
        after[i] = (before[i][0] + int(ghz * 1e9 * 1e-4), before[i][1] + ticks, x, 0)
    after[3][2] = 5  # moved: not used
    c = bench.clock_ghz(before, after)
    assert c["per_xcc"]["0"] == pytest.approx(2.0)
    assert c["per_xcc"]["7"] == pytest.approx(2.07)
    assert c["mean"] == pytest.approx(2.035, abs=1e-4)
    assert c["interval_s"] == pytest.approx(1e-4)
    assert bench.clock_ghz(before[:0], after[:0]) is None


def _fake_results(B, H, G, S, D, rng):
    refs = []
    for b in range(B):
        for h in range(H):
            refs.append(((b, h), {n: rng.standard_normal((S, D)) if n != "lse" else rng.standard_normal(S)
                                  for n in bench.OUTPUTS}))
    return refs


def test_receipt_passes_and_fails_at_the_bar():
    rng = np.random.default_rng(1)
    B, H, G, S, D = 2, 4, 2, 5, 3
    refs = _fake_results(B, H, G, S, D, rng)
    full = {n: np.zeros((B, H if n in ("o", "lse", "dq") else H // G) + ((S, D) if n != "lse" else (S,)))
            for n in bench.OUTPUTS}
    for (b, h), r in refs:
        for n in ("o", "lse", "dq"):
            full[n][b, h] = r[n]
        for n in ("dk", "dv"):
            full[n][b, h // G] += r[n]  # a key/value head's gradient sums its group
    gpu = {n: (lambda a: (lambda b, h: a[b, h]))(a) for n, a in full.items()}
    rec = bench.compare_heads(gpu, refs, "bf16", G)
    assert rec["status"] == "PASS" and rec["heads"] == B * H and rec["kv_heads"] == B * H // G
    full["dv"][1, 1, 2, 0] += 0.019
    assert bench.compare_heads(gpu, refs, "bf16", G)["status"] == "PASS"
    full["dv"][1, 1, 2, 0] += 0.002  # 0.021 > 2e-2
    rec = bench.compare_heads(gpu, refs, "bf16", G)
    assert rec["status"] == "FAIL" and rec["max_err"]["dv"] == pytest.approx(0.021, rel=1e-2)
    assert bench.compare_heads(gpu, refs, "f16", G)["status"] == "FAIL"
    # a partial group: dK/dV are not compared (their sums need every query head)
    rec = bench.compare_heads(gpu, refs[:1], "bf16", G)
    assert rec["kv_heads"] == 0 and "dv" not in rec["max_err"] and rec["status"] == "PASS"
    # fp32: relative to the tensor's largest magnitude
    full["dv"][1, 1, 2, 0] -= 0.021
    full["o"][0, 0, 0, 0] += 1e-5 * np.abs(np.concatenate([r["o"].ravel() for _, r in refs])).max()
    assert bench.compare_heads(gpu, refs, "f32", G)["status"] == "PASS"
    full["o"][0, 0, 0, 0] += 2e-4 * np.abs(np.concatenate([r["o"].ravel() for _, r in refs])).max()
    assert bench.compare_heads(gpu, refs, "f32", G)["status"] == "FAIL"
    assert bench.compare_heads(gpu, [], "bf16", G)["status"] == "FAIL"  # no sample, no receipt


def test_step_statistics():
    durations = iter([1.0, 2.0, 3.0, 4.0, 100.0])

    def step():
        FakeEvent.clock += next(durations)

    st = bench.step_statistics(step, 5, fake_torch())
    assert st["n"] == 5 and st["median"] == 3.0 and st["min"] == 1.0
    assert st["p95"] == pytest.approx(np.percentile([1, 2, 3, 4, 100], 95), abs=1e-5)
    lo, hi = st["ci95_median"]
    assert 1.0 <= lo <= 3.0 <= hi <= 100.0
    # `between` runs after each step, outside its event pair
    FakeEvent.clock = 0.0
    durations = iter([1.0] * 4)
    st = bench.step_statistics(step, 4, fake_torch(), between=lambda: setattr(FakeEvent, "clock", FakeEvent.clock + 50))
    assert st["median"] == 1.0 and st["min"] == 1.0


def test_kernel_units_add_up_to_the_metric():
    """fwd 2 units + dQ 1 + dK/dV 4 = 7 B H S^2 D (the split backward's recomputed
    products are not algorithmic)."""
    w = si.WORKLOADS["gpt205m_bf16"]
    u = bench.kernel_units(w)
    assert u["fwd"]["flops"] + u["bwd_dq"]["flops"] + u["bwd_dkdv"]["flops"] == pytest.approx(w.flops)
    assert u["bwd"]["flops"] == pytest.approx(u["bwd_dq"]["flops"] + u["bwd_dkdv"]["flops"])
    assert u["fwd"]["flops"] == pytest.approx(2 * w.flops / 7)


def test_traffic_lookup_needs_matching_sources():
    """A recorded traffic figure is used only while its kernel's sources hash to
    the recorded value."""
    for kernel in ("fwd", "bwd_dq", "bwd_dkdv"):
        got = bench.read_traffic(kernel, "gpt205m_bf16")
        with open(bench.TRAFFIC_FILE) as f:
            rec = [ln.split() for ln in f if ln.startswith(kernel + " gpt205m_bf16 ")]
        if rec and rec[0][2] == bench.kernel_sources_hash(kernel):
            assert got == float(rec[0][3]) + float(rec[0][4])
        else:
            assert got is None
    assert bench.read_traffic("fwd", "no_such_workload") is None


def test_receipt_of_output_pairs():
    """The decode / fp8 receipt: absolute bar for 16-bit types, relative for fp32, and
    a non-finite error fails."""
    ok = bench.receipt_of({"o": 0.019, "lse": 0.001}, {"o": 3.0, "lse": 10.0}, "bf16", "x")
    assert ok["status"] == "PASS" and ok["max_err"] == {"o": 0.019, "lse": 0.001}
    assert bench.receipt_of({"o": 0.021, "lse": 0.0}, {"o": 3.0, "lse": 1.0}, "bf16", "x")["status"] == "FAIL"
    assert bench.receipt_of({"o": 0.004, "lse": 0.0}, {"o": 3.0, "lse": 1.0}, "f16", "x")["status"] == "PASS"
    assert bench.receipt_of({"o": 0.006, "lse": 0.0}, {"o": 3.0, "lse": 1.0}, "f16", "x")["status"] == "FAIL"
    # fp32: relative to max |oracle|
    assert bench.receipt_of({"o": 2e-4, "lse": 0.0}, {"o": 10.0, "lse": 1.0}, "f32", "x")["status"] == "PASS"
    assert bench.receipt_of({"o": 2e-3, "lse": 0.0}, {"o": 10.0, "lse": 1.0}, "f32", "x")["status"] == "FAIL"
    assert bench.receipt_of({"o": float("nan"), "lse": 0.0}, {"o": 1.0, "lse": 1.0}, "bf16", "x")["status"] == "FAIL"
