"""Forward + backward causal attention throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = attn_fwd + attn_bwd (dQ pass that also forms delta, dK/dV pass) over one
batch of synthetic inputs already resident in HBM.  Prints ONE JSON line:
forward+backward TFLOP/s under the 7*B*H*S^2*D causal convention, the roofline
of the dominant kernel (algorithmic FLOPs / its average HIP-event duration over a
timed pass), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.

Protocol (Iron "Kernel Engineering Guide", §6.1-6.2): a PASS receipt first (the
session's own outputs at the timed shape against the oracle that the CPU
baseline runs, on the heads it covers; a mismatch exits with status 3); the
clock warmed by CLOCK_WARM_SECONDS of untimed steps before the W warm-up steps;
the shader clock measured over the timed region and reported with the peak at
that clock; a file lock around the timed sections; both dispatch orders; and a
second, fresh session (a child process, run after this one's timed sections)
whose outputs must be bitwise equal to this session's.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import seeded_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA: twice the bf16 rate
# The fp8-QK forward runs half its FLOPs (Q K^T) at the fp8 rate and half (P V) at
# the bf16 rate: its MFMA-time bound is the harmonic combination of the two.
PEAK_FP8QK_FWD_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")
TIMES_FILE = os.path.join(ROOT, "profiles", "kernel_times.txt")
# Untimed steps before the warm-up: a cold GPU runs at a lower DVFS clock state
# (after 10 steps of the headline workload the clock had not settled: ~15% lower
# throughput than after 0.3 s of steps).
CLOCK_WARM_SECONDS = 0.3
DEFAULT_WARMUP = 20
CU_COUNT = 256
BF16_FLOP_PER_CLK_CU = 4096  # dense bf16 / fp16 MFMA: 2516.6 TFLOP/s at 2.4 GHz
LOCK_FILE = os.path.join(os.environ.get("TMPDIR", "/tmp"), "causal_attn_bench.lock")
OUTPUTS = ("o", "lse", "dq", "dk", "dv")
# Parity bars of the receipt (the same as the GPU parity tests): bf16 inputs
# max |gpu - oracle| <= 2e-2; fp16 5e-3 (three more fraction bits than bf16);
# fp32 max |gpu - oracle| / max |oracle| <= 1e-4 per tensor.
RECEIPT_TOL = {"bf16": ("abs", 2e-2), "f16": ("abs", 5e-3), "f32": ("rel", 1e-4)}


METRIC_TRAIN = "causal attention fwd+bwd TFLOP/s (bf16) on 1 GPU; % of MFMA peak"


def host_cores() -> int:
    """CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def blas_threads() -> int:
    """Threads the host BLAS (numpy's matmul, which the oracle uses) runs with."""
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return host_cores()


class GpuLock:
    """An exclusive file lock around the timed sections, so that two invocations
    on one machine never time against each other."""

    def __enter__(self):
        import fcntl
        self.f = open(LOCK_FILE, "w")
        fcntl.flock(self.f, fcntl.LOCK_EX)
        return self

    def __exit__(self, *exc):
        import fcntl
        fcntl.flock(self.f, fcntl.LOCK_UN)
        self.f.close()
        return False


def clock_ghz(before, after):
    """Average shader clock (GHz) over the interval between two clock samples
    (arrays of [n, 4] uint64 from attn_clock_sample: cycles, 100 MHz ticks, XCC
    id, 0), from the workgroups that ran on the same XCC in both samples: per XCC
    the median of the per-workgroup estimates, then the mean over XCCs."""
    b = np.asarray(before, dtype=np.float64)
    a = np.asarray(after, dtype=np.float64)
    same = b[:, 2] == a[:, 2]
    dt = (a[:, 1] - b[:, 1]) / 100e6
    ok = same & (dt > 0)
    if not ok.any():
        return None
    est = (a[:, 0] - b[:, 0])[ok] / dt[ok] / 1e9
    xcc = b[ok, 2]
    per = {int(x): float(np.median(est[xcc == x])) for x in np.unique(xcc)}
    return {"mean": round(float(np.mean(list(per.values()))), 4),
            "per_xcc": {str(k): round(v, 4) for k, v in sorted(per.items())},
            "interval_s": round(float(np.median(dt[ok])), 6)}


class ClockWindow:
    """Shader-clock samples (attn_clock_sample) on the launch stream just outside a
    timed region; .ghz() gives clock_ghz() over the interval."""

    def __init__(self, torch, dev, stream, bd, n=256):
        self.bd, self.stream, self.n = bd, stream, n
        self.buf = [torch.empty((n, 4), dtype=torch.int64, device=dev) for _ in range(2)]

    def sample(self, i):
        st = self.bd.c_attn_clock_sample(self.buf[i].data_ptr(), self.n, self.stream)
        if st != 0:
            raise RuntimeError(f"attn_clock_sample: {self.bd.status_string(st)}")

    def ghz(self):
        return clock_ghz(self.buf[0].cpu().numpy().view(np.uint64), self.buf[1].cpu().numpy().view(np.uint64))


def receipt_of(errs: dict, bigs: dict, dtype: str, what: str) -> dict:
    """PASS / FAIL receipt from max |GPU - oracle| (errs) and max |oracle| (bigs)."""
    kind, tol = RECEIPT_TOL[dtype]
    worst = {n: (errs[n] / bigs[n] if bigs[n] > 0 else errs[n]) if kind == "rel" else errs[n] for n in errs}
    ok = all(np.isfinite(v) and v <= tol for v in worst.values())
    return {"status": "PASS" if ok else "FAIL", "checked": what,
            "max_err": {n: float(f"{v:.3g}") for n, v in worst.items()},
            "bar": f"max |d| <= {tol}" if kind == "abs" else f"max |d| / max |oracle| <= {tol}"}


def fail_receipt(metric: str, receipt: dict, workload: str):
    print(json.dumps({"metric": metric, "receipt": receipt, "config": {"workload": workload}}), flush=True)
    print("bench.py: the receipt failed; no timing is reported", file=sys.stderr)
    sys.exit(3)


def compare_heads(gpu: dict, ref_heads: list, dtype: str, G: int) -> dict:
    """The receipt: the session's outputs (gpu: name -> callable (b, h) -> float64
    array) against the oracle's per-head results [((b, h), {o, lse, dq, dk, dv})].
    O, LSE and dQ compare per query head; dK and dV per key/value head, as the sum
    of its G query heads' oracle contributions, for the key/value heads whose
    whole group is in the sample."""
    kind, tol = RECEIPT_TOL[dtype]
    err = {n: 0.0 for n in OUTPUTS}
    big = {n: 0.0 for n in OUTPUTS}
    groups = {}
    for (b, h), r in ref_heads:
        for n in ("o", "lse", "dq"):
            d = np.abs(gpu[n](b, h) - r[n])
            err[n] = max(err[n], float(d.max()))
            big[n] = max(big[n], float(np.abs(r[n]).max()))
        g = groups.setdefault((b, h // G), {"n": 0, "dk": 0.0, "dv": 0.0})
        g["n"] += 1
        g["dk"] = g["dk"] + r["dk"]
        g["dv"] = g["dv"] + r["dv"]
    nkv = 0
    for (b, kh), g in groups.items():
        if g["n"] != G:
            continue
        nkv += 1
        for n in ("dk", "dv"):
            err[n] = max(err[n], float(np.abs(gpu[n](b, kh) - g[n]).max()))
            big[n] = max(big[n], float(np.abs(g[n]).max()))
    worst = {n: (err[n] / big[n] if big[n] > 0 else err[n]) if kind == "rel" else err[n] for n in OUTPUTS}
    if nkv == 0:
        worst.pop("dk")
        worst.pop("dv")
    ok = bool(ref_heads) and all(v <= tol for v in worst.values())
    return {"status": "PASS" if ok else "FAIL", "heads": len(ref_heads), "kv_heads": nkv,
            "max_err": {n: float(f"{v:.3g}") for n, v in worst.items()},
            "bar": f"{'max |d| / max |oracle|' if kind == 'rel' else 'max |d|'} <= {tol:g}"}


def step_statistics(step, k, torch, between=None) -> dict:
    """k steps, each bracketed by HIP events: median, min and p95 of the step time
    (ms), and a bootstrap 95% interval of the median (10^4 resamples, fixed seed).
    `between` runs untimed after each step (a cache-clearing write)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        step()
        b.record()
        if between is not None:
            between()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    rng = np.random.default_rng(0)
    boot = np.median(t[rng.integers(0, len(t), size=(10000, len(t)))], axis=1)
    out = {"n": k, "median": round(float(np.median(t)), 5), "min": round(float(t.min()), 5),
           "p95": round(float(np.percentile(t, 95)), 5),
           "ci95_median": [round(float(np.percentile(boot, 2.5)), 5), round(float(np.percentile(boot, 97.5)), 5)]}
    return out


def clock_warm(step, torch, seconds: float = CLOCK_WARM_SECONDS) -> int:
    """Untimed steps (in groups of 10) until `seconds` of wall time have passed, so
    that the clock has left its idle state before the warm-up; returns the count."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n


def warm_up(step, args, torch) -> int:
    """Run the untimed warm-up (after clock_warm); return the number of steps run:
    --warmup W runs exactly W, the default DEFAULT_WARMUP."""
    n = DEFAULT_WARMUP if args.warmup is None else args.warmup
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    return n


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed warm-up steps (default {DEFAULT_WARMUP}); they follow {CLOCK_WARM_SECONDS} s of "
                         "untimed steps that warm the clock")
    ap.add_argument("--workload", default="gpt205m_bf16",
                    choices=sorted(si.WORKLOADS) + sorted(si.GQA_WORKLOADS) + sorted(si.F16_WORKLOADS)
                    + sorted(si.DECODE_WORKLOADS) + sorted(si.FP8_WORKLOADS),
                    help="grouped key/value head workloads run attn_fwd_gqa / attn_bwd_gqa")
    ap.add_argument("--bwd", choices=("split", "atomic"), default="split",
                    help="backward: attn_bwd (dQ pass + dK/dV pass, deterministic) or attn_bwd_atomic "
                         "(dK/dV pass with fp32 atomic dQ; D = 64, one query head per key/value head)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many fwd+bwd steps and exit (for rocprofv3), no JSON")
    ap.add_argument("--sessions", type=int, default=2, choices=(1, 2),
                    help="2: repeat the measurement in a fresh process afterwards (training workloads)")
    ap.add_argument("--expect-digest", default=None, help=argparse.SUPPRESS)
    return ap.parse_args()


def kernel_units(w):
    """Algorithmic work per launch of each kernel.

    One 'GEMM unit' is one S x S x D contraction over the visible (causal) half:
    B*H*S^2*D FLOPs (2 FLOPs per multiply-add, halved by causality).  The
    forward does 2 units (QK^T, PV); the backward's 5 units are S, dP, dV, dK in
    the dK/dV pass and dQ in the dQ pass (the dQ pass's recomputed S and dP are
    not algorithmic work).  The dQ pass also reads O to form delta = rowsum(dO o O)
    and writes delta, which the dK/dV pass reads.  With grouped key/value heads the
    units count query heads (the work is the same); K, V, dK, dV are H_kv/H the size,
    and "bwd" is the whole backward (both passes).
    """
    unit = w.B * w.H * w.S * w.S * w.D * (1.0 if w.causal else 2.0)
    elem = 4 if w.dtype == "f32" else 2
    tensor = w.B * w.H * w.S * w.D * elem
    kvt = tensor // w.H * w.kv_heads
    rows = w.B * w.H * w.S * 4
    return {
        "fwd": {"flops": 2 * unit, "bytes": tensor + 2 * kvt + tensor + rows},
        "bwd_dq": {"flops": 1 * unit, "bytes": 3 * tensor + 2 * kvt + rows + tensor + rows},
        "bwd_dkdv": {"flops": 4 * unit, "bytes": 2 * tensor + 2 * kvt + 2 * rows + 2 * kvt},
        "bwd": {"flops": 5 * unit, "bytes": 3 * tensor + 2 * kvt + rows + tensor + 2 * kvt},
    }


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it still matches the kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(rf"^{re.escape(kernel)}\s+{re.escape(workload)}\s+(\S+)\s+(\S+)\s+(\S+)\s*$", text, flags=re.M)
    if not m:
        return None
    src_hash, fetch_b, write_b = m.group(1), float(m.group(2)), float(m.group(3))
    if kernel_sources_hash(kernel) != src_hash:
        return None
    return fetch_b + write_b


def read_kernel_time(kernel: str, workload: str):
    """Average duration (us) of the kernel under rocprofv3 --kernel-trace --stats, from
    the committed summary, if it still matches the kernel source."""
    if not os.path.exists(TIMES_FILE):
        return None
    text = open(TIMES_FILE).read()
    m = re.search(rf"^{re.escape(kernel)}\s+{re.escape(workload)}\s+(\S+)\s+(\S+)\s*$", text, flags=re.M)
    if not m or kernel_sources_hash(kernel) != m.group(1):
        return None
    return float(m.group(2))


# The sources each timed kernel is compiled from: its traffic figures stay valid
# while these are unchanged.
KERNEL_SOURCES = {
    "fwd": ("attn_fwd_mfma.hip", "attn_direct.h", "attn_tiles.h", "attn_device.h", "attn_launch.h"),
    "bwd_dq": ("attn_bwd_mfma.hip", "attn_direct.h", "attn_tiles.h", "attn_device.h", "attn_launch.h"),
    "bwd_dkdv": ("attn_bwd_mfma.hip", "attn_direct.h", "attn_tiles.h", "attn_device.h", "attn_launch.h"),
}


def kernel_sources_hash(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the kernel's source files, in the order listed."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_attention_flash_amd", "csrc")
    for f in KERNEL_SOURCES.get(kernel, ()):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(w, x, target_s: float):
    """Time the fp64 oracle (fwd + bwd, head by head) on a bounded sample of the
    workload; return the baseline record and the oracle's per-head results (the
    receipt compares the session's outputs against them)."""
    from oracle import attention_head
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head = w.flops / len(heads)
    G = w.H // w.kv_heads  # query head h reads key/value head h // G
    done = []
    t0 = time.perf_counter()
    for b, h in heads:
        r = attention_head(x["q"][b, h], x["k"][b, h // G], x["v"][b, h // G], x["do"][b, h], w.scale, w.causal)
        done.append(((b, h), r))
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    rec = {
        "value": round(len(done) * per_head / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "host_cores": host_cores(),
        "kind": "oracle",
        "sample": f"{len(done)} of {len(heads)} heads (S={w.S}, D={w.D}), fwd+bwd in fp64, {dt:.1f} s; "
                  f"cores = the BLAS threads the oracle's products ran on, host_cores = this process's "
                  f"CPU affinity",
    }
    return rec, done


def decode_bench(args, dev):
    """One decode step per iteration (attn_decode: the split pass and, for several
    chunks, the merge pass) over a resident cache; value = algorithmic HBM bytes
    per second: each sequence's cache rows in use (K and V), plus q, O and LSE.
    Steps rotate over copies of the cache totalling >= 1 GiB (cold MALL)."""
    import torch

    import causal_attention_flash_amd as caf

    w = si.DECODE_WORKLOADS[args.workload]
    x = si.make_decode_inputs(w, seed=0)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]

    def dev_t(name):
        if w.dtype == "f32":
            return torch.from_numpy(x[name]).to(dev)
        return torch.from_numpy(x[name + "_bits"].view(np.int16)).to(dev).view(tdt)

    q, k, v = (dev_t(n) for n in ("q", "k", "v"))
    # Consecutive steps read different copies of the cache (as a model's layers
    # do), at least 1 GiB in all, so no step finds its cache in the 256 MB MALL.
    cache_bytes = 2 * k.numel() * k.element_size()
    ncopy = max(1, -(-(1 << 30) // cache_bytes))
    kcs = [k] + [k.clone() for _ in range(ncopy - 1)]
    vcs = [v] + [v.clone() for _ in range(ncopy - 1)]
    lens = x["kv_lens"] if x["kv_lens"] is not None else np.full(w.B, w.L, np.int32)
    kl = torch.from_numpy(lens.astype(np.int32)).to(dev)
    dt = {"bf16": caf.ATTN_BF16, "f16": caf.ATTN_F16, "f32": caf.ATTN_F32}[w.dtype]
    bd = caf._binding
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    nws = bd.c_attn_decode_workspace_bytes(w.B, w.H, w.Hkv, w.L, w.D, dt)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    it = [0]

    def step():
        i = it[0] % ncopy
        it[0] += 1
        st = bd.c_attn_decode(q.data_ptr(), kcs[i].data_ptr(), vcs[i].data_ptr(), kl.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), ws.data_ptr(), nws, w.B, w.H, w.Hkv, w.L, w.D, w.scale, dt, stream)
        if st != 0:
            raise caf.AttnError(st, "decode")

    elem = q.element_size()
    nbytes = float(lens.sum()) * w.Hkv * w.D * elem * 2 + 2 * w.B * w.H * w.D * elem + w.B * w.H * 4
    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        print(f"profile run: {args.profile_steps} steps of {w.name}", flush=True)
        return
    # the session's own first step, then the oracle on the sequences the CPU
    # baseline covers and the receipt, before any timing
    step()
    torch.cuda.synchronize()
    o_host = o.to(torch.float64).cpu().numpy()
    lse_host = lse.to(torch.float64).cpu().numpy()
    cpu_rec, receipt = None, None
    if not args.no_cpu_baseline:
        from oracle import decode
        t0 = time.perf_counter()
        nb = 0
        done_bytes = 0.0
        errs = {"o": 0.0, "lse": 0.0}
        bigs = {"o": 0.0, "lse": 0.0}
        lse_pattern = True
        while nb < w.B and time.perf_counter() - t0 < args.cpu_seconds:
            b = slice(nb, nb + 1)
            ro, rl = decode(x["q"][b], x["k"][b], x["v"][b], w.scale, lens[b])
            errs["o"] = max(errs["o"], float(np.abs(o_host[b] - ro).max()))
            bigs["o"] = max(bigs["o"], float(np.abs(ro).max()))
            fin = np.isfinite(rl)
            lse_pattern &= bool((np.isfinite(lse_host[b]) == fin).all())
            if fin.any():
                errs["lse"] = max(errs["lse"], float(np.abs(lse_host[b][fin] - rl[fin]).max()))
                bigs["lse"] = max(bigs["lse"], float(np.abs(rl[fin]).max()))
            done_bytes += float(lens[nb]) * w.Hkv * w.D * elem * 2 + 2 * w.H * w.D * elem + w.H * 4
            nb += 1
        dtc = time.perf_counter() - t0
        cpu_rec = {"value": round(done_bytes / dtc / 1e9, 4), "unit": "GB/s",
                   "cores": blas_threads(), "host_cores": host_cores(), "kind": "oracle",
                   "sample": f"{nb} of {w.B} sequences, fp64 decode, {dtc:.1f} s"}
        receipt = receipt_of(errs, bigs, w.dtype, f"O and LSE of {nb} of {w.B} sequences, all heads")
        if not lse_pattern:
            receipt["status"] = "FAIL"
            receipt["lse_pattern"] = "empty sequences (LSE = -inf) differ from the oracle's"
        if receipt["status"] != "PASS":
            fail_receipt("decode attention step, algorithmic HBM GB/s on 1 GPU", receipt, w.name)
    clk = ClockWindow(torch, dev, stream, bd)
    clock_warm(step, torch)
    nwarm = warm_up(step, args, torch)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clk.sample(0)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    clk.sample(1)
    torch.cuda.synchronize()
    clock = clk.ghz()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    # per-call durations (events around each call on the launch stream)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    durs = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    mean_ms = sum(durs) / len(durs)
    value = nbytes * args.steps / (gpu_ms * 1e-3) / 1e9
    # A call is the split pass and the merge pass back to back on the stream, so the
    # timed region's events over K calls give its mean duration; events around every
    # call add gaps of their own (kept beside it as decode_per_call_events).
    call_ms = gpu_ms / args.steps
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": "decode attention step, algorithmic HBM GB/s on 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(gpu_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "L": w.L, "D": w.D,
                   "kv_lens": [int(n) for n in lens], "cache_copies": ncopy, "parallelism": "none (1 GPU)"},
        "tokens_per_s": round(w.B * args.steps / (gpu_ms * 1e-3), 1),
        "wall_s_timed": round(wall, 4),
        "kernel_ms": {"decode": round(call_ms, 5), "decode_per_call_events": round(mean_ms, 5)},
        "roofline": {"kernel": "decode (split + merge passes)", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 5),
                     "traffic": None,
                     "time_base": "HIP-event duration of the timed region / K calls (split and merge passes "
                                  "back to back on the launch stream)"},
        "clock_ghz": clock,
    }
    if receipt is not None:
        result["receipt"] = receipt
    if cpu_rec is not None:
        result["cpu_baseline"] = cpu_rec
    print(json.dumps(result), flush=True)


def fp8_bench(args, dev):
    """Forward with fp8 (E4M3) Q and K (attn_fwd_fp8qk); value = algorithmic forward
    TFLOP/s (4*B*H*S^2*D, halved for causal).  The bf16 forward on the same
    (bf16-exact) values is timed beside it."""
    import torch

    import causal_attention_flash_amd as caf

    w = si.FP8_WORKLOADS[args.workload]
    x = si.make_fp8_inputs(w, seed=0)
    bd = caf._binding
    q8 = torch.from_numpy(x["q8"]).to(dev)
    k8 = torch.from_numpy(x["k8"]).to(dev)
    v = torch.from_numpy(x["v_bits"].view(np.int16)).to(dev).view(torch.bfloat16 if w.v_dtype == "bf16" else torch.float16)
    dt = caf.ATTN_BF16 if w.v_dtype == "bf16" else caf.ATTN_F16
    o = torch.empty((w.B, w.H, w.S, w.D), dtype=v.dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step():
        st = bd.c_attn_fwd_fp8qk(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                                 w.Hkv, w.S, w.D, w.scale, x["q_descale"], x["k_descale"], int(w.causal), dt, stream)
        if st != 0:
            raise caf.AttnError(st, "fwd_fp8qk")

    if args.profile_steps:
        for _ in range(args.profile_steps):
            step()
        torch.cuda.synchronize()
        print(f"profile run: {args.profile_steps} steps of {w.name}", flush=True)
        return
    # the session's own first step, then the oracle on the heads the CPU baseline
    # covers and the receipt, before any timing
    step()
    torch.cuda.synchronize()
    o_host = o.to(torch.float64).cpu().numpy()
    lse_host = lse.to(torch.float64).cpu().numpy()
    metric = "causal attention forward TFLOP/s, fp8 (E4M3) Q and K, on 1 GPU"
    cpu_rec, receipt = None, None
    if not args.no_cpu_baseline:
        from oracle import fp8qk_forward
        G = w.H // w.Hkv
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        t0 = time.perf_counter()
        done = 0
        errs = {"o": 0.0, "lse": 0.0}
        bigs = {"o": 0.0, "lse": 0.0}
        for b, h in heads:
            ro, rl = fp8qk_forward(x["q8"][b:b + 1, h:h + 1], x["k8"][b:b + 1, h // G:h // G + 1],
                                   x["v"][b:b + 1, h // G:h // G + 1], x["q_descale"], x["k_descale"], w.scale,
                                   w.causal)
            errs["o"] = max(errs["o"], float(np.abs(o_host[b, h] - ro[0, 0]).max()))
            bigs["o"] = max(bigs["o"], float(np.abs(ro).max()))
            errs["lse"] = max(errs["lse"], float(np.abs(lse_host[b, h] - rl[0, 0]).max()))
            bigs["lse"] = max(bigs["lse"], float(np.abs(rl).max()))
            done += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dtc = time.perf_counter() - t0
        cpu_rec = {"value": round(done * w.fwd_flops / len(heads) / dtc / 1e12, 6),
                   "unit": "TFLOP/s", "cores": blas_threads(), "host_cores": host_cores(), "kind": "oracle",
                   "sample": f"{done} of {len(heads)} heads (S={w.S}, D={w.D}), fp64 forward, {dtc:.1f} s"}
        # the fp8 parity bar: O and LSE within the bf16 bar (the oracle sees the
        # same E4M3 values, so the bar covers the kernel's own rounding)
        receipt = receipt_of(errs, bigs, "bf16", f"O and LSE of {done} of {len(heads)} heads")
        if receipt["status"] != "PASS":
            fail_receipt(metric, receipt, w.name)
    clk = ClockWindow(torch, dev, stream, bd)
    clock_warm(step, torch)
    nwarm = warm_up(step, args, torch)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clk.sample(0)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    clk.sample(1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    clock = clk.ghz()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    mean_ms = sum(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)) / args.steps
    # the bf16 forward on the same values: torch's own E4M3 conversion on the host
    # (every E4M3 value and its power-of-two descaled form is exact in bf16)
    def decoded(codes, descale):
        f = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * descale
        return f.to(torch.bfloat16).to(dev)

    qb = decoded(x["q8"], x["q_descale"])
    kb = decoded(x["k8"], x["k_descale"])
    vb = v if w.v_dtype == "bf16" else v.to(torch.bfloat16)

    def step_bf16():
        st = bd.c_attn_fwd_gqa(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                               w.Hkv, w.S, w.D, w.scale, int(w.causal), caf.ATTN_BF16, stream)
        if st != 0:
            raise caf.AttnError(st, "fwd_gqa")

    warm_up(step_bf16, args, torch)
    ev0.record()
    for _ in range(args.steps):
        step_bf16()
    ev1.record()
    torch.cuda.synchronize()
    bf16_ms = ev0.elapsed_time(ev1) / args.steps
    value = w.fwd_flops * args.steps / (gpu_ms * 1e-3) / 1e12
    achieved = w.fwd_flops / (mean_ms * 1e-3) / 1e12
    result = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(gpu_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (Q, K) / " + w.v_dtype + " (V, P, O)",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "S": w.S, "D": w.D, "causal": w.causal,
                   "q_descale": x["q_descale"], "k_descale": x["k_descale"], "parallelism": "none (1 GPU)"},
        "wall_s_timed": round(wall, 4),
        "kernel_ms": {"fwd_fp8qk": round(mean_ms, 5), "fwd_bf16_same_values": round(bf16_ms, 5)},
        "roofline": {"kernel": "fwd_fp8qk", "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": round(PEAK_FP8QK_FWD_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8QK_FWD_TFLOPS, 5), "traffic": None,
                     "time_base": "mean of the per-launch HIP-event durations over K steps (second timed pass)"},
        "clock_ghz": clock,
    }
    if receipt is not None:
        result["receipt"] = receipt
    if cpu_rec is not None:
        result["cpu_baseline"] = cpu_rec
    print(json.dumps(result), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every (batch, head) is independent; see the sharding note in the design). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_attention_flash_amd as caf

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    caf.load_library()
    dev = torch.device("cuda:0")
    if args.workload in si.FP8_WORKLOADS:
        fp8_bench(args, dev)
        return
    if args.workload in si.DECODE_WORKLOADS:
        decode_bench(args, dev)
        return
    w = {**si.WORKLOADS, **si.GQA_WORKLOADS, **si.F16_WORKLOADS}[args.workload]
    grouped = w.kv_heads != w.H
    atomic = args.bwd == "atomic"
    if atomic and (grouped or w.D != 64 or w.dtype == "f32"):
        raise SystemExit("--bwd atomic needs D = 64, bf16 or fp16, one query head per key/value head")
    x = si.make_inputs(w, seed=0)

    def dev_t(name):
        if w.dtype in ("bf16", "f16"):
            tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
            return torch.from_numpy(x[name + "_bits"].view(np.int16)).to(dev).view(tdt)
        return torch.from_numpy(x[name]).to(dev)

    q, k, v, do = (dev_t(n) for n in ("q", "k", "v", "do"))
    B, H, S, D = q.shape
    dt = {"bf16": caf.ATTN_BF16, "f16": caf.ATTN_F16, "f32": caf.ATTN_F32}[w.dtype]
    causal = int(w.causal)
    scale = w.scale
    bd = caf._binding
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    Hkv = k.shape[1]
    nws = (bd.c_attn_bwd_gqa_workspace_bytes(B, H, Hkv, S, D, dt) if grouped
           else bd.c_attn_bwd_atomic_workspace_bytes(B, H, S, D, dt) if atomic
           else bd.c_attn_bwd_workspace_bytes(B, H, S, D, dt))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = {n: t.data_ptr() for n, t in dict(q=q, k=k, v=v, o=o, lse=lse, do=do, dq=dq, dk=dk, dv=dv, ws=ws).items()}

    def chk(st, where):
        if st != 0:
            raise caf.AttnError(st, where)

    def fwd():
        if grouped:
            chk(bd.c_attn_fwd_gqa(P["q"], P["k"], P["v"], P["o"], P["lse"], B, H, Hkv, S, D, scale, causal, dt, stream),
                "fwd_gqa")
        else:
            chk(bd.c_attn_fwd(P["q"], P["k"], P["v"], P["o"], P["lse"], B, H, S, D, scale, causal, dt, stream), "fwd")

    def bwd():
        if atomic:
            chk(bd.c_attn_bwd_atomic(P["q"], P["k"], P["v"], P["o"], P["do"], P["lse"], P["dq"], P["dk"], P["dv"],
                                     P["ws"], nws, B, H, S, D, scale, causal, dt, stream), "bwd_atomic")
        elif grouped:
            chk(bd.c_attn_bwd_gqa(P["q"], P["k"], P["v"], P["o"], P["do"], P["lse"], P["dq"], P["dk"], P["dv"],
                                  P["ws"], nws, B, H, Hkv, S, D, scale, causal, dt, stream), "bwd_gqa")
        else:
            chk(bd.c_attn_bwd(P["q"], P["k"], P["v"], P["o"], P["do"], P["lse"], P["dq"], P["dk"], P["dv"], P["ws"],
                              nws, B, H, S, D, scale, causal, dt, stream), "bwd")

    def dq_delta():
        chk(bd.c_attn_bwd_dq_delta(P["q"], P["k"], P["v"], P["o"], P["do"], P["lse"], P["ws"], P["dq"], B, H, S, D,
                                   scale, causal, dt, stream), "dq_delta")

    def dkdv():
        chk(bd.c_attn_bwd_dkdv(P["q"], P["k"], P["v"], P["do"], P["lse"], P["ws"], P["dk"], P["dv"], B, H, S, D,
                               scale, causal, dt, stream), "dkdv")


    if args.profile_steps:
        # A plain copy of known size first: the counters' reading for it calibrates
        # FETCH_SIZE / WRITE_SIZE to bytes (copy_bytes read, copy_bytes written).
        copy_bytes = 1 << 29
        src = torch.ones(copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        for i in range(args.profile_steps):
            fwd()
            bwd()
        torch.cuda.synchronize()
        print(f"profile run: copy of {copy_bytes} bytes, then {args.profile_steps} steps of {w.name}", flush=True)
        return

    step_fn = lambda: (fwd(), bwd())  # noqa: E731
    bwd_first = lambda: (bwd(), fwd())  # noqa: E731

    # ---- the session's own outputs at the timed shape (the receipt checks them)
    step_fn()
    torch.cuda.synchronize()
    outs = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    digest = output_digest(outs, torch, skip=("dq",) if atomic else ())
    host = {n: t.detach().cpu() for n, t in outs.items()}
    gpu_head = {n: (lambda t: (lambda b, h: t[b, h].to(torch.float64).numpy()))(t) for n, t in host.items()}

    baseline, receipt = None, None
    if not args.no_cpu_baseline:
        baseline, ref_heads = cpu_baseline(w, x, args.cpu_seconds)
        receipt = compare_heads(gpu_head, ref_heads, w.dtype, w.H // w.kv_heads)
    elif args.expect_digest:
        receipt = {"status": "PASS" if digest == args.expect_digest else "FAIL",
                   "kind": "outputs bitwise equal to the first session's (which passed the oracle check)"}
    if receipt is not None and receipt["status"] != "PASS":
        print(json.dumps({"metric": METRIC_TRAIN, "receipt": receipt, "config": {"workload": w.name}}), flush=True)
        print("bench.py: the receipt failed; no timing is reported", file=sys.stderr)
        sys.exit(3)

    clk_n = 256
    clk = [torch.empty((clk_n, 4), dtype=torch.int64, device=dev) for _ in range(2)]

    def clock_sample(i):
        chk(bd.c_attn_clock_sample(clk[i].data_ptr(), clk_n, stream), "clock_sample")

    with GpuLock():
        nclock = clock_warm(step_fn, torch)
        nwarm = warm_up(step_fn, args, torch)

        # ---- timed region: exactly K steps of fwd + bwd, the shader clock sampled
        # just outside it
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        clock_sample(0)
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(args.steps):
            fwd()
            bwd()
        ev1.record()
        clock_sample(1)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        ms_per_step = gpu_ms / args.steps
        clock = clock_ghz(clk[0].cpu().numpy().view(np.uint64), clk[1].cpu().numpy().view(np.uint64))

        # ---- per-kernel durations: the same K steps, each kernel attn_bwd launches
        # (in its order) bracketed by events; the grouped form has no stage entry
        # points, so there the backward is timed as one (its dQ and dK/dV passes), and
        # so is the atomic-dQ backward (delta, zero fill, fused pass, dQ conversion),
        # the fp32 backward and the 16-bit D = 64 backward of grids whose 128-row dQ
        # and dK/dV blocks fit in three rounds at two per CU: attn_bwd runs those as
        # one launch
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        one_launch = w.dtype == "f32" or (D == 64 and 2 * -(-S // 128) * B * H <= 6 * cus)
        if grouped or atomic or one_launch:
            names = ("fwd", "bwd")
            calls = (fwd, bwd)
        else:
            names = ("fwd", "bwd_dq", "bwd_dkdv")
            calls = (fwd, dq_delta, dkdv)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            evs[i][0].record()
            for j, fn in enumerate(calls):
                fn()
                evs[i][j + 1].record()
        torch.cuda.synchronize()
        durations = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]
                     for j, n in enumerate(names)}
        per_kernel = {n: statistics.median(d) for n, d in durations.items()}
        per_kernel_mean = {n: sum(d) / len(d) for n, d in durations.items()}

        # ---- per-step distribution (the same K steps, one event pair each), in
        # both dispatch orders; then cache-cold: 512 MiB written between steps (more
        # than the 256 MB MALL), untimed
        steps_warm = step_statistics(step_fn, args.steps, torch)
        steps_rev = step_statistics(bwd_first, args.steps, torch)
        scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        steps_cold = step_statistics(step_fn, args.steps, torch, between=lambda: scratch.fill_(1.0))
        del scratch

    units = kernel_units(w)
    dom = max(names, key=lambda n: per_kernel_mean[n])
    dom_ms = per_kernel_mean[dom]
    mfma_peak = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS  # fp16 dense MFMA peak = bf16
    achieved = units[dom]["flops"] / (dom_ms * 1e-3) / 1e12
    traffic = read_traffic(dom, w.name)
    prof_us = read_kernel_time(dom, w.name)

    value = w.flops * args.steps / (gpu_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_TRAIN,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": nwarm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "S": w.S, "D": w.D,
                   "causal": bool(w.causal), "backward": "attn_bwd_atomic" if atomic else "attn_bwd",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)"},
        "pct_of_mfma_peak": round(100.0 * value / mfma_peak, 3),
        "receipt": receipt,
        "clock_warm": {"seconds": CLOCK_WARM_SECONDS, "steps": nclock},
        "clock_ghz": clock,
        "wall_s_timed": round(wall, 4),
        "kernel_ms": {n: round(per_kernel_mean[n], 5) for n in names},
        "kernel_ms_median": {n: round(per_kernel[n], 5) for n in names},
        "step_ms": steps_warm,
        "step_ms_bwd_first": steps_rev,
        "step_ms_cache_cold": steps_cold,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": mfma_peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / mfma_peak, 5),
            "traffic": traffic,
            "time_base": "mean of the kernel's per-launch HIP-event durations over K steps (second timed pass)",
            "frac_rocprof": (round(units[dom]["flops"] / (prof_us * 1e-6) / 1e12 / mfma_peak, 5)
                             if prof_us else None),
        },
        "output_digest": digest,
    }
    if clock and w.dtype != "f32":
        peak_clk = CU_COUNT * BF16_FLOP_PER_CLK_CU * clock["mean"] * 1e9 / 1e12
        result["roofline"]["peak_at_clock"] = round(peak_clk, 1)
        result["roofline"]["frac_at_clock"] = round(achieved / peak_clk, 5)
    if baseline is not None:
        result["cpu_baseline"] = baseline
    if args.sessions > 1:
        result["sessions"] = [session_summary(result)] + second_session(args, digest)
    print(json.dumps(result), flush=True)


def output_digest(outs: dict, torch, skip=()) -> str:
    """sha256 (first 16 hex digits) of the output tensors' bytes, in a fixed order;
    `skip` leaves out outputs that are not bitwise reproducible (atomic dQ)."""
    import hashlib
    h = hashlib.sha256()
    for n in OUTPUTS:
        if n in outs and n not in skip:
            h.update(outs[n].detach().contiguous().view(-1).view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()[:16]


def session_summary(d: dict) -> dict:
    return {"value": d.get("value"), "ms_per_step": d.get("ms_per_step"),
            "clock_ghz": (d.get("clock_ghz") or {}).get("mean"), "receipt": (d.get("receipt") or {}).get("status")}


def second_session(args, digest: str) -> list:
    """The same measurement in a fresh process (sequentially, after this one's timed
    sections), its outputs checked bitwise against this session's."""
    cmd = [sys.executable, os.path.abspath(__file__), "--gpus", "1", "--steps", str(args.steps),
           "--workload", args.workload, "--bwd", args.bwd, "--no-cpu-baseline", "--sessions", "1",
           "--expect-digest", digest]
    if args.warmup is not None:
        cmd += ["--warmup", str(args.warmup)]
    import subprocess
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    if r.returncode != 0 or not lines:
        print(r.stderr[-2000:], file=sys.stderr)
        print("bench.py: the second session failed", file=sys.stderr)
        sys.exit(3)
    return [session_summary(json.loads(lines[-1]))]


if __name__ == "__main__":
    main()
