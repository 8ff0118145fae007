"""GPU parity for grouped key/value heads: attn_fwd_gqa / attn_bwd_gqa through the C ABI
against the fp64 oracle's gqa_forward / gqa_backward (same seeded inputs on both
sides).  Tolerances: tests/gpu_util.py.  For a key/value head, dK and dV sum the
contributions of its G query heads, so the oracle is run per group (the G query
heads of one key/value head) and compared on every element of that group.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import gqa_backward, gqa_forward
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def run_gqa(x, w, device, causal=True):
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    q, k, v, do = (gu.to_device(x, n, w.dtype, device) for n in ("q", "k", "v", "do"))
    o, lse = caf.attn_fwd_gqa(q, k, v, scale=w.scale, causal=causal)
    dq, dk, dv = caf.attn_bwd_gqa(q, k, v, o, do, lse, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return {n: gu.to_host64(t) for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


def check_groups(x, w, gpu, groups, causal=True, label=""):
    """Compare the GPU outputs of the listed (b, key/value head) groups with the oracle."""
    G = w.H // w.kv_heads
    errs = {n: (0.0, 0.0) for n in gu.OUTPUTS}
    for b, j in groups:
        qs, ks = slice(j * G, (j + 1) * G), slice(j, j + 1)
        q, do = x["q"][b:b + 1, qs], x["do"][b:b + 1, qs]
        k, v = x["k"][b:b + 1, ks], x["v"][b:b + 1, ks]
        o, lse = gqa_forward(q, k, v, w.scale, causal)
        dq, dk, dv = gqa_backward(q, k, v, do, w.scale, causal)
        ref = {"o": o[0], "lse": lse[0], "dq": dq[0], "dk": dk[0], "dv": dv[0]}
        got = {"o": gpu["o"][b, qs], "lse": gpu["lse"][b, qs], "dq": gpu["dq"][b, qs],
               "dk": gpu["dk"][b, ks], "dv": gpu["dv"][b, ks]}
        for n in gu.OUTPUTS:
            assert np.isfinite(got[n]).all(), f"{n}: non-finite GPU output"
            e, m = float(np.abs(got[n] - ref[n]).max()), float(np.abs(ref[n]).max())
            errs[n] = (max(errs[n][0], e), max(errs[n][1], m))
    gu.check(errs, w.dtype, label)


@pytest.mark.parametrize("B,H,Hkv,S,D,dtype,causal", [
    (2, 8, 2, 300, 64, "bf16", True),
    (2, 8, 2, 300, 64, "bf16", False),
    (1, 8, 1, 257, 128, "bf16", True),
    (2, 6, 2, 65, 64, "f32", True),
    (1, 4, 2, 129, 128, "f32", False),
    (1, 4, 2, 1, 64, "bf16", True),
    (3, 16, 4, 200, 64, "bf16", True),
    (2, 8, 2, 300, 80, "bf16", True),
    (1, 6, 3, 130, 96, "bf16", False),
    (1, 4, 2, 70, 80, "f32", True),
])
def test_gqa_small_shapes_every_head(device, B, H, Hkv, S, D, dtype, causal):
    w = si.Workload("gqa", B, H, S, D, dtype, 1.0, 1.0, 0.1 if dtype == "bf16" else 1.0, causal, Hkv=Hkv)
    print(f"\n[gqa] B={B} H={H} Hkv={Hkv} S={S} D={D} {dtype} causal={causal}", flush=True)
    x = si.make_inputs(w, seed=7)
    gpu = run_gqa(x, w, device, causal)
    check_groups(x, w, gpu, [(b, j) for b in range(B) for j in range(Hkv)], causal, "all groups")


@pytest.mark.parametrize("name", list(si.GQA_WORKLOADS))
def test_gqa_workloads_sampled_groups(device, name):
    w = si.GQA_WORKLOADS[name]
    print(f"\n[gqa] {name}: B={w.B} H={w.H} Hkv={w.kv_heads} S={w.S} D={w.D}", flush=True)
    x = si.make_inputs(w, seed=0)
    gpu = run_gqa(x, w, device)
    groups = [(0, 0)] if w.S > 2048 else [(0, 0), (w.B - 1, w.kv_heads - 1)]
    check_groups(x, w, gpu, groups, True, f"{name} groups={groups}")
    # O_0 = V_0 exactly for causal attention, for every query head of the group
    G = w.H // w.kv_heads
    for b, j in groups:
        for h in range(j * G, (j + 1) * G):
            np.testing.assert_array_equal(gpu["o"][b, h, 0], x["v"][b, j, 0])


def test_one_head_per_group_matches_mha_bitwise(device):
    """attn_fwd_gqa / attn_bwd_gqa with H_kv = H are attn_fwd / attn_bwd."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    w = si.Workload("g1", 2, 4, 333, 64, "bf16", 1.0, 1.0, 0.1)
    x = si.make_inputs(w, seed=3)
    q, k, v, do = (gu.to_device(x, n, "bf16", device) for n in ("q", "k", "v", "do"))
    o1, l1 = caf.attn_fwd(q, k, v)
    o2, l2 = caf.attn_fwd_gqa(q, k, v)
    g1 = caf.attn_bwd(q, k, v, o1, do, l1)
    g2 = caf.attn_bwd_gqa(q, k, v, o1, do, l1)
    torch.cuda.synchronize()
    for a, b in ((o1, o2), (l1, l2)) + tuple(zip(g1, g2)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
def test_grouped_query_outputs_match_repeated_kv_bitwise(device, D):
    """O, LSE and dQ of a query head depend only on its key/value head: the grouped
    call and the per-head call on K/V repeated G times agree bit for bit; dK/dV of a
    key/value head equal the sum of the per-head dK/dV over its group (to bf16 rounding).
    At D = 128 both backward calls run their passes on concurrent streams."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    w = si.Workload("g4", 2, 8, 300, D, "bf16", 1.0, 1.0, 0.1, Hkv=2)
    x = si.make_inputs(w, seed=5)
    q, k, v, do = (gu.to_device(x, n, "bf16", device) for n in ("q", "k", "v", "do"))
    kr, vr = (t.repeat_interleave(4, dim=1).contiguous() for t in (k, v))
    o1, l1 = caf.attn_fwd_gqa(q, k, v)
    o2, l2 = caf.attn_fwd(q, kr, vr)
    dq1, dk1, dv1 = caf.attn_bwd_gqa(q, k, v, o1, do, l1)
    dq2, dk2, dv2 = caf.attn_bwd(q, kr, vr, o2, do, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)
    for g, r in ((dk1, dk2), (dv1, dv2)):
        summed = r.float().view(2, 2, 4, 300, D).sum(dim=2)
        assert (g.float() - summed).abs().max().item() <= 2e-2


@pytest.mark.parametrize("i", range(24))
def test_gqa_random_shapes(device, i):
    """Seeded sweep: group size G in {2, 3, 4, 8, 16}, key/value heads, head dim,
    dtype, causality and a ragged S; every group against the oracle."""
    rng = np.random.default_rng(2000 + i)
    G = int(rng.choice([2, 3, 4, 8, 16]))
    Hkv = int(rng.integers(1, 3))
    D = int(rng.choice([64, 80, 96, 128]))
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    causal = bool(rng.integers(0, 2))
    S = int(np.exp(rng.uniform(0.0, np.log(700.0))))
    B = int(rng.integers(1, 3))
    w = si.Workload(f"gqa_rand{i}", B, G * Hkv, S, D, dtype, 1.0, 1.0, 1.0 if dtype == "f32" else 0.1, causal, Hkv)
    print(f"\n[gqa random {i}] B={B} H={w.H} Hkv={Hkv} S={S} D={D} {dtype} causal={causal}", flush=True)
    x = si.make_inputs(w, seed=7000 + i)
    gpu = run_gqa(x, w, device, causal)
    check_groups(x, w, gpu, [(b, j) for b in range(B) for j in range(Hkv)], causal, f"gqa random case {i}")
