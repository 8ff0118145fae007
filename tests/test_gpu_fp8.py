"""GPU parity for the forward with fp8 (OCP E4M3) Q and K (attn_fwd_fp8qk through the
C ABI) against the fp64 oracle's fp8qk_forward on the same seeded codes.

Tolerance: the bf16 bar, max |err| <= 2e-2 for O and LSE (tests/gpu_util.py), also
for fp16 V.  Derivation: the oracle sums the exact products of the decoded
values in fp64; the fp8 matrix instruction sums them in fp32 with a narrower
internal alignment, measured at up to ~6e-5 of the dot product's magnitude.  For
the sigma-4 draw at D = 128 (|q.k| up to ~200 before the 1/sqrt(D) scale) that
moves a logit by ~1e-3, P by ~1e-3 relative and O by ~1e-3 * max|V| < 5e-3;
the bf16 roundings of P and O, which the bf16 bar was set for, stay the larger
terms.
"""
import json
import os

import numpy as np
import pytest

import seeded_inputs as si
from oracle import fp8qk_forward
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def run(x, w, device, causal=None):
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    q8 = torch.from_numpy(np.ascontiguousarray(x["q8"])).to(device)
    k8 = torch.from_numpy(np.ascontiguousarray(x["k8"])).to(device)
    v = gu.to_device(x, "v", w.v_dtype, device)
    o, lse = caf.attn_fwd_fp8qk(q8, k8, v, x["q_descale"], x["k_descale"], scale=w.scale,
                                causal=w.causal if causal is None else causal)
    torch.cuda.synchronize()
    return gu.to_host64(o), gu.to_host64(lse)


def check(o, lse, ro, rl, label, heads=None):
    if heads is not None:
        o, lse = np.stack([o[b, h] for b, h in heads]), np.stack([lse[b, h] for b, h in heads])
    errs = {"o": (float(np.abs(o - ro).max()), float(np.abs(ro).max())),
            "lse": (float(np.abs(lse - rl).max()), float(np.abs(rl).max()))}
    assert np.isfinite(o).all() and np.isfinite(lse).all(), label
    errs.update({n: (0.0, 1.0) for n in ("dq", "dk", "dv")})  # forward only
    gu.check(errs, "bf16", label)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("v_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S,H,Hkv", [(1, 4, 4), (2, 2, 1), (63, 4, 4), (65, 4, 2), (129, 3, 1), (300, 8, 2),
                                     (1000, 2, 2)])
def test_fp8qk_shapes(device, S, H, Hkv, D, v_dtype, causal):
    w = si.Fp8Workload("f8", 2, H, Hkv, S, D, v_dtype, 1.0, 1.0, causal)
    print(f"\n[fp8qk] S={S} H={H} Hkv={Hkv} D={D} v={v_dtype} causal={causal}", flush=True)
    x = si.make_fp8_inputs(w, seed=S * 5 + D + H)
    o, lse = run(x, w, device)
    ro, rl = fp8qk_forward(x["q8"], x["k8"], x["v"], x["q_descale"], x["k_descale"], w.scale, causal)
    check(o, lse, ro, rl, f"S={S} H={H}/{Hkv} D={D} {v_dtype} causal={causal}")


@pytest.mark.parametrize("name", list(si.FP8_WORKLOADS))
def test_fp8qk_workloads(device, name):
    """Full size, the launch bench.py times; sampled heads against the oracle (the
    long workload's sigma-4 logits included)."""
    w = si.FP8_WORKLOADS[name]
    print(f"\n[fp8qk] {name}: B={w.B} H={w.H} S={w.S} D={w.D}", flush=True)
    x = si.make_fp8_inputs(w, seed=0)
    o, lse = run(x, w, device)
    heads = [(0, 0), (w.B - 1, w.H - 1)] if w.S > 4096 else [(0, 0), (1 % w.B, 5 % w.H), (w.B - 1, w.H - 1)]
    G = w.H // w.Hkv
    ro, rl = [], []
    for b, h in heads:
        r = fp8qk_forward(x["q8"][b:b + 1, h:h + 1], x["k8"][b:b + 1, h // G:h // G + 1],
                          x["v"][b:b + 1, h // G:h // G + 1], x["q_descale"], x["k_descale"], w.scale, w.causal)
        ro.append(r[0][0, 0])
        rl.append(r[1][0, 0])
    check(o, lse, np.stack(ro), np.stack(rl), f"{name} heads={heads}", heads)
    # O_0 = V_0: the first query sees one key with weight exactly 1
    for b, h in heads:
        np.testing.assert_array_equal(o[b, h, 0], x["v"][b, h // G, 0])


def test_fp8qk_matches_bf16_forward_on_the_same_values(device):
    """E4M3 values times power-of-two descales are exact in bf16: the bf16 forward on
    those values computes the same function with 16-bit products, so the two GPU
    paths agree far inside the oracle tolerance (only the accumulation of the
    scores differs)."""
    import causal_attention_flash_amd as caf
    from oracle import e4m3_decode
    torch = gu.torch_mod()
    w = si.FP8_WORKLOADS["gpt205m_fp8qk"].with_shape(B=1, H=4, Hkv=4, S=700)
    x = si.make_fp8_inputs(w, seed=2)
    o8, l8 = run(x, w, device)
    q = (e4m3_decode(x["q8"]) * x["q_descale"]).astype(np.float32)
    k = (e4m3_decode(x["k8"]) * x["k_descale"]).astype(np.float32)
    np.testing.assert_array_equal(si.round_to_bf16(q), q)
    np.testing.assert_array_equal(si.round_to_bf16(k), k)
    qb, kb = (torch.from_numpy(si.f32_to_bf16_bits(a).view(np.int16)).to(device).view(torch.bfloat16) for a in (q, k))
    o, lse = caf.attn_fwd(qb, kb, gu.to_device(x, "v", "bf16", device), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert np.abs(gu.to_host64(o) - o8).max() <= 2 ** -7
    # LSE = m + log l with l the sum of the bf16-rounded P (each term off by at most
    # 2^-9 relative, so log l by at most 2^-9); the two paths can use different key
    # tiles, hence different reference points for P: they differ by at most 2^-8
    assert np.abs(gu.to_host64(lse) - l8).max() <= 2 ** -8


def test_fp8qk_accumulator_width_cell(device):
    """Rigel §6: one 448 and 127 terms of 0.0625 sum to 455.9375 (an fp16 accumulator
    would stay at 448); all are E4M3 values, so the fp8 instruction sees them
    exactly.  Single key: LSE = the dot product (up to the fp32 exp2/log2 round trip)."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    with open(os.path.join(GOLDEN, "accumulator_width.json")) as f:
        g = json.load(f)
    D = g["D"]
    q = np.full((1, 1, 1, D), g["q"]["rest"])
    q[..., 0] = g["q"]["first"]
    k = np.full((1, 1, 1, D), g["k"]["rest"])
    k[..., 0] = g["k"]["first"]
    q8 = torch.from_numpy(si.f32_to_e4m3_codes(q)).to(device)
    k8 = torch.from_numpy(si.f32_to_e4m3_codes(k)).to(device)
    v = torch.randn(1, 1, 1, D, device=device).to(torch.bfloat16)
    o, lse = caf.attn_fwd_fp8qk(q8, k8, v, 1.0, 1.0, scale=g["scale"], causal=True)
    torch.cuda.synchronize()
    assert abs(lse.item() - g["lse"]) <= g["lse"] * 2 ** -20, lse.item()
    assert abs(lse.item() - g["lse_with_narrow_accumulator"]) > 1.0
    assert torch.equal(o, v)


def test_fp8qk_deterministic_and_float8_dtype(device):
    """Run to run bitwise equal; torch.float8_e4m3fn tensors are accepted as codes."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    w = si.Fp8Workload("det", 2, 4, 2, 333, 64, "bf16")
    x = si.make_fp8_inputs(w, seed=9)
    a = run(x, w, device)
    b = run(x, w, device)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    q8 = torch.from_numpy(x["q8"]).to(device).view(torch.float8_e4m3fn)
    k8 = torch.from_numpy(x["k8"]).to(device).view(torch.float8_e4m3fn)
    o, lse = caf.attn_fwd_fp8qk(q8, k8, gu.to_device(x, "v", "bf16", device), x["q_descale"], x["k_descale"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.to_host64(o), a[0])


@pytest.mark.parametrize("i", range(24))
def test_fp8qk_random_shapes(device, i):
    """Seeded sweep: group size, head dim, V type, causality, a ragged S, the
    query/key spread and a scale other than 1/sqrt(D)."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    rng = np.random.default_rng(3000 + i)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    v_dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.integers(0, 2))
    S = int(np.exp(rng.uniform(0.0, np.log(1200.0))))
    sigma_qk = float(rng.choice([0.5, 1.0, 2.0]))
    w = si.Fp8Workload(f"f8rand{i}", int(rng.integers(1, 3)), G * Hkv, Hkv, S, D, v_dtype, sigma_qk, 1.0, causal)
    scale = float(rng.uniform(0.5, 1.5)) / np.sqrt(D)
    print(f"\n[fp8 random {i}] B={w.B} H={w.H} Hkv={Hkv} S={S} D={D} v={v_dtype} causal={causal} "
          f"sigma_qk={sigma_qk} scale={scale:.4f}", flush=True)
    x = si.make_fp8_inputs(w, seed=9000 + i)
    q8 = torch.from_numpy(np.ascontiguousarray(x["q8"])).to(device)
    k8 = torch.from_numpy(np.ascontiguousarray(x["k8"])).to(device)
    v = gu.to_device(x, "v", w.v_dtype, device)
    o, lse = caf.attn_fwd_fp8qk(q8, k8, v, x["q_descale"], x["k_descale"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = fp8qk_forward(x["q8"], x["k8"], x["v"], x["q_descale"], x["k_descale"], scale, causal)
    check(gu.to_host64(o), gu.to_host64(lse), ro, rl, f"fp8 random case {i}")
