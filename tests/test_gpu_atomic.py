"""GPU parity for the backward with atomic dQ (attn_bwd_atomic through the C ABI):
against the fp64 oracle on the same seeded inputs (the bf16 / fp16 bars of
tests/gpu_util.py), and against attn_bwd: dV comes from the same code and must be
bit-identical; dK differs only through delta (formed by another pass, fp32 sums in
another order) and dQ only in the order of its fp32 sums.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_head
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def run_both(x, w, device, causal=True):
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    q, k, v, do = (gu.to_device(x, n, w.dtype, device) for n in ("q", "k", "v", "do"))
    o, lse = caf.attn_fwd(q, k, v, scale=w.scale, causal=causal)
    ref = caf.attn_bwd(q, k, v, o, do, lse, scale=w.scale, causal=causal)
    got = caf.attn_bwd_atomic(q, k, v, o, do, lse, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    out = {"o": gu.to_host64(o), "lse": gu.to_host64(lse)}
    out.update({n: gu.to_host64(t) for n, t in zip(("dq", "dk", "dv"), got)})
    base = {n: gu.to_host64(t) for n, t in zip(("dq", "dk", "dv"), ref)}
    return out, base


def oracle_heads(x, w, heads, causal=True):
    res = {n: [] for n in gu.OUTPUTS}
    for b, h in heads:
        r = attention_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], w.scale, causal)
        for n in gu.OUTPUTS:
            res[n].append(r[n])
    return {n: np.stack(v) for n, v in res.items()}


def check_against_attn_bwd(got, base, dtype):
    # dV does not depend on delta: the same code, bit for bit
    np.testing.assert_array_equal(got["dv"], base["dv"])
    # dK: delta comes from the preprocess pass here and from the dQ pass in
    # attn_bwd (fp32 sums in another order); dQ: dS from the other operand layout
    # (S = Q K^T instead of K Q^T; a 16-bit rounding of dS can fall the other way)
    # and the sums in another order.  Both sit inside the oracle bound checked
    # above; here a sanity bound of a fifth of it.
    tol = (gu.BF16_ABS_TOL if dtype == "bf16" else gu.F16_ABS_TOL) / 5
    for n in ("dq", "dk"):
        assert np.abs(got[n] - base[n]).max() <= tol, n


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 255, 256, 257, 300, 1000])
def test_atomic_shapes(device, S, dtype, causal):
    w = si.Workload("atomic", 2, 3, S, 64, dtype, 1.0, 1.0, 0.1, causal)
    print(f"\n[atomic] S={S} {dtype} causal={causal}", flush=True)
    x = si.make_inputs(w, seed=S * 3 + (dtype == "f16"))
    got, base = run_both(x, w, device, causal)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    gu.check(gu.errors(got, oracle_heads(x, w, heads, causal), heads), dtype, f"S={S} {dtype} causal={causal}")
    check_against_attn_bwd(got, base, dtype)


def test_atomic_headline_workload(device):
    """Full size, the launch bench.py times with --bwd atomic; sampled heads against
    the oracle, every element against attn_bwd."""
    w = si.WORKLOADS["gpt205m_bf16"]
    x = si.make_inputs(w, seed=0)
    got, base = run_both(x, w, device)
    heads = [(0, 0), (1, 7), (2, 11), (3, 15)]
    gu.check(gu.errors(got, oracle_heads(x, w, heads), heads), "bf16", f"gpt205m heads={heads}")
    check_against_attn_bwd(got, base, "bf16")


def test_atomic_unsupported(device):
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    for D, dt in ((128, torch.bfloat16), (80, torch.bfloat16), (64, torch.float32)):
        q = torch.zeros(1, 2, 8, D, dtype=dt, device=device)
        lse = torch.zeros(1, 2, 8, dtype=torch.float32, device=device)
        with pytest.raises(caf.AttnError):
            caf.attn_bwd_atomic(q, q, q, q, q, lse)


@pytest.mark.parametrize("S", [45, 100])
def test_atomic_dense_ragged_negative_logits(device, S):
    """Non-causal, S not a multiple of 32, every scaled score near -20 (so LSE is
    about -16): the key slots past S in the last key block would give P =
    exp(-LSE) ~ 1e7 and, in fp16, an infinite dS; those slots must not reach dQ."""
    w = si.Workload("atomic_neg", 1, 2, S, 64, "f16", 1.0, 1.0, 0.1, False)
    x = si.make_inputs(w, seed=9100 + S)
    rng = np.random.default_rng(9200 + S)
    e1 = np.zeros(64, np.float32)
    e1[0] = 1.0
    # q . k * scale ~ 12 * -13.5 / 8 = -20.25, plus a small spread
    q = 12.0 * e1 + 0.05 * rng.standard_normal((1, 2, S, 64)).astype(np.float32)
    k = -13.5 * e1 + 0.05 * rng.standard_normal((1, 2, S, 64)).astype(np.float32)
    for name, val in (("q", q), ("k", k)):
        bits = si.f32_to_f16_bits(val)
        x[name + "_bits"] = bits
        x[name] = si.f16_bits_to_f32(bits)
    print(f"\n[atomic dense negative logits] S={S} f16", flush=True)
    got, base = run_both(x, w, device, causal=False)
    heads = [(0, 0), (0, 1)]
    ref = oracle_heads(x, w, heads, causal=False)
    assert ref["lse"].max() < -13.0
    gu.check(gu.errors(got, ref, heads), "f16", f"dense negative logits S={S}")
    check_against_attn_bwd(got, base, "f16")


@pytest.mark.parametrize("i", range(16))
def test_atomic_random_shapes(device, i):
    """Seeded sweep: batch, heads, dtype, causality and a ragged S (D = 64)."""
    rng = np.random.default_rng(4000 + i)
    dtype = str(rng.choice(["bf16", "f16"]))
    causal = bool(rng.integers(0, 2))
    S = int(np.exp(rng.uniform(0.0, np.log(1500.0))))
    w = si.Workload(f"atomic_rand{i}", int(rng.integers(1, 3)), int(rng.integers(1, 5)), S, 64, dtype, 1.0, 1.0,
                    0.1, causal)
    print(f"\n[atomic random {i}] B={w.B} H={w.H} S={S} {dtype} causal={causal}", flush=True)
    x = si.make_inputs(w, seed=8000 + i)
    got, base = run_both(x, w, device, causal)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    gu.check(gu.errors(got, oracle_heads(x, w, heads, causal), heads), dtype, f"atomic random case {i}")
    check_against_attn_bwd(got, base, dtype)
