"""GPU parity for decode attention (attn_decode through the C ABI) against the fp64
oracle's decode on the same seeded inputs.  Tolerances as for the other paths
(tests/gpu_util.py): fp32 max|err| / max|ref| <= 1e-4 per output, bf16 max|err|
<= 2e-2, fp16 max|err| <= 5e-3.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import decode
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def to_dev(x, name, dtype, device):
    torch = gu.torch_mod()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x[name], dtype=np.float32)).to(device)
    bits = np.ascontiguousarray(x[name + "_bits"]).view(np.int16)
    return torch.from_numpy(bits).to(device).view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def run(x, w, device, lens=None):
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    q, k, v = (to_dev(x, n, w.dtype, device) for n in ("q", "k", "v"))
    kl = None if lens is None else torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(device)
    o, lse = caf.attn_decode(q, k, v, kv_lens=kl, scale=w.scale)
    torch.cuda.synchronize()
    return gu.to_host64(o), gu.to_host64(lse)


def check(o, lse, ro, rl, dtype, label):
    assert np.isfinite(o).all(), label
    empty = np.isneginf(rl)
    assert (np.isneginf(lse) == empty).all(), f"{label}: LSE -inf pattern"
    errs = {"o": (float(np.abs(o - ro).max()), float(np.abs(ro).max())),
            "lse": (float(np.abs(lse[~empty] - rl[~empty]).max()) if (~empty).any() else 0.0,
                    float(np.abs(rl[~empty]).max()) if (~empty).any() else 0.0)}
    errs.update({n: (0.0, 1.0) for n in ("dq", "dk", "dv")})  # decode has no gradients
    gu.check(errs, dtype, label)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 80, 96, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2), (16, 2), (6, 2)])
def test_decode_shapes(device, dtype, D, H, Hkv):
    """Group sizes 1, 4, 8 (one tile of query heads), 16 (two tiles) and 3 (tiles of one)."""
    w = si.DecodeWorkload("d", 3, H, Hkv, 300, D, dtype, ragged=False)
    print(f"\n[decode] H={H} Hkv={Hkv} L=300 D={D} {dtype}", flush=True)
    x = si.make_decode_inputs(w, seed=H * 7 + D)
    o, lse = run(x, w, device)
    ro, rl = decode(x["q"], x["k"], x["v"], w.scale)
    check(o, lse, ro, rl, dtype, f"H={H} Hkv={Hkv} D={D} {dtype}")


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 255, 256, 257, 1000, 4097, 20000])
def test_decode_lengths(device, L):
    """One chunk and several (the split-and-merge path), tails not a multiple of anything."""
    w = si.DecodeWorkload("dl", 2, 8, 2, L, 64, "bf16", ragged=False)
    x = si.make_decode_inputs(w, seed=L)
    o, lse = run(x, w, device)
    ro, rl = decode(x["q"], x["k"], x["v"], w.scale)
    check(o, lse, ro, rl, "bf16", f"L={L}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_ragged_lengths(device, dtype):
    """Per-sequence lengths, including 0 (no key: O = 0, LSE = -inf), 1, L and values
    beyond L or negative (clamped to [0, L]); rows past a sequence's length hold
    NaN and must never be read."""
    L = 5000
    lens = [0, 1, 2, 257, 4096, L, L + 100, -3]
    w = si.DecodeWorkload("dr", len(lens), 8, 4, L, 128, dtype, ragged=False)
    x = si.make_decode_inputs(w, seed=11)
    clamped = np.clip(np.array(lens), 0, L)
    for b, n in enumerate(clamped):
        for name in ("k", "v"):
            x[name][b, :, n:] = np.nan
            if dtype != "f32":
                x[name + "_bits"][b, :, n:] = 0x7FC0 if dtype == "bf16" else 0x7E00
    o, lse = run(x, w, device, lens)
    ro, rl = decode(x["q"], x["k"], x["v"], w.scale, clamped)
    check(o, lse, ro, rl, dtype, f"ragged {dtype}")
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()


@pytest.mark.parametrize("name", list(si.DECODE_WORKLOADS))
def test_decode_workloads(device, name):
    """Full size, the launch bench.py times, every head against the oracle."""
    w = si.DECODE_WORKLOADS[name]
    print(f"\n[decode] {name}: B={w.B} H={w.H} Hkv={w.Hkv} L={w.L} D={w.D}", flush=True)
    x = si.make_decode_inputs(w, seed=0)
    o, lse = run(x, w, device, x["kv_lens"])
    ro, rl = decode(x["q"], x["k"], x["v"], w.scale, x["kv_lens"])
    check(o, lse, ro, rl, w.dtype, name)


def test_decode_deterministic_and_lens_none(device):
    """Run to run bitwise equal; kv_lens = None equals every length set to L."""
    w = si.DecodeWorkload("dd", 4, 16, 4, 3000, 64, "bf16", ragged=False)
    x = si.make_decode_inputs(w, seed=5)
    a = run(x, w, device)
    b = run(x, w, device)
    c = run(x, w, device, [w.L] * w.B)
    for u, v in ((a, b), (a, c)):
        np.testing.assert_array_equal(u[0], v[0])
        np.testing.assert_array_equal(u[1], v[1])


def test_decode_is_last_row_of_forward(device):
    """Decode of the newest query over the whole cache equals the causal forward's
    last row on the same sequence (both on the GPU; bf16 output rounding apart)."""
    import causal_attention_flash_amd as caf
    torch = gu.torch_mod()
    w = si.WORKLOADS["gpt12m_bf16"].with_shape(B=2, H=4, S=777)
    x = si.make_inputs(w, seed=8)
    q, k, v = (gu.to_device(x, n, "bf16", device) for n in ("q", "k", "v"))
    o, lse = caf.attn_fwd(q, k, v)
    od, ld = caf.attn_decode(q[:, :, -1].contiguous(), k, v)
    torch.cuda.synchronize()
    assert (od.float() - o[:, :, -1].float()).abs().max().item() <= 2 ** -8 * 4
    assert (ld - lse[:, :, -1]).abs().max().item() <= 1e-3
