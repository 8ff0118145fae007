"""Seeded generator: determinism, bf16 rounding, draw scales."""
import numpy as np
import pytest

import seeded_inputs as si


def test_same_seed_same_bytes():
    w = si.WORKLOADS["gpt12m_bf16"].with_shape(B=1, H=2, S=64)
    a = si.make_inputs(w, seed=0)
    b = si.make_inputs(w, seed=0)
    c = si.make_inputs(w, seed=1)
    for n in ("q", "k", "v", "do"):
        assert a[n].tobytes() == b[n].tobytes()
        assert a[n + "_bits"].tobytes() == b[n + "_bits"].tobytes()
        assert a[n].tobytes() != c[n].tobytes()


def test_bf16_round_to_nearest_even_ties():
    # 1 + 2^-8 lies exactly halfway between bf16 neighbours 1 and 1 + 2^-7:
    # the tie goes to the even mantissa (1.0).
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                  1.0 + 2.0 ** -8 + 2.0 ** -20, 65504.0, 0.0, -0.0], dtype=np.float32)
    r = si.round_to_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0 + 2.0 ** -6  # tie between 1+2^-7 (odd) and 1+2^-6 (even)
    assert r[2] == -1.0
    assert r[3] == 1.0 + 2.0 ** -7  # above the tie rounds up
    assert r[4] == 65536.0
    assert r[5] == 0.0 and not np.signbit(r[5])
    assert r[6] == 0.0 and np.signbit(r[6])


def test_bf16_special_values():
    x = np.array([np.inf, -np.inf, np.nan, 3.4e38], dtype=np.float32)
    r = si.round_to_bf16(x)
    assert r[0] == np.inf and r[1] == -np.inf and np.isnan(r[2])
    assert r[3] == np.inf  # beyond the largest finite bf16


def test_bf16_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = si.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_f16_round_to_nearest_even_ties():
    # binary16 has 10 fraction bits: 1 + 2^-11 is halfway between 1 and 1 + 2^-10
    # and goes to the even neighbour 1; 1 + 3*2^-11 lies between 1 + 2^-10 (odd)
    # and 1 + 2^-9 (even) and goes to 1 + 2^-9; 65520 is the tie between 65504 and
    # the next step (65536, beyond the range) and overflows to infinity.
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -(1.0 + 2.0 ** -11),
                  1.0 + 2.0 ** -11 + 2.0 ** -20, 65504.0, 65519.0, 65520.0, 2.0 ** -24, 2.0 ** -26],
                 dtype=np.float32)
    r = si.f16_bits_to_f32(si.f32_to_f16_bits(x))
    assert r[0] == 1.0
    assert r[1] == 1.0 + 2.0 ** -9
    assert r[2] == -1.0
    assert r[3] == 1.0 + 2.0 ** -10
    assert r[4] == 65504.0 and r[5] == 65504.0
    assert r[6] == np.inf
    assert r[7] == 2.0 ** -24            # smallest subnormal, exact
    assert r[8] == 0.0                   # a quarter of it rounds to zero
    # bit patterns of a few exact values
    np.testing.assert_array_equal(si.f32_to_f16_bits(np.array([1.0, -2.0, 0.5], np.float32)),
                                  np.array([0x3C00, 0xC000, 0x3800], np.uint16))


def test_values_are_f16_exact_and_scaled():
    w = si.WORKLOADS["long8191_bf16"].with_shape(S=512, dtype="f16")
    x = si.make_inputs(w, seed=0)
    for n, sigma in (("q", 4.0), ("k", 4.0), ("v", 1.0), ("do", 0.1)):
        np.testing.assert_array_equal(si.f16_bits_to_f32(si.f32_to_f16_bits(x[n])), x[n])
        np.testing.assert_array_equal(si.f32_to_f16_bits(x[n]), x[n + "_bits"])
        assert abs(x[n].std() / sigma - 1.0) < 0.01
    # the same draw as the bf16 workload before rounding: values agree to bf16 precision
    xb = si.make_inputs(w.with_shape(dtype="bf16"), seed=0)
    # (binary16 subnormals below 2^-14 hold absolute, not relative, precision)
    np.testing.assert_allclose(x["q"], xb["q"], rtol=2 ** -8, atol=2 ** -24)


def test_values_are_bf16_exact_and_scaled():
    w = si.WORKLOADS["long8191_bf16"].with_shape(S=512)
    x = si.make_inputs(w, seed=0)
    for n, sigma in (("q", 4.0), ("k", 4.0), ("v", 1.0), ("do", 0.1)):
        np.testing.assert_array_equal(si.round_to_bf16(x[n]), x[n])
        assert abs(x[n].std() / sigma - 1.0) < 0.01
        assert abs(x[n].mean()) < 0.01 * sigma


def test_f32_workload_untouched():
    w = si.WORKLOADS["tiny_f32"]
    x = si.make_inputs(w, seed=0)
    assert "q_bits" not in x
    rng = np.random.Generator(np.random.PCG64(0))
    np.testing.assert_array_equal(x["q"], rng.standard_normal((1, 4, 128, 64), dtype=np.float32))


def test_flop_convention():
    w = si.WORKLOADS["gpt205m_bf16"]
    assert w.flops == pytest.approx(120.26e9, rel=1e-3)
    assert w.fwd_flops == pytest.approx(34.36e9, rel=1e-3)


# --------------------------------------------------------------- fp8 (E4M3)


def test_e4m3_encoder_matches_torch_in_range():
    """Round to nearest even onto the OCP E4M3 grid: torch's float8_e4m3fn
    conversion is an independent implementation of the same rounding (within
    +-448; beyond it torch gives NaN where this encoder saturates)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 3e-2, 1.0, 40.0, 200.0)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(si.f32_to_e4m3_codes(x), ref)


def test_e4m3_encoder_edges():
    # ties to even on the grid: 1 + 1/16 lies halfway between 1 (m=0) and 1.125 (m=1)
    assert si.f32_to_e4m3_codes(np.array([1.0625]))[0] == 0x38
    assert si.f32_to_e4m3_codes(np.array([1.1875]))[0] == 0x3A  # halfway 1.125 / 1.25 -> m=2
    # subnormals: quantum 2^-9; half of it ties to 0, 1.5 quanta to 2
    assert list(si.f32_to_e4m3_codes(np.array([2.0 ** -10, 1.5 * 2.0 ** -9, 2.0 ** -9, 2.0 ** -6]))) == [0, 2, 1, 8]
    # saturation at 448 (the Rigel paper, §6: E4M3 has no infinity and clamps to +-448)
    sat = si.f32_to_e4m3_codes(np.array([449.0, 464.0, 1e9, np.inf, -np.inf, -500.0]))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert si.f32_to_e4m3_codes(np.array([np.nan]))[0] & 0x7F == 0x7F
    assert si.f32_to_e4m3_codes(np.array([-0.0]))[0] == 0x80


def test_fp8_inputs():
    w = si.FP8_WORKLOADS["long8191_fp8qk"].with_shape(S=300)
    x = si.make_fp8_inputs(w, seed=3)
    for n in ("q", "k"):
        c, d = x[n + "8"], x[n + "_descale"]
        assert c.dtype == np.uint8 and c.shape == (1, 16 if n == "q" else w.Hkv, 300, 128)
        assert d == 2.0 ** round(np.log2(d))  # a power of two
        assert not ((c & 0x7F) == 0x7F).any()  # no NaN codes
        # the largest magnitude lands in the top binade of the grid
        assert (c & 0x7F).max() >= 0x70
    np.testing.assert_array_equal(si.bf16_bits_to_f32(x["v_bits"]), x["v"])
    assert si.FP8_WORKLOADS["gpt205m_fp8qk"].fwd_flops == pytest.approx(34.36e9, rel=1e-3)
