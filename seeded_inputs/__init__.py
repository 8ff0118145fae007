"""Seeded synthetic inputs for causal attention: Q, K, V and the upstream gradient dO.

This module is shared by the oracle side and the GPU side of every test and of the
bench.  It holds no attention arithmetic, only random draws and the float32 ->
bfloat16 / float16 roundings that turn a draw into a 16-bit tensor.

Draw recipe (one recipe for every workload):

* one numpy ``PCG64(seed)`` generator per call;
* float32 standard normals drawn in the order Q, K, V, dO; Q and dO of shape
  [B, H, S, D], K and V of shape [B, H_kv, S, D] (H_kv = H unless the workload
  groups its key/value heads);
* each draw multiplied by its standard deviation in float32;
* for bf16 workloads, every value rounded to the nearest bfloat16, ties to even;
  for f16 workloads, to the nearest IEEE binary16 (the standard float32 ->
  float16 conversion, ties to even, overflow to infinity).

The returned arrays are float32 holding exactly the values the GPU consumes, so
the oracle and the GPU path read identical numbers.

Decode workloads (one new query row per head against a key/value cache) draw, from
one ``PCG64(seed)`` stream, float32 normals for q [B, H, D], then the caches K and V
[B, H_kv, L, D], rounded like the other workloads; with ragged lengths the
per-sequence cache lengths follow as integers uniform in [L/2, L] (numpy's
``Generator.integers``, endpoint included).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "GQA_WORKLOADS",
    "F16_WORKLOADS",
    "DecodeWorkload",
    "DECODE_WORKLOADS",
    "make_decode_inputs",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "round_to_bf16",
    "f32_to_f16_bits",
    "f16_bits_to_f32",
    "f32_to_e4m3_codes",
    "Fp8Workload",
    "FP8_WORKLOADS",
    "make_fp8_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention workload: shape, input dtype and the draw scales."""

    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str  # "f32", "bf16" or "f16"
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    sigma_do: float = 1.0
    causal: bool = True
    Hkv: int = 0  # key/value heads; 0 = H (one per query head)

    @property
    def kv_heads(self) -> int:
        return self.Hkv if self.Hkv else self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Algorithmic fwd+bwd FLOPs, 7*B*H*S^2*D for causal (half of dense)."""
        dense = 14.0 * self.B * self.H * self.S * self.S * self.D
        return dense / 2.0 if self.causal else dense

    @property
    def fwd_flops(self) -> float:
        dense = 4.0 * self.B * self.H * self.S * self.S * self.D
        return dense / 2.0 if self.causal else dense

    @property
    def bwd_flops(self) -> float:
        return self.flops - self.fwd_flops

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the library is measured and checked on.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 4, 128, 64, "f32", 1.0, 1.0, 1.0),
    "gpt12m_bf16": Workload("gpt12m_bf16", 8, 6, 256, 64, "bf16", 1.0, 1.0, 0.1),
    "gpt125m_bf16": Workload("gpt125m_bf16", 8, 12, 1024, 64, "bf16", 1.0, 1.0, 0.1),
    "gpt205m_bf16": Workload("gpt205m_bf16", 4, 16, 2048, 64, "bf16", 1.0, 1.0, 0.1),
    "long8191_bf16": Workload("long8191_bf16", 1, 16, 8191, 128, "bf16", 4.0, 1.0, 0.1),
}

# Grouped key/value heads (GQA) at the shapes of common decoder models: the
# headline workload with 4 query heads per key/value head, and a head_dim 128
# model with 32 query and 8 key/value heads.  Same draw recipe and scales.
GQA_WORKLOADS = {
    "gqa4_gpt205m_bf16": Workload("gqa4_gpt205m_bf16", 4, 16, 2048, 64, "bf16", 1.0, 1.0, 0.1, Hkv=4),
    "gqa8_d128_bf16": Workload("gqa8_d128_bf16", 1, 32, 4096, 128, "bf16", 1.0, 1.0, 0.1, Hkv=8),
}

# fp16 inputs: the headline shape and the long-sequence stress shape with the
# same draws, rounded to IEEE binary16 instead of bfloat16.
F16_WORKLOADS = {
    "gpt205m_f16": Workload("gpt205m_f16", 4, 16, 2048, 64, "f16", 1.0, 1.0, 0.1),
    "long8191_f16": Workload("long8191_f16", 1, 16, 8191, 128, "f16", 4.0, 1.0, 0.1),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns.

    NaN stays NaN (quiet); infinities stay infinite; values beyond the bf16 range
    round to infinity as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out = np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), out)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest, ties to even); return the uint16 bit patterns.

    Values beyond the binary16 range round to infinity (IEEE overflow).
    """
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen binary16 bit patterns to float32 (exact)."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round values to OCP FP8 E4M3 (nearest, ties to even, saturating at +-448);
    return the uint8 codes.  NaN -> 0x7F (sign kept); infinities saturate to 448.

    E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; the quantum is
    2^(E - 3) for a value in [2^E, 2^(E+1)), E >= -6, and 2^-9 below 2^-6.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), 448.0)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))  # a' = f * 2^ex, f in [0.5, 1)
    quantum = np.ldexp(1.0, ex - 1 - 3)
    r = np.minimum(np.round(a / quantum) * quantum, 448.0)  # np.round: ties to even
    sub = r < 2.0 ** -6
    m_sub = np.round(r / 2.0 ** -9).astype(np.int64)
    _, er = np.frexp(np.where(sub, 1.0, r))
    E = er - 1
    m_norm = np.round((np.where(sub, 1.0, r) / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)
    code = np.where(sub, m_sub, ((E + 7) << 3) | m_norm).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | sign).astype(np.uint8)


@dataclasses.dataclass(frozen=True)
class Fp8Workload:
    """Forward with fp8 (E4M3) Q and K: shape, V's type and the draw scales."""

    name: str
    B: int
    H: int
    Hkv: int
    S: int
    D: int
    v_dtype: str  # "bf16" or "f16"
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    causal: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def fwd_flops(self) -> float:
        """Algorithmic forward FLOPs, 4*B*H*S^2*D, halved for causal."""
        dense = 4.0 * self.B * self.H * self.S * self.S * self.D
        return dense / 2.0 if self.causal else dense

    def with_shape(self, **kw) -> "Fp8Workload":
        return dataclasses.replace(self, **kw)


# fp8 Q/K at the headline shape and at the long-sequence stress shape (sigma 4
# on Q and K: logits of sigma ~16), V in bf16.
FP8_WORKLOADS = {
    "gpt205m_fp8qk": Fp8Workload("gpt205m_fp8qk", 4, 16, 16, 2048, 64, "bf16", 1.0, 1.0),
    "long8191_fp8qk": Fp8Workload("long8191_fp8qk", 1, 16, 16, 8191, 128, "bf16", 4.0, 1.0),
}


def make_fp8_inputs(w: Fp8Workload, seed: int = 0) -> dict:
    """Draw Q, K, V from ``PCG64(seed)`` (standard normals times the sigmas) and
    quantise Q and K per tensor: descale = the power of two at or above
    max|x| / 448, codes = E4M3(x / descale).

    Returns ``q8, k8`` (uint8 codes, [B, H, S, D] and [B, H_kv, S, D]),
    ``q_descale, k_descale`` (floats), ``v`` (float32, exact in v_dtype) and ``v_bits``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in (("q", (w.B, w.H, w.S, w.D)), ("k", (w.B, w.Hkv, w.S, w.D))):
        x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(w.sigma_qk)
        amax = float(np.abs(x).max()) if x.size else 1.0
        descale = 2.0 ** math.ceil(math.log2(amax / 448.0)) if amax > 0 else 1.0
        out[name + "8"] = f32_to_e4m3_codes(x.astype(np.float64) / descale)
        out[name + "_descale"] = descale
    v = rng.standard_normal(size=(w.B, w.Hkv, w.S, w.D), dtype=np.float32) * np.float32(w.sigma_v)
    if w.v_dtype == "bf16":
        out["v_bits"] = f32_to_bf16_bits(v)
        out["v"] = bf16_bits_to_f32(out["v_bits"])
    elif w.v_dtype == "f16":
        out["v_bits"] = f32_to_f16_bits(v)
        out["v"] = f16_bits_to_f32(out["v_bits"])
    else:
        raise ValueError(f"unknown v dtype {w.v_dtype!r}")
    return out


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw Q, K, V, dO for workload ``w`` from ``PCG64(seed)``.

    Returns a dict with float32 arrays ``q, k, v, do`` (q and do [B, H, S, D], k and
    v [B, H_kv, S, D]; exact in the workload's 16-bit type for bf16 and f16
    workloads) and, for those, their uint16 bit patterns under ``q_bits, k_bits,
    v_bits, do_bits``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    qshape = (w.B, w.H, w.S, w.D)
    kvshape = (w.B, w.kv_heads, w.S, w.D)
    out = {}
    for name, sigma in (("q", w.sigma_qk), ("k", w.sigma_qk), ("v", w.sigma_v), ("do", w.sigma_do)):
        x = rng.standard_normal(size=kvshape if name in ("k", "v") else qshape, dtype=np.float32)
        x *= np.float32(sigma)
        if w.dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[name + "_bits"] = bits
            x = bf16_bits_to_f32(bits)
        elif w.dtype == "f16":
            bits = f32_to_f16_bits(x)
            out[name + "_bits"] = bits
            x = f16_bits_to_f32(bits)
        elif w.dtype != "f32":
            raise ValueError(f"unknown dtype {w.dtype!r}")
        out[name] = x
    return out


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: B sequences, H query heads (one row each) over caches of up
    to L rows of H_kv key/value heads."""

    name: str
    B: int
    H: int
    Hkv: int
    L: int
    D: int
    dtype: str  # "f32", "bf16" or "f16"
    ragged: bool = True

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def with_shape(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# Decode steps at the shapes of the headline model (16 heads of 64, 4K context)
# and of a grouped-head model with head_dim 128 (32 query / 8 key/value heads, 8K
# context); eight sequences each, with a mix of cache lengths.
DECODE_WORKLOADS = {
    "decode_gpt205m_bf16": DecodeWorkload("decode_gpt205m_bf16", 8, 16, 16, 4096, 64, "bf16"),
    "decode_gqa8_d128_bf16": DecodeWorkload("decode_gqa8_d128_bf16", 8, 32, 8, 8192, 128, "bf16"),
}


def _round(x: np.ndarray, dtype: str):
    """float32 draw -> (values exact in dtype as float32, uint16 bits or None)."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    if dtype == "f16":
        bits = f32_to_f16_bits(x)
        return f16_bits_to_f32(bits), bits
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x, None


def make_decode_inputs(w: DecodeWorkload, seed: int = 0) -> dict:
    """Draw q, k, v (and kv_lens when ragged) for decode workload ``w``.

    Returns float32 arrays ``q`` [B, H, D], ``k`` and ``v`` [B, H_kv, L, D] (exact in
    the workload's type; uint16 bit patterns under ``*_bits`` for 16-bit types) and
    ``kv_lens`` (int32 [B], or None when every sequence uses all L rows).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, shape in (("q", (w.B, w.H, w.D)), ("k", (w.B, w.Hkv, w.L, w.D)), ("v", (w.B, w.Hkv, w.L, w.D))):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x, bits = _round(x, w.dtype)
        out[name] = x
        if bits is not None:
            out[name + "_bits"] = bits
    out["kv_lens"] = rng.integers(w.L // 2, w.L, size=w.B, endpoint=True).astype(np.int32) if w.ragged else None
    return out
