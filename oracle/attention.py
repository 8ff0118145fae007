"""Plain fp64 CPU oracle for scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The library
never routes through it, and it shares no code with the GPU path.

What it computes is the plain definition, written out with the full score matrix
materialised per (batch, head).  The fused GPU method reaches the same result up
to rounding order (the flash formulation is exact, see "Cooperative tensors,
reductions, and building a fused attention kernel", §1 "Why cooperative tensors
exist"), so the oracle is the definition, not the tiled algorithm:

* scores, softmax and output: S = scale * Q K^T, P = softmax over each row of S,
  O = P V  (same guide, §1; Forge RESEARCH.md §6 "Fused attention design",
  where the scale multiplies Q K^T before the softmax);
* causal mask: for query row i, key column j takes part only when j <= i, with
  row and column in global coordinates (same guide, §5.3 causal-mask snippet and
  §9 "the assembled kernel");
* log-sum-exp: one value per query row, L_i = m_i + ln(l_i) with m_i the row
  maximum and l_i the sum of exp(s_ij - m_i), natural log, in the scaled score
  domain (Forge RESEARCH.md §6, the quantity the forward saves for backward);
* backward: with upstream gradient dO, dV = P^T dO, dP = dO V^T,
  delta_i = sum_j P_ij dP_ij, dS = P o (dP - delta), dQ = scale * dS K,
  dK = scale * dS^T Q  (Forge RESEARCH.md §6, the dQ / dK-dV pass description
  with P recomputed from L, and the "D term" paragraph; the chain rule through
  softmax).

All arithmetic is float64.  Inputs are widened exactly from the float32 values
the GPU consumes (bf16 inputs are bf16-exact float32 values).  Masked entries are
excluded exactly: they contribute 0 to every sum, which is what a finite mask
value on the GPU reaches whenever a row has at least one visible key (always
true for causal self-attention: key i is visible to query i).

Grouped key/value heads (GQA): with H query heads and H_kv key/value heads
(H a multiple of H_kv, G = H / H_kv), query head h reads key/value head h // G
of the same batch entry -- the index map of Forge RESEARCH.md §6 ("GQA",
kv_head = q_head / (n_heads / n_kv_heads)), with no copies of K and V.  Each
query head is then plain attention on its key/value head, and because a
key/value head feeds G query heads, its dK and dV are the sums of the G heads'
contributions (the chain rule through the shared input).

Decode (one new query row per head against a key/value cache): the query is the
newest position, appended after its own key and value, so under the causal rule
it sees every cached row; it is plain attention of one row over the first n
cache rows (Forge RESEARCH.md §6, the decode path of "forge generate": one query
row against a long cache).  With per-sequence cache lengths, batch entry b uses
its first kv_lens[b] rows; a length of 0 leaves no visible key, and the result
is o = 0, LSE = -inf (the convention of a row whose exponential sum is 0).

fp8 query and key (inference forward): Q and K arrive as OCP FP8 E4M3 codes with
one dequantisation factor each.  The Rigel paper (§6 on the low-precision
formats) states that the E4M3 values are the OCP grid, with no infinity (overflow
saturates to 448 on encoding; codes 0x7F and 0xFF are NaN), and (same section,
the accumulator-width probe) that fp8 products are accumulated in at least fp32.
Each code is decoded exactly to float64 from the format's definition (sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 gives the
subnormals m * 2^-9), multiplied by its factor, and the result is plain
attention on those values: the oracle sums the exact products in float64, the
definition the GPU's fp32 matrix-instruction sums approximate.

Parity status: pinned.  Each function here is checked in tests/test_oracle_pins.py
against closed forms, invariants, central finite differences, torch's float64
scaled_dot_product_attention on tiny shapes (with enable_gqa for the grouped
form), and the one numeric cell the pages print (Rigel §6, the 455.9375
accumulator probe).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "head_forward",
    "head_backward",
    "attention_forward",
    "attention_backward",
    "attention_head",
    "gqa_forward",
    "gqa_backward",
    "decode_head",
    "decode",
    "e4m3_decode",
    "fp8qk_forward",
]


def _visible(S: int, causal: bool) -> np.ndarray:
    """Boolean [S, S] matrix: True where query i may attend key j (j <= i if causal)."""
    if not causal:
        return np.ones((S, S), dtype=bool)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    return j <= i


def _probabilities(q, k, scale, causal):
    """Scores, visibility, row max, row LSE and P for one head (all float64)."""
    S = q.shape[0]
    s = scale * (q @ k.T)
    vis = _visible(S, causal)
    s_vis = np.where(vis, s, -np.inf)
    m = s_vis.max(axis=1)  # finite: every row has >= 1 visible key
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    lse = m + np.log(l)
    p = np.where(vis, np.exp(s - lse[:, None]), 0.0)
    return s, vis, lse, p


def head_forward(q, k, v, scale: float, causal: bool = True):
    """One head: q [S, D], k [S, D], v [S, Dv] -> (o [S, Dv], lse [S]), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    _, _, lse, p = _probabilities(q, k, scale, causal)
    o = p @ v
    return o, lse


def head_backward(q, k, v, do, scale: float, causal: bool = True):
    """One head: gradients of sum(dO * O) -> (dq, dk, dv), plus (o, lse), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, lse, p = _probabilities(q, k, scale, causal)
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, o, lse


def attention_head(q, k, v, do, scale: float, causal: bool = True) -> dict:
    """All five outputs of one head as a dict (o, lse, dq, dk, dv)."""
    dq, dk, dv, o, lse = head_backward(q, k, v, do, scale, causal)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _heads(x):
    B, H = x.shape[:2]
    for b in range(B):
        for h in range(H):
            yield b, h


def attention_forward(q, k, v, scale: float, causal: bool = True):
    """[B, H, S, D] inputs -> (o [B, H, S, D], lse [B, H, S]), float64, head by head."""
    B, H, S, _ = q.shape
    o = np.empty(v.shape, dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    for b, h in _heads(q):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool = True):
    """[B, H, S, D] inputs -> (dq, dk, dv), float64, head by head."""
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    for b, h in _heads(q):
        dq[b, h], dk[b, h], dv[b, h], _, _ = head_backward(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv


def _group(q, k):
    """G = H / H_kv for q [B, H, S, D] and k [B, H_kv, S, D]."""
    H, Hkv = q.shape[1], k.shape[1]
    if Hkv < 1 or H % Hkv != 0 or q.shape[0] != k.shape[0]:
        raise ValueError(f"query heads {H} must be a multiple of key/value heads {Hkv}")
    return H // Hkv


def gqa_forward(q, k, v, scale: float, causal: bool = True):
    """q [B, H, S, D], k and v [B, H_kv, S, D] -> (o [B, H, S, D], lse [B, H, S]).

    Query head h attends with key/value head h // (H / H_kv); float64, head by head.
    """
    G = _group(q, k)
    B, H, S, _ = q.shape
    o = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    for b, h in _heads(q):
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h // G], v[b, h // G], scale, causal)
    return o, lse


def gqa_backward(q, k, v, do, scale: float, causal: bool = True):
    """Gradients for the grouped form: dq [B, H, S, D]; dk, dv [B, H_kv, S, D], each
    key/value head's gradient summed over the G query heads that read it."""
    G = _group(q, k)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b, h in _heads(q):
        dq_h, dk_h, dv_h, _, _ = head_backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h], scale, causal)
        dq[b, h] = dq_h
        dk[b, h // G] += dk_h
        dv[b, h // G] += dv_h
    return dq, dk, dv


def decode_head(q, k, v, scale: float):
    """One query row q [D] against cache rows k [n, D], v [n, Dv], all visible ->
    (o [Dv], lse), float64.  n = 0 gives (zeros, -inf)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64), -np.inf
    s = scale * (k @ q)
    m = s.max()
    lse = m + np.log(np.exp(s - m).sum())
    p = np.exp(s - lse)
    return p @ v, lse


def decode(q, k, v, scale: float, kv_lens=None):
    """q [B, H, D]; k, v [B, H_kv, L, D] caches; kv_lens [B] rows in use (None = L)
    -> (o [B, H, D], lse [B, H]), float64.  Query head h reads cache head
    h // (H / H_kv); batch entry b reads its first kv_lens[b] rows."""
    B, H, _ = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    if Hkv < 1 or H % Hkv != 0 or k.shape[0] != B:
        raise ValueError(f"query heads {H} must be a multiple of key/value heads {Hkv}")
    G = H // Hkv
    o = np.empty((B, H, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        n = L if kv_lens is None else int(kv_lens[b])
        for h in range(H):
            o[b, h], lse[b, h] = decode_head(q[b, h], k[b, h // G, :n], v[b, h // G, :n], scale)
    return o, lse


def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64 values, exactly.

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0 the
    mantissa m: e = 0 gives the subnormal m / 8 * 2^-6, otherwise (1 + m / 8) * 2^(e - 7);
    the two codes with e = 15 and m = 7 (0x7F, 0xFF) are NaN, and there is no
    infinity, so e = 15 with m < 7 are ordinary values up to 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def fp8qk_forward(q8, k8, v, q_descale: float, k_descale: float, scale: float, causal: bool = True):
    """q8 [B, H, S, D] and k8 [B, H_kv, S, D] E4M3 codes, v [B, H_kv, S, D] values
    -> (o [B, H, S, D], lse [B, H, S]), float64: plain attention on
    q = decode(q8) * q_descale and k = decode(k8) * k_descale (grouped heads as
    gqa_forward)."""
    q = e4m3_decode(q8) * float(q_descale)
    k = e4m3_decode(k8) * float(k_descale)
    return gqa_forward(q, k, np.asarray(v, dtype=np.float64), scale, causal)
