"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each test is chosen so that a plausible slip in the oracle (a dropped scale, a
mask off by one, a transposed operand, a wrong sign in the softmax backward, a
log2-vs-ln LSE, a missing delta term) fails at least one of them:

* closed forms: one token; identical keys (uniform attention -> running mean of
  V, LSE = scale*q.k + ln(count)); constant V; zero upstream gradient;
* invariants: P rows sum to 1 and vanish above the diagonal (read out through
  V = identity); O_0 = V_0 and dQ_0 = 0; causality; sum_j dK_j = 0;
  sum_j dV_j = sum_i dO_i; dV of the last key; shift invariance of the keys;
  head permutation;
* central finite differences of L = sum(dO * O) in float64;
* torch's float64 scaled_dot_product_attention with autograd (a library
  routine the attention guide's Core AI section uses as the definition) on
  tiny shapes;
* the one numeric cell the pages print: Rigel §6's accumulator-width probe,
  448 + 127 * 0.0625 = 455.9375 (tests/golden/accumulator_width.json);
* grouped key/value heads: torch's float64 scaled_dot_product_attention with
  enable_gqa and autograd; central finite differences through a shared key/value
  head (pins the summation of dK/dV over the group); the index map h -> h // G
  (a tiled or mis-ordered map fails the repeat identity against the pinned
  per-head oracle).
"""
import json
import os

import numpy as np
import pytest

from oracle import (attention_backward, attention_forward, attention_head, decode, decode_head, gqa_backward,
                    gqa_forward, head_backward, head_forward)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


# ---------------------------------------------------------------- closed forms


@pytest.mark.parametrize("causal", [True, False])
def test_single_token(causal):
    rng = np.random.default_rng(1)
    q, k, v, do = (_rand(rng, 1, 7) for _ in range(4))
    scale = 0.37
    r = attention_head(q, k, v, do, scale, causal)
    np.testing.assert_array_equal(r["o"], v)
    assert r["lse"][0] == pytest.approx(scale * float(q[0] @ k[0]), abs=1e-14)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dv"], do, atol=1e-15)


def test_identical_keys_causal_is_running_mean():
    rng = np.random.default_rng(2)
    S, D = 11, 5
    q = _rand(rng, S, D)
    krow = _rand(rng, D)
    k = np.tile(krow, (S, 1))
    v = _rand(rng, S, 3)
    scale = 0.8
    o, lse = head_forward(q, k, v, scale, causal=True)
    counts = np.arange(1, S + 1)
    running_mean = np.cumsum(v, axis=0) / counts[:, None]
    np.testing.assert_allclose(o, running_mean, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, scale * (q @ krow) + np.log(counts), rtol=1e-13, atol=1e-13)


def test_identical_keys_dense_is_mean():
    rng = np.random.default_rng(3)
    S, D = 9, 4
    q = _rand(rng, S, D)
    krow = _rand(rng, D)
    k = np.tile(krow, (S, 1))
    v = _rand(rng, S, D)
    o, lse = head_forward(q, k, v, 1.3, causal=False)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (S, 1)), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, 1.3 * (q @ krow) + np.log(S), rtol=1e-13, atol=1e-13)


def test_zero_queries_uniform_attention():
    rng = np.random.default_rng(4)
    S, D = 8, 6
    q = np.zeros((S, D))
    k, v = _rand(rng, S, D), _rand(rng, S, D)
    o, lse = head_forward(q, k, v, 0.5, causal=True)
    counts = np.arange(1, S + 1)
    np.testing.assert_allclose(o, np.cumsum(v, axis=0) / counts[:, None], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(counts), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_constant_values_give_zero_qk_gradients(causal):
    rng = np.random.default_rng(5)
    S, D = 10, 6
    q, k, do = _rand(rng, S, D), _rand(rng, S, D), _rand(rng, S, D)
    c = _rand(rng, D)
    v = np.tile(c, (S, 1))
    r = attention_head(q, k, v, do, 0.4, causal)
    np.testing.assert_allclose(r["o"], v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-13)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-13)


def test_zero_upstream_gradient():
    rng = np.random.default_rng(6)
    q, k, v = (_rand(rng, 7, 4) for _ in range(3))
    r = attention_head(q, k, v, np.zeros((7, 4)), 0.5, True)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(r[name], 0.0)


# ----------------------------------------------------------------- invariants


@pytest.mark.parametrize("causal", [True, False])
def test_probabilities_via_identity_values(causal):
    """With V = I the output is P itself: rows sum to 1, zero above the diagonal."""
    rng = np.random.default_rng(7)
    S, D = 13, 5
    q, k = _rand(rng, S, D, sigma=2.0), _rand(rng, S, D, sigma=2.0)
    p, lse = head_forward(q, k, np.eye(S), 0.6, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert (p >= 0).all()
    if causal:
        assert (p[np.triu_indices(S, 1)] == 0.0).all()
        assert (np.diag(p) > 0).all()
    # softmax definition, entry by entry, against the returned LSE
    s = 0.6 * q @ k.T
    for i in range(S):
        for j in range(S):
            if causal and j > i:
                continue
            assert p[i, j] == pytest.approx(np.exp(s[i, j] - lse[i]), rel=1e-12)


def test_first_row_and_first_query_gradient():
    rng = np.random.default_rng(8)
    S, D = 12, 8
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    r = attention_head(q, k, v, do, 0.35, True)
    np.testing.assert_array_equal(r["o"][0], v[0])
    np.testing.assert_allclose(r["dq"][0], 0.0, atol=1e-15)


def test_causality_future_keys_do_not_leak():
    rng = np.random.default_rng(9)
    S, D, cut = 16, 8, 6
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    o1, lse1 = head_forward(q, k, v, 0.3, True)
    k2, v2 = k.copy(), v.copy()
    k2[cut + 1:] = _rand(rng, S - cut - 1, D, sigma=5.0)
    v2[cut + 1:] = _rand(rng, S - cut - 1, D, sigma=5.0)
    o2, lse2 = head_forward(q, k2, v2, 0.3, True)
    np.testing.assert_array_equal(o1[: cut + 1], o2[: cut + 1])
    np.testing.assert_array_equal(lse1[: cut + 1], lse2[: cut + 1])
    assert not np.allclose(o1[cut + 1:], o2[cut + 1:])


@pytest.mark.parametrize("causal", [True, False])
def test_gradient_sums(causal):
    rng = np.random.default_rng(10)
    S, D = 17, 6
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    r = attention_head(q, k, v, do, 0.45, causal)
    # each row of dS sums to zero, so the key gradients sum to zero
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    # each row of P sums to one, so the value gradients sum to the upstream sum
    np.testing.assert_allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)
    # delta_i = dO_i . O_i equals sum_j P_ij dP_ij (P read out via V = I)
    p, _ = head_forward(q, k, np.eye(S), 0.45, causal)
    dp = do @ v.T
    np.testing.assert_allclose((p * dp).sum(axis=1), (do * r["o"]).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_last_key_gradient():
    rng = np.random.default_rng(11)
    S, D = 9, 5
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    r = attention_head(q, k, v, do, 0.5, True)
    p, _ = head_forward(q, k, np.eye(S), 0.5, True)
    np.testing.assert_allclose(r["dv"][S - 1], p[S - 1, S - 1] * do[S - 1], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_key_shift_invariance(causal):
    rng = np.random.default_rng(12)
    S, D, scale = 14, 7, 0.42
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    u = _rand(rng, D)
    a = attention_head(q, k, v, do, scale, causal)
    b = attention_head(q, k + u, v, do, scale, causal)
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(b[name], a[name], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(b["lse"], a["lse"] + scale * (q @ u), rtol=1e-12, atol=1e-12)


def test_batched_matches_per_head_and_heads_permute():
    rng = np.random.default_rng(13)
    B, H, S, D = 2, 3, 10, 4
    q, k, v, do = (_rand(rng, B, H, S, D) for _ in range(4))
    o, lse = attention_forward(q, k, v, 0.5, True)
    dq, dk, dv = attention_backward(q, k, v, do, 0.5, True)
    for b in range(B):
        for h in range(H):
            r = attention_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            np.testing.assert_array_equal(o[b, h], r["o"])
            np.testing.assert_array_equal(lse[b, h], r["lse"])
            np.testing.assert_array_equal(dq[b, h], r["dq"])
            np.testing.assert_array_equal(dk[b, h], r["dk"])
            np.testing.assert_array_equal(dv[b, h], r["dv"])
    perm = [2, 0, 1]
    o2, lse2 = attention_forward(q[:, perm], k[:, perm], v[:, perm], 0.5, True)
    np.testing.assert_array_equal(o2, o[:, perm])
    np.testing.assert_array_equal(lse2, lse[:, perm])


# ------------------------------------------------------- finite differences


def _loss(q, k, v, do, scale, causal):
    o, _ = head_forward(q, k, v, scale, causal)
    return float((do * o).sum())


@pytest.mark.parametrize("S,D", [(5, 3), (9, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_central_finite_differences(S, D, causal):
    rng = np.random.default_rng(100 + S + D)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    dq, dk, dv, _, _ = head_backward(q, k, v, do, scale, causal)
    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / max(np.abs(g).max(), 1e-300)
        assert err <= 1e-6, (name, err)


def test_lse_gradient_finite_difference():
    """d LSE_i / d q_i = scale * sum_j P_ij k_j: pins LSE as a natural-log log-sum-exp."""
    rng = np.random.default_rng(14)
    S, D, scale = 6, 4, 0.7
    q, k = _rand(rng, S, D), _rand(rng, S, D)
    p, lse = head_forward(q, k, np.eye(S), scale, True)
    i, h = 4, 1e-6
    for d in range(D):
        qp, qm = q.copy(), q.copy()
        qp[i, d] += h
        qm[i, d] -= h
        _, lp = head_forward(qp, k, np.eye(S), scale, True)
        _, lm = head_forward(qm, k, np.eye(S), scale, True)
        fd = (lp[i] - lm[i]) / (2 * h)
        assert fd == pytest.approx(scale * float(p[i] @ k[:, d]), rel=1e-7, abs=1e-9)


# ---------------------------------------------------------- library routine


@pytest.mark.parametrize("S,D", [(1, 8), (7, 4), (33, 16)])
@pytest.mark.parametrize("causal", [True, False])
def test_against_torch_sdpa_float64(S, D, causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(200 + S)
    B, H = 2, 3
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (_rand(rng, B, H, S, D) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do, dtype=torch.float64))
    o, lse = attention_forward(q, k, v, scale, causal)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    scores = scale * torch.tensor(q) @ torch.tensor(k).transpose(-1, -2)
    if causal:
        scores = scores.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(scores, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------- printed numeric cell


def test_accumulator_width_cell():
    with open(os.path.join(GOLDEN, "accumulator_width.json")) as f:
        g = json.load(f)
    D = g["D"]
    q = np.full((1, D), g["q"]["rest"])
    q[0, 0] = g["q"]["first"]
    k = np.full((1, D), g["k"]["rest"])
    k[0, 0] = g["k"]["first"]
    o, lse = head_forward(q, k, np.ones((1, 2)), g["scale"], True)
    assert lse[0] == g["lse"]  # exact: every term and partial sum is a dyadic rational
    assert g["lse_with_narrow_accumulator"] != g["lse"]


# ------------------------------------------------------ grouped key/value heads


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (4, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_against_torch_sdpa_float64(H, Hkv, causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(300 + H + Hkv)
    B, S, D = 2, 9, 4
    scale = 1.0 / np.sqrt(D)
    q, do = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    to.backward(torch.tensor(do, dtype=torch.float64))
    o, lse = gqa_forward(q, k, v, scale, causal)
    dq, dk, dv = gqa_backward(q, k, v, do, scale, causal)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_gqa_repeat_identity_and_index_map():
    """Grouped attention equals per-head attention on K/V repeated G times along the
    head axis (query head h reads key/value head h // G); its dK/dV are the per-head
    gradients summed over each group."""
    rng = np.random.default_rng(31)
    B, H, Hkv, S, D = 2, 6, 2, 7, 5
    G = H // Hkv
    scale = 0.4
    q, do = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse = gqa_forward(q, k, v, scale)
    o_ref, lse_ref = attention_forward(q, kr, vr, scale)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(lse, lse_ref)
    dq, dk, dv = gqa_backward(q, k, v, do, scale)
    dq_ref, dk_ref, dv_ref = attention_backward(q, kr, vr, do, scale)
    np.testing.assert_array_equal(dq, dq_ref)
    np.testing.assert_allclose(dk, dk_ref.reshape(B, Hkv, G, S, D).sum(axis=2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv, dv_ref.reshape(B, Hkv, G, S, D).sum(axis=2), rtol=1e-13, atol=1e-14)
    # a tiled map (h -> h % Hkv) is a different function on these inputs
    o_tiled, _ = attention_forward(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), scale)
    assert np.abs(o_tiled - o).max() > 1e-3


def test_gqa_finite_differences_through_shared_heads():
    rng = np.random.default_rng(32)
    B, H, Hkv, S, D = 1, 4, 2, 5, 3
    scale = 0.6
    q, do = _rand(rng, B, H, S, D), _rand(rng, B, H, S, D)
    k, v = _rand(rng, B, Hkv, S, D), _rand(rng, B, Hkv, S, D)
    dq, dk, dv = gqa_backward(q, k, v, do, scale)

    def loss():
        o, _ = gqa_forward(q, k, v, scale)
        return float((do * o).sum())

    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - g).max() / np.abs(g).max()
        assert err <= 1e-6, (name, err)


def test_gqa_rejects_non_divisible_heads():
    q = np.zeros((1, 5, 3, 2))
    k = np.zeros((1, 2, 3, 2))
    with pytest.raises(ValueError):
        gqa_forward(q, k, k, 1.0)


# ------------------------------------------------------------------- decode


def test_decode_is_last_row_of_causal_attention():
    """The newest position under the causal rule sees every cached key: decode of
    q_{n-1} over rows 0..n-1 is the last row of the (independently pinned) causal
    forward on the same sequence."""
    rng = np.random.default_rng(400)
    for n, D in ((1, 8), (5, 4), (40, 16)):
        q, k, v = (_rand(rng, n, D) for _ in range(3))
        scale = 1.0 / np.sqrt(D)
        o_full, lse_full = head_forward(q, k, v, scale, True)
        o, lse = decode_head(q[-1], k, v, scale)
        np.testing.assert_allclose(o, o_full[-1], rtol=1e-13, atol=1e-14)
        assert abs(lse - lse_full[-1]) < 1e-13


def test_decode_closed_forms():
    rng = np.random.default_rng(401)
    D = 8
    q, k0, v0 = _rand(rng, D), _rand(rng, D), _rand(rng, D)
    # one cached row: o = v_0, lse = scale q.k_0
    o, lse = decode_head(q, k0[None], v0[None], 0.5)
    np.testing.assert_array_equal(o, v0)
    assert lse == pytest.approx(0.5 * q @ k0, abs=1e-15)
    # identical keys: uniform weights, o = mean of the values, lse = s + ln n
    n = 7
    vals = _rand(rng, n, D)
    o, lse = decode_head(q, np.repeat(k0[None], n, axis=0), vals, 0.5)
    np.testing.assert_allclose(o, vals.mean(axis=0), rtol=1e-14, atol=1e-15)
    assert lse == pytest.approx(0.5 * q @ k0 + np.log(n), abs=1e-14)
    # no cached row: o = 0, lse = -inf
    o, lse = decode_head(q, np.zeros((0, D)), np.zeros((0, D)), 0.5)
    np.testing.assert_array_equal(o, np.zeros(D))
    assert lse == -np.inf


def test_decode_ignores_cache_order_and_rows_past_length():
    """No position dependence among visible rows (a consistent permutation of keys
    and values changes nothing), and rows at or past a sequence's length are never
    read (NaN there leaves the result finite and unchanged)."""
    rng = np.random.default_rng(402)
    B, H, Hkv, L, D = 3, 4, 2, 12, 8
    q = _rand(rng, B, H, D)
    k, v = _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    lens = np.array([12, 5, 1])
    o, lse = decode(q, k, v, 0.3, lens)
    perm = rng.permutation(5)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, :5], v2[1, :, :5] = k[1][:, perm], v[1][:, perm]
    k2[1, :, 5:], v2[1, :, 5:] = np.nan, np.nan
    k2[2, :, 1:], v2[2, :, 1:] = np.nan, np.nan
    o2, lse2 = decode(q, k2, v2, 0.3, lens)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)
    # batch entry 2 with one row: its query heads return that row's values
    np.testing.assert_array_equal(o[2, 0], v[2, 0, 0])
    np.testing.assert_array_equal(o[2, 3], v[2, 1, 0])


@pytest.mark.parametrize("H,Hkv", [(4, 2), (6, 1), (4, 4)])
def test_decode_against_torch_sdpa_float64(H, Hkv):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(403 + H * Hkv)
    B, L, D = 2, 11, 8
    scale = 1.0 / np.sqrt(D)
    q = _rand(rng, B, H, D)
    k, v = _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D)
    tq = torch.tensor(q[:, :, None, :])
    to = torch.nn.functional.scaled_dot_product_attention(tq, torch.tensor(k), torch.tensor(v), scale=scale,
                                                          enable_gqa=True)
    o, lse = decode(q, k, v, scale)
    np.testing.assert_allclose(o, to[:, :, 0].numpy(), rtol=1e-12, atol=1e-13)
    G = H // Hkv
    kr = torch.tensor(k).repeat_interleave(G, dim=1)
    ref_lse = torch.logsumexp(scale * (tq @ kr.transpose(-1, -2))[:, :, 0], dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ fp8 Q, K


def test_e4m3_decode_matches_torch_on_every_code():
    """All 256 codes against torch's float8_e4m3fn (an independent implementation
    of the OCP E4M3 format), NaN codes included."""
    torch = pytest.importorskip("torch")
    from oracle import e4m3_decode
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_e4m3_grid_facts():
    """The Rigel paper, §6: the E4M3 grid is the OCP one, 448 is its largest value,
    there is no infinity; 0x7F/0xFF are the only NaNs; sign symmetric; strictly
    increasing over the positive codes; smallest subnormal 2^-9, smallest normal 2^-6."""
    from oracle import e4m3_decode
    v = e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(v)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert not np.isinf(v).any()
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    np.testing.assert_array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert (np.diff(v[0x00:0x7F]) > 0).all()
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0


def test_fp8qk_accumulator_width_cell():
    """Rigel §6's cell through the fp8 oracle: one 448 and 127 terms 0.0625, all E4M3
    values (tests/golden/accumulator_width.json)."""
    import seeded_inputs as si
    from oracle import fp8qk_forward
    with open(os.path.join(GOLDEN, "accumulator_width.json")) as f:
        g = json.load(f)
    D = g["D"]
    q = np.full((1, 1, 1, D), g["q"]["rest"])
    q[..., 0] = g["q"]["first"]
    k = np.full((1, 1, 1, D), g["k"]["rest"])
    k[..., 0] = g["k"]["first"]
    q8, k8 = si.f32_to_e4m3_codes(q), si.f32_to_e4m3_codes(k)
    _, lse = fp8qk_forward(q8, k8, np.ones((1, 1, 1, D)), 1.0, 1.0, g["scale"], True)
    assert lse[0, 0, 0] == g["lse"]


def test_fp8qk_descales_and_grouping():
    """The descale factors multiply the scores (q_descale * k_descale * scale enters
    only as a product), and heads group as in gqa_forward."""
    from oracle import e4m3_decode, fp8qk_forward
    rng = np.random.default_rng(8)
    q8 = rng.integers(0, 0x70, size=(2, 4, 9, 64), dtype=np.uint8) | (rng.integers(0, 2, (2, 4, 9, 64)) << 7).astype(np.uint8)
    k8 = rng.integers(0, 0x70, size=(2, 2, 9, 64), dtype=np.uint8)
    v = rng.standard_normal((2, 2, 9, 64))
    o1, l1 = fp8qk_forward(q8, k8, v, 0.25, 0.5, 0.125, True)
    o2, l2 = fp8qk_forward(q8, k8, v, 1.0, 1.0, 0.125 * 0.125, True)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)
    o3, l3 = gqa_forward(e4m3_decode(q8) * 0.25, e4m3_decode(k8) * 0.5, v, 0.125, True)
    np.testing.assert_array_equal(o1, o3)
    np.testing.assert_array_equal(l1, l3)
