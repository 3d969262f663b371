"""Pins for the backward oracle (oracle.backward), checked against things other
than its own formulas: central differences of the pure-Python brute-force
forward, torch's float64 autodiff of a plain forward written in torch ops, and
closed forms (constant keys, a single visible key, zero gate weight, the
key-sum of dV)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

MODES = ["elementwise", "headwise", "none"]


def draw(rng, B, S, Hq, Hkv, D, dm, mode, extra=0):
    N = Hq * D if mode == "elementwise" else Hq
    return dict(X=rng.standard_normal((B, S, dm)), W=rng.standard_normal((dm, N)) / math.sqrt(dm),
                Q=rng.standard_normal((B, S, Hq, D)), K=rng.standard_normal((B, S + extra, Hkv, D)),
                V=rng.standard_normal((B, S + extra, Hkv, D)), dYg=rng.standard_normal((B, S, Hq, D)))


def brute_loss(t, mode):
    Yg = brute.gated_sdpa(t["X"], t["W"], t["Q"], t["K"], t["V"], mode)
    dY = t["dYg"]
    B, S, Hq, D = dY.shape
    return math.fsum(Yg[b][i][h][d] * dY[b, i, h, d]
                     for b in range(B) for i in range(S) for h in range(Hq) for d in range(D))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(1, 4, 2, 1, 3, 5, 0), (2, 3, 4, 2, 2, 3, 2)])
def test_central_differences_of_brute_forward(mode, shape):
    """Every gradient entry against (L(x+h) - L(x-h)) / 2h with L = Σ dY'·Y'(inputs)."""
    B, S, Hq, Hkv, D, dm, extra = shape
    rng = np.random.default_rng(5 + sum(shape))
    t = draw(rng, B, S, Hq, Hkv, D, dm, mode, extra)
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], mode)
    names = ["Q", "K", "V"] + ([] if mode == "none" else ["X", "W"])
    h = 1e-5
    for name in names:
        arr = t[name]
        g = got["d" + name]
        assert g.shape == arr.shape
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = brute_loss(t, mode)
            arr[idx] = keep - h
            lm = brute_loss(t, mode)
            arr[idx] = keep
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * (1 + abs(fd)), (name, idx, fd, g[idx])


def torch_forward(X, W, Q, K, V, mode):
    """A plain torch statement of the forward (float64, CPU) for autodiff."""
    B, S, Hq, D = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    Kr = K.repeat_interleave(G, dim=2)
    Vr = V.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", Q, Kr) / math.sqrt(D)
    visible = torch.arange(Skv)[None, :] <= (torch.arange(S) + (Skv - S))[:, None]
    s = s.masked_fill(~visible, float("-inf"))
    Y = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), Vr)
    if mode == "none":
        return Y
    g = torch.sigmoid(X @ W)
    g = g.reshape(B, S, Hq, D) if mode == "elementwise" else g.reshape(B, S, Hq, 1)
    return Y * g


@pytest.mark.parametrize("mode", MODES)
def test_matches_torch_float64_autodiff(mode):
    rng = np.random.default_rng(21)
    t = draw(rng, 2, 9, 6, 2, 4, 7, mode, extra=3)
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], mode)
    tt = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k != "dYg")) for k, v in t.items()}
    Yg = torch_forward(tt["X"], tt["W"], tt["Q"], tt["K"], tt["V"], mode)
    (Yg * tt["dYg"]).sum().backward()
    for name in ["Q", "K", "V"] + ([] if mode == "none" else ["X", "W"]):
        want = tt[name].grad.numpy()
        assert np.max(np.abs(got["d" + name] - want)) <= 1e-12 * (1 + np.max(np.abs(want))), name


def test_constant_keys_give_zero_query_gradient():
    """Every row of dS sums to zero, so with all keys equal dQ = Σ_j dS_ij k / √D = 0."""
    rng = np.random.default_rng(3)
    t = draw(rng, 1, 7, 4, 2, 5, 3, "elementwise")
    t["K"][:] = t["K"][:, :1]
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], "elementwise")
    assert np.max(np.abs(got["dQ"])) <= 1e-13


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
def test_key_sum_of_dv_is_gated_upstream_sum(mode):
    """Rows of P sum to one, so Σ_j dV_j = Σ over the group's rows of dY = dY' ⊙ g."""
    rng = np.random.default_rng(8)
    t = draw(rng, 2, 6, 4, 2, 3, 5, mode)
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], mode)
    g = oracle.gate_values(oracle.sigmoid(oracle.gate_scores(t["X"], t["W"])), 4, 3, mode)
    dY = t["dYg"] * g
    want = dY.reshape(2, 6, 2, 2, 3).sum(axis=(1, 3))       # [B, Hkv, D]: rows and the group's heads
    assert np.max(np.abs(got["dV"].sum(axis=1) - want)) <= 1e-12


def test_single_key_passes_gradient_to_value_only():
    """With one token the output is its value row: dV = dY' ⊙ g, dQ = dK = 0."""
    rng = np.random.default_rng(4)
    t = draw(rng, 2, 1, 2, 1, 4, 3, "elementwise")
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], "elementwise")
    g = oracle.gate_values(oracle.sigmoid(oracle.gate_scores(t["X"], t["W"])), 2, 4, "elementwise")
    assert np.max(np.abs(got["dQ"])) == 0.0 and np.max(np.abs(got["dK"])) == 0.0
    assert np.max(np.abs(got["dV"][:, 0, 0] - (t["dYg"] * g)[:, 0].sum(axis=1))) <= 1e-15


def test_zero_gate_weight():
    """W = 0: every gate is 1/2, so dZ = dg/4, dX = 0 and dW = Xᵀ·(dY' ⊙ Y)/4."""
    rng = np.random.default_rng(9)
    t = draw(rng, 1, 5, 2, 2, 3, 4, "elementwise")
    t["W"][:] = 0.0
    got = oracle.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], t["dYg"], "elementwise")
    Y = oracle.sdpa(t["Q"], t["K"], t["V"])
    dg = (t["dYg"] * Y).reshape(5, 6)
    assert np.max(np.abs(got["dX"])) == 0.0
    assert np.max(np.abs(got["dW"] - t["X"][0].T @ dg / 4)) <= 1e-14
    dQ, dK, dV = oracle.sdpa_backward(t["Q"], t["K"], t["V"], t["dYg"] / 2)
    assert np.max(np.abs(got["dV"] - dV)) <= 1e-15


@pytest.mark.parametrize("mode", ["elementwise", "headwise", "none"])
def test_sampled_backward_equals_the_full_one(mode):
    """The sampled form (used at full workload sizes) is the full backward's
    result restricted to the chosen heads, gate columns and rows."""
    rng = np.random.default_rng(31)
    B, S, Hq, Hkv, D, dm = 2, 37, 6, 3, 8, 12
    t = draw(rng, B, S, Hq, Hkv, D, dm, mode)
    X, W, Q, K, V, dY = (t[k] for k in ("X", "W", "Q", "K", "V", "dYg"))
    full = oracle.gated_sdpa_backward(X, W, Q, K, V, dY, mode)
    kv, rows = [2, 0], [0, 5, 36]
    part = oracle.gated_sdpa_backward_sampled(X, W, Q, K, V, dY, mode, kv, rows)
    G = Hq // Hkv
    assert list(part["q_heads"]) == [4, 5, 0, 1]
    np.testing.assert_allclose(part["dQ"], full["dQ"][:, :, part["q_heads"]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dK"], full["dK"][:, :, kv], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dV"], full["dV"][:, :, kv], rtol=1e-12, atol=1e-12)
    if mode == "none":
        assert part["dW"] is None and part["dX"] is None
        return
    per = D if mode == "elementwise" else 1
    assert len(part["w_cols"]) == G * len(kv) * per
    np.testing.assert_allclose(part["dW"], full["dW"][:, part["w_cols"]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(part["dX"], full["dX"][:, rows], rtol=1e-12, atol=1e-12)
