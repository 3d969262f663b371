"""Pins for the fp64 oracle, against things other than itself.

Each test names what fixes the expected value: brute-force loops on tiny
inputs, a library SDPA in float64, closed forms, invariants the pages state,
and the parameter counts the pages print.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import variants
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B, S, Hq, Hkv, D, dm, mode, Skv=None, wscale=None):
    Skv = S if Skv is None else Skv
    N = Hq * D if mode == "elementwise" else Hq
    X = rng.standard_normal((B, S, dm))
    W = rng.standard_normal((dm, N)) * (wscale if wscale is not None else 1 / math.sqrt(dm))
    Q = rng.standard_normal((B, S, Hq, D))
    K = rng.standard_normal((B, Skv, Hkv, D))
    V = rng.standard_normal((B, Skv, Hkv, D))
    return X, W, Q, K, V


def torch_sdpa_f64(Q, K, V):
    """torch's scaled_dot_product_attention on the CPU in float64, GQA by
    repeating each key/value head over its group of query heads."""
    B, S, Hq, D = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)
    k = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    v = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    if S == Skv:
        y = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    else:
        assert S == 1   # a single query at the last position sees every key
        y = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    return y.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------- brute force
TINY = []
_r = np.random.default_rng(1234)
for _ in range(24):
    Hkv = int(_r.choice([1, 2]))
    G = int(_r.choice([1, 2, 4]))
    TINY.append(dict(B=int(_r.integers(1, 3)), S=int(_r.choice([1, 2, 3, 5, 7, 9])),
                     Hq=Hkv * G, Hkv=Hkv, D=int(_r.choice([1, 2, 4])), dm=int(_r.choice([1, 3, 6])),
                     mode=str(_r.choice(["elementwise", "headwise", "none"])),
                     extra_kv=int(_r.choice([0, 0, 3]))))


@pytest.mark.parametrize("case", TINY, ids=[str(i) for i in range(len(TINY))])
def test_oracle_matches_brute_force(case):
    rng = np.random.default_rng(hash(str(case)) % (2 ** 32))
    mode = case["mode"]
    gmode = mode if mode != "none" else "elementwise"
    Skv = case["S"] + case["extra_kv"]
    X, W, Q, K, V = rand_case(rng, case["B"], case["S"], case["Hq"], case["Hkv"], case["D"],
                              case["dm"], gmode, Skv=Skv, wscale=1.0)
    got = oracle.gated_sdpa(X, W, Q, K, V, mode)
    want = np.array(brute.gated_sdpa(X, W, Q, K, V, mode))
    assert got.shape == want.shape
    assert np.max(np.abs(got - want)) <= 1e-12


def test_gate_scores_match_brute_force():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 5, 6))
    W = rng.standard_normal((6, 7))
    Z = oracle.gate_scores(X, W)
    for b in range(3):
        for i in range(5):
            for n in range(7):
                ref = math.fsum(X[b, i, k] * W[k, n] for k in range(6))
                assert abs(Z[b, i, n] - ref) <= 1e-13


def test_sigmoid_closed_forms():
    z = np.array([0.0, 40.0, -40.0, 1.0, -1.0, 800.0, -800.0])
    g = oracle.sigmoid(z)
    assert g[0] == 0.5
    assert g[1] == 1.0                      # e^-40 ~ 4.2e-18 is below half an ulp of 1.0
    assert abs(g[2] - math.exp(-40.0)) <= 1e-30
    assert abs(g[3] - 1 / (1 + math.exp(-1))) <= 1e-16
    assert abs(g[3] + g[4] - 1.0) <= 1e-16   # sigma(z) + sigma(-z) = 1
    assert g[5] == 1.0 and g[6] == 0.0 and np.all(np.isfinite(g))


# ------------------------------------------------------- library SDPA pin
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 1, 1, 1, 8), (2, 17, 4, 4, 16), (1, 33, 8, 2, 32),
                                            (2, 70, 6, 1, 8), (1, 600, 4, 2, 16)])
def test_sdpa_matches_torch_float64(B, S, Hq, Hkv, D):
    rng = np.random.default_rng(S)
    _, _, Q, K, V = rand_case(rng, B, S, Hq, Hkv, D, 4, "headwise")
    Y = oracle.sdpa(Q, K, V)
    assert np.max(np.abs(Y - torch_sdpa_f64(Q, K, V))) <= 1e-12


def test_decode_matches_torch_float64():
    rng = np.random.default_rng(5)
    _, _, Q, K, V = rand_case(rng, 3, 1, 8, 2, 16, 4, "headwise", Skv=300)
    Y = oracle.sdpa(Q, K, V)
    assert np.max(np.abs(Y - torch_sdpa_f64(Q, K, V))) <= 1e-12


# ------------------------------------------------------- gate closed forms
def _case(seed=3, B=2, S=40, Hq=4, Hkv=2, D=8, dm=6, mode="elementwise"):
    return rand_case(np.random.default_rng(seed), B, S, Hq, Hkv, D, dm, mode)


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
def test_saturated_gate_is_plain_sdpa(mode):
    X, W, Q, K, V = _case(mode=mode)
    W[:] = 0.0
    W[0, :] = 1.0
    X[..., 0] = 40.0                     # every gate logit is exactly 40, sigma(40) == 1.0
    Yg = oracle.gated_sdpa(X, W, Q, K, V, mode)
    Y = oracle.gated_sdpa(X, W, Q, K, V, "none")
    assert np.array_equal(Yg, Y)
    assert np.max(np.abs(Yg - torch_sdpa_f64(Q, K, V))) <= 1e-12


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
def test_zero_gate_weight_halves_output(mode):
    X, W, Q, K, V = _case(mode=mode)
    W[:] = 0.0                            # sigma(0) = 1/2 exactly
    Yg = oracle.gated_sdpa(X, W, Q, K, V, mode)
    Y = oracle.gated_sdpa(X, W, Q, K, V, "none")
    assert np.array_equal(Yg, Y / 2)


def test_negative_saturation_closes_gate():
    X, W, Q, K, V = _case()
    W[:] = 0.0
    W[0, :] = 1.0
    X[..., 0] = -40.0
    Yg = oracle.gated_sdpa(X, W, Q, K, V, "elementwise")
    Y = oracle.gated_sdpa(X, W, Q, K, V, "none")
    assert np.all(np.abs(Yg) <= 5e-18 * np.abs(Y))


def test_headwise_equals_elementwise_with_broadcast_columns():
    X, Wh, Q, K, V = _case(mode="headwise")
    Hq, D = Q.shape[2], Q.shape[3]
    We = np.repeat(Wh, D, axis=1)         # column h*D + d copies headwise column h
    Yh = oracle.gated_sdpa(X, Wh, Q, K, V, "headwise")
    Ye = oracle.gated_sdpa(X, We, Q, K, V, "elementwise")
    assert np.max(np.abs(Yh - Ye)) <= 1e-15
    # brute force evaluates each column with an exactly rounded sum: bit-identical
    Xs, Whs, Qs, Ks, Vs = (a[:1, :6] if a.ndim > 2 else a for a in (X, Wh, Q, K, V))
    Wes = np.repeat(Whs, D, axis=1)
    assert brute.gated_sdpa(Xs, Whs, Qs, Ks, Vs, "headwise") == brute.gated_sdpa(Xs, Wes, Qs, Ks, Vs, "elementwise")


def test_elementwise_gate_column_layout():
    """Gate column h*D + d multiplies head h, dim d (the [.., n_h, d_h] view)."""
    X, W, Q, K, V = _case(Hq=3, Hkv=3, D=4)
    Hq, D = 3, 4
    Y = oracle.sdpa(Q, K, V)
    Yg, g = oracle.gated_sdpa(X, W, Q, K, V, "elementwise", return_gate=True)
    for h in range(Hq):
        for d in range(D):
            assert np.array_equal(Yg[:, :, h, d], Y[:, :, h, d] * g[:, :, h * D + d])


# ------------------------------------------------------- softmax invariants
def test_softmax_rows_sum_to_one_and_mask_is_exact():
    _, _, Q, K, V = _case(S=37)
    Y, lse, P = oracle.sdpa(Q, K, V, return_lse=True, return_probs=True)
    S = Q.shape[1]
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-13
    assert np.all(P >= 0)
    upper = np.triu(np.ones((S, S), dtype=bool), k=1)
    assert np.all(P[..., upper] == 0.0)
    # lse is consistent with the probabilities of key 0: P[i,0] = exp(s_i0 - lse_i)
    B, _, Hq, D = Q.shape
    G = Hq // K.shape[2]
    for h in range(Hq):
        s0 = np.einsum("bid,bd->bi", Q[:, :, h], K[:, 0, h // G]) / math.sqrt(D)
        assert np.max(np.abs(np.exp(s0 - lse[:, h]) - P[:, h, :, 0])) <= 1e-13


def test_row_zero_is_first_value_times_gate():
    X, W, Q, K, V = _case()
    Yg, g = oracle.gated_sdpa(X, W, Q, K, V, "elementwise", return_gate=True)
    B, S, Hq, D = Q.shape
    G = Hq // K.shape[2]
    for h in range(Hq):
        assert np.array_equal(Yg[:, 0, h, :], V[:, 0, h // G, :] * g[:, 0, h * D:(h + 1) * D])


def test_zero_queries_give_prefix_means():
    _, _, Q, K, V = _case(S=50)
    Q[:] = 0.0                                   # every score 0 -> uniform weights over the prefix
    Y = oracle.sdpa(Q, K, V)
    G = Q.shape[2] // K.shape[2]
    cnt = np.arange(1, Q.shape[1] + 1)[None, :, None, None]
    mean = np.cumsum(V, axis=1) / cnt
    assert np.max(np.abs(Y - np.repeat(mean, G, axis=2))) <= 1e-12


@pytest.mark.parametrize("i0", [0, 5, 31, 48])
def test_future_keys_do_not_change_earlier_rows(i0):
    X, W, Q, K, V = _case(S=50)
    Y1 = oracle.gated_sdpa(X, W, Q, K, V, "elementwise")
    K2, V2 = K.copy(), V.copy()
    sgn = np.where(np.random.default_rng(0).random(K[:, i0 + 1:].shape) < 0.5, -1.0, 1.0)
    K2[:, i0 + 1:] = 1e4 * sgn
    V2[:, i0 + 1:] = -1e4 * sgn
    Y2 = oracle.gated_sdpa(X, W, Q, K2, V2, "elementwise")
    assert np.array_equal(Y1[:, :i0 + 1], Y2[:, :i0 + 1])
    if i0 + 1 < Q.shape[1]:
        assert not np.allclose(Y1[:, i0 + 1:], Y2[:, i0 + 1:])


def test_gqa_equals_mha_with_repeated_kv():
    X, W, Q, K, V = _case(Hq=8, Hkv=2)
    G = 4
    Yg = oracle.gated_sdpa(X, W, Q, K, V, "elementwise")
    Ym = oracle.gated_sdpa(X, W, Q, np.repeat(K, G, axis=2), np.repeat(V, G, axis=2), "elementwise")
    assert np.max(np.abs(Yg - Ym)) <= 1e-15


def test_rows_subset_matches_full():
    X, W, Q, K, V = _case(S=40)
    full = oracle.gated_sdpa(X, W, Q, K, V, "elementwise")
    rows = np.array([0, 1, 17, 39])
    part = oracle.gated_sdpa(X, W, Q, K, V, "elementwise", rows=rows)
    assert np.max(np.abs(full[:, rows] - part[:, rows])) <= 1e-14
    assert np.all(np.isnan(np.delete(part, rows, axis=1)))


def test_decode_is_last_row_of_prefill():
    X, W, Q, K, V = _case(S=33)
    full = oracle.gated_sdpa(X, W, Q, K, V, "elementwise")
    dec = oracle.gated_decode(X[:, -1:], W, Q[:, -1:], K, V, "elementwise")
    assert np.max(np.abs(full[:, -1:] - dec)) <= 1e-14


# ------------------------------------------------------- printed numbers
def test_gate_param_counts_match_table1():
    with open(os.path.join(GOLDEN, "gate_params_table1.json")) as f:
        gold = json.load(f)
    a = gold["architecture_inferred"]
    Lyr, dm, q, k, dk = a["layers"], a["d_model"], a["q_heads"], a["kv_heads"], a["d_k"]
    computed = {
        5: Lyr * oracle.gate_param_count(dm, q, dk, "elementwise"),
        6: Lyr * dm * k * dk,
        7: Lyr * dm * k * dk,
        8: Lyr * dm * q * dk,
        9: Lyr * dm * dm,
        10: Lyr * oracle.gate_param_count(dm, q, dk, "headwise"),
        11: Lyr * dm * k,
        # head-shared: the width the variants oracle's layout consumes (the n×q×d_k
        # scores it then averages over the q heads)
        12: Lyr * dm * variants.gate_width("shared", q, dk),
    }
    # that layout turns a score row of this width into one n×d_k gate for all heads
    assert variants.gate_layout(np.zeros((1, 1, variants.gate_width("shared", q, dk))), q, dk,
                                "shared").shape == (1, 1, 1, dk)
    assert variants.gate_width("elementwise", q, dk) * dm == oracle.gate_param_count(dm, q, dk, "elementwise")
    assert variants.gate_width("headwise", q, dk) * dm == oracle.gate_param_count(dm, q, dk, "headwise")
    for row in gold["rows"]:
        printed = row["params_M"]
        unit = 1.0 if float(printed).is_integer() else 0.1
        assert abs(computed[row["row"]] / 1e6 - printed) <= unit, row
    # "1/125 of elementwise": the ratio of the two G1 widths is d_k
    assert computed[5] / computed[10] == dk
    assert abs(201 / 1.6 - 125) < 1.0
