"""Pins of the gating-variant oracle (oracle.variants): brute-force loops,
closed forms of the activations, and invariants between variants."""
import math

import numpy as np
import pytest

import oracle
from oracle import variants as ov


def draw(rng, B, S, Hq, Hkv, D, dm, N):
    return dict(X=rng.standard_normal((B, S, dm)), W=rng.standard_normal((dm, N)) / math.sqrt(dm),
                Q=rng.standard_normal((B, S, Hq, D)), K=rng.standard_normal((B, S, Hkv, D)),
                V=rng.standard_normal((B, S, Hkv, D)))


def sig(z):
    return 1 / (1 + math.exp(-z)) if z >= 0 else math.exp(z) / (1 + math.exp(z))


def brute_variant(t, mode, act, combine, norm):
    """Pure-Python loops: SDPA row, optional RMSNorm, activation, combine.
    K and V may hold Skv >= S keys: query i then sits at position i + Skv - S
    (a decode step has S = 1 and sees every cached key)."""
    X, W, Q, K, V = (t[k] for k in "XWQKV")
    B, S, Hq, D = Q.shape
    G = Hq // K.shape[2]
    off = K.shape[1] - S
    dm = X.shape[2]
    f = {"identity": lambda z: z, "sigmoid": sig, "ns_sigmoid": lambda z: 0.5 + 0.5 * sig(z),
         "silu": lambda z: z * sig(z)}[act]
    out = np.empty(Q.shape)
    for b in range(B):
        for i in range(S):
            for h in range(Hq):
                c = h // G
                s = [math.fsum(Q[b, i, h, d] * K[b, j, c, d] for d in range(D)) / math.sqrt(D)
                     for j in range(i + off + 1)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                y = [math.fsum(w[j] * V[b, j, c, d] for j in range(i + off + 1)) / tot for d in range(D)]
                if norm == "rms":
                    r = math.sqrt(math.fsum(v * v for v in y) / D + ov.RMS_EPS)
                    y = [v / r for v in y]
                for d in range(D):
                    if mode == "none":
                        out[b, i, h, d] = y[d]
                        continue
                    if mode == "shared":
                        # every head's activated score for dim d, averaged over the heads
                        g = math.fsum(f(math.fsum(X[b, i, k] * W[k, hh * D + d] for k in range(dm)))
                                      for hh in range(Hq)) / Hq
                    else:
                        col = {"elementwise": h * D + d, "headwise": h}[mode]
                        g = f(math.fsum(X[b, i, k] * W[k, col] for k in range(dm)))
                    out[b, i, h, d] = y[d] * g if combine == "mul" else y[d] + g
    return out


CASES = [("elementwise", "ns_sigmoid", "mul", None), ("headwise", "sigmoid", "add", None),
         ("elementwise", "silu", "add", None), ("shared", "sigmoid", "mul", None),
         ("none", "sigmoid", "mul", "rms"), ("elementwise", "sigmoid", "mul", "rms"),
         ("shared", "identity", "add", "rms"), ("headwise", "ns_sigmoid", "mul", "rms")]


@pytest.mark.parametrize("mode,act,combine,norm", CASES)
def test_matches_brute_force(mode, act, combine, norm):
    B, S, Hq, Hkv, D, dm = 2, 5, 4, 2, 3, 4
    N = {"elementwise": Hq * D, "headwise": Hq, "shared": Hq * D, "none": 1}[mode]
    t = draw(np.random.default_rng(len(mode) + len(act)), B, S, Hq, Hkv, D, dm, N)
    got = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], mode, act, combine, norm)
    assert np.max(np.abs(got - brute_variant(t, mode, act, combine, norm))) <= 1e-12


@pytest.mark.parametrize("mode,act,combine,norm", CASES)
def test_decode_shape_matches_brute_force(mode, act, combine, norm):
    """The same variants for one decode step: a single query per batch against a
    cache of L keys that holds it (the gate at the decode merge)."""
    B, L, Hq, Hkv, D, dm = 3, 7, 4, 2, 3, 4
    N = {"elementwise": Hq * D, "headwise": Hq, "shared": Hq * D, "none": 1}[mode]
    rng = np.random.default_rng(7 + len(mode) + len(act))
    t = draw(rng, B, L, Hq, Hkv, D, dm, N)
    t["X"], t["Q"] = t["X"][:, -1:], t["Q"][:, -1:]          # the newest token queries the cache
    got = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], mode, act, combine, norm)
    assert got.shape == (B, 1, Hq, D)
    assert np.max(np.abs(got - brute_variant(t, mode, act, combine, norm))) <= 1e-12


def test_default_decode_variant_is_the_decode_oracle_bitwise():
    rng = np.random.default_rng(11)
    for mode, N in (("elementwise", 4 * 3), ("headwise", 4)):
        t = draw(rng, 2, 9, 4, 2, 3, 5, N)
        t["X"], t["Q"] = t["X"][:, -1:], t["Q"][:, -1:]
        got = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], mode)
        want = oracle.gated_decode(t["X"], t["W"], t["Q"], t["K"], t["V"], mode)
        assert np.array_equal(got, want), mode


def test_activation_closed_forms():
    z = np.array([-40.0, -1.0, 0.0, 1.0, 40.0])
    assert np.array_equal(ov.activation(z, "identity"), z)
    ns = ov.activation(z, "ns_sigmoid")
    assert ns[2] == 0.75 and ns[4] == 1.0 and abs(ns[0] - 0.5) <= 1e-17 and np.all((ns >= 0.5) & (ns <= 1))
    si = ov.activation(z, "silu")
    assert si[2] == 0.0 and si[4] == 40.0 and abs(si[0]) <= 40 * math.exp(-40) * 1.0001
    assert abs(si[3] - 1 / (1 + math.exp(-1))) <= 1e-16 and abs(si[1] + math.exp(-1) / (1 + math.exp(-1))) <= 1e-16


def test_default_variant_is_the_g1_oracle_bitwise():
    t = draw(np.random.default_rng(1), 2, 9, 4, 2, 4, 6, 16)
    a = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], "elementwise")
    b = oracle.gated_sdpa(t["X"], t["W"], t["Q"], t["K"], t["V"], "elementwise")
    assert np.array_equal(a, b)


def test_shared_equals_elementwise_when_heads_share_weights():
    """With the same weight block for every head, all heads' scores are equal, so
    their mean is that score: head-shared == elementwise."""
    rng = np.random.default_rng(2)
    Hq, D = 4, 4
    t = draw(rng, 1, 11, Hq, 2, D, 6, D)
    Wt = np.tile(t["W"], (1, Hq))                        # column h*D + d = column d, every head
    a = ov.gated_sdpa_variant(t["X"], Wt, t["Q"], t["K"], t["V"], "shared", "ns_sigmoid", "add")
    b = ov.gated_sdpa_variant(t["X"], Wt, t["Q"], t["K"], t["V"], "elementwise", "ns_sigmoid", "add")
    assert np.max(np.abs(a - b)) <= 1e-15


def test_shared_averages_activated_scores_not_logits():
    """Two heads whose logits for a dimension are 4 and 0: the shared gate is
    (σ(4) + σ(0)) / 2 = 0.7410..., not σ((4 + 0) / 2) = σ(2) = 0.8807...
    (the mean of the activated scores, "GatedAttention [2025]" §1.3.2 (ii))."""
    B, S, Hq, Hkv, D, dm = 1, 1, 2, 1, 1, 1
    X = np.ones((B, S, dm))
    W = np.array([[4.0, 0.0]])                            # head 0 logit 4, head 1 logit 0
    Q = np.zeros((B, S, Hq, D)); K = np.zeros((B, S, Hkv, D)); V = np.ones((B, S, Hkv, D))
    got = ov.gated_sdpa_variant(X, W, Q, K, V, "shared")  # Y = V = 1, so Y' is the gate
    want = (1 / (1 + math.exp(-4.0)) + 0.5) / 2
    assert abs(got[0, 0, 0, 0] - want) <= 1e-16 and abs(got[0, 0, 1, 0] - want) <= 1e-16
    assert abs(want - 1 / (1 + math.exp(-2.0))) > 0.1
    # with the identity activation the two readings coincide: the gate is the mean logit
    got_id = ov.gated_sdpa_variant(X, W, Q, K, V, "shared", "identity")
    assert got_id[0, 0, 0, 0] == 2.0


def test_additive_with_zero_weight():
    t = draw(np.random.default_rng(3), 1, 7, 2, 1, 4, 5, 8)
    t["W"][:] = 0.0
    Y = oracle.sdpa(t["Q"], t["K"], t["V"])
    for act, const in [("sigmoid", 0.5), ("silu", 0.0), ("identity", 0.0), ("ns_sigmoid", 0.75)]:
        got = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], "elementwise", act, "add")
        assert np.array_equal(got, Y + const), act


def test_rms_norm_gives_unit_rms_and_is_scale_free():
    t = draw(np.random.default_rng(4), 2, 13, 4, 2, 8, 6, 1)
    Yn = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], "none", norm="rms")
    Y = oracle.sdpa(t["Q"], t["K"], t["V"])
    ms = np.mean(Y * Y, axis=-1)
    rms = np.sqrt(np.mean(Yn * Yn, axis=-1))
    assert np.max(np.abs(rms - np.sqrt(ms / (ms + ov.RMS_EPS)))) <= 1e-12 and np.all(rms <= 1)
    Yn4 = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], 4 * t["V"], "none", norm="rms")
    # only ε breaks scale freedom: the two differ by a factor within 1 ± ε/(2·ms)
    bound = np.abs(Yn) * (ov.RMS_EPS / (2 * ms))[..., None] * 1.001 + 1e-15
    assert np.all(np.abs(Yn4 - Yn) <= bound)
    assert np.array_equal(np.sign(Yn), np.sign(Y))


def test_value_gate_g2():
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D, dm = 2, 10, 4, 2, 3, 5
    t = draw(rng, B, S, Hq, Hkv, D, dm, Hkv * D)
    Y = oracle.sdpa(t["Q"], t["K"], t["V"])
    Wsat = np.zeros((dm, Hkv * D))
    Xsat = np.zeros((B, S, dm))
    Xsat[..., 0] = 1.0
    Wsat[0, :] = 40.0                                    # logits +40: σ == 1.0 exactly
    assert np.array_equal(ov.value_gated_sdpa(Xsat, Wsat, t["Q"], t["K"], t["V"], "elementwise"), Y)
    W0 = np.zeros((dm, Hkv))                             # headwise, σ(0) = 1/2: SDPA is linear in V
    assert np.max(np.abs(ov.value_gated_sdpa(t["X"], W0, t["Q"], t["K"], t["V"], "headwise") - Y / 2)) <= 1e-15
    # brute force: gate each value row, then attend
    got = ov.value_gated_sdpa(t["X"], t["W"], t["Q"], t["K"], t["V"], "elementwise")
    Vg = np.empty_like(t["V"])
    for b in range(B):
        for j in range(S):
            for c in range(Hkv):
                for d in range(D):
                    z = math.fsum(t["X"][b, j, k] * t["W"][k, c * D + d] for k in range(dm))
                    Vg[b, j, c, d] = t["V"][b, j, c, d] * sig(z)
    assert np.max(np.abs(got - oracle.sdpa(t["Q"], t["K"], Vg))) <= 1e-14


def test_rows_subset_equals_full():
    t = draw(np.random.default_rng(9), 2, 30, 4, 2, 4, 6, 16)
    full = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], "shared", "silu", "add", "rms")
    rows = [0, 7, 29]
    part = ov.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], "shared", "silu", "add", "rms", rows=rows)
    assert np.array_equal(part, full[:, rows])
