"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each.

The mutation is textual, applied to the oracle's source in memory; the mutated
copy is loaded as a throwaway module.  The real oracle is never modified.
"""
import importlib.util
import math
import os
import types

import numpy as np
import pytest

from oracle import brute

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gated_sdpa.py")

MUTANTS = {
    "scale_1_over_D": ("scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
    "gqa_interleaved": ("heads = np.arange(c * G, (c + 1) * G)", "heads = np.arange(c, Hq, Hkv)"),
    "mask_excludes_self": ("<= pos[:, None]", "< pos[:, None]"),
    "mask_top_left": ("pos = r + off", "pos = r"),
    "gate_columns_transposed": ("return g.reshape(B, S, Hq, D)", "return g.reshape(B, S, D, Hq).transpose(0, 1, 3, 2)"),
    "sigmoid_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-Z[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(Z[pos]))"),
    "no_normalisation": ("P = p / l ", "P = p "),
    "first_kv_head_only": ("Kc = K[b, :, c, :]", "Kc = K[b, :, 0, :]"),
    "keys_as_values": ("y = P @ Vc[:n_keys]", "y = P @ Kc[:n_keys]"),
    "last_key_dropped": ("n_keys = int(pos.max()) + 1", "n_keys = int(pos.max())"),
    "gate_weight_transposed": ("return X @ W\n", "return X @ W.T\n"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def pins_pass(orc):
    """A compact run of the pins from test_oracle.py against an oracle module."""
    rng = np.random.default_rng(11)
    try:
        for (B, S, Hq, Hkv, D, dm, extra, mode) in [(1, 5, 4, 2, 3, 3, 0, "elementwise"),
                                                    (2, 4, 2, 1, 2, 2, 3, "headwise"),
                                                    (1, 6, 3, 3, 2, 6, 0, "elementwise")]:
            N = Hq * D if mode == "elementwise" else Hq
            X = rng.standard_normal((B, S, dm))
            W = rng.standard_normal((dm, N))
            Q = rng.standard_normal((B, S, Hq, D))
            K = rng.standard_normal((B, S + extra, Hkv, D))
            V = rng.standard_normal((B, S + extra, Hkv, D))
            got = orc.gated_sdpa(X, W, Q, K, V, mode)
            want = np.array(brute.gated_sdpa(X, W, Q, K, V, mode))
            if got.shape != want.shape or not np.max(np.abs(got - want)) <= 1e-12:
                return False
    except Exception:
        return False
    return True


def test_unmutated_copy_passes():
    with open(SRC) as f:
        src = f.read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    assert pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not pins_pass(load_mutant(name))


# ---------------------------------------------------------------- backward oracle
BWD_SRC = os.path.join(os.path.dirname(SRC), "backward.py")

BWD_MUTANTS = {
    "sigmoid_derivative_dropped": ("    dZ = dg * g * (1.0 - g)                        #", "    dZ = dg * g  #"),
    "softmax_row_term_dropped": ("dS = P * (dP - (dP * P).sum(axis=-1, keepdims=True))", "dS = P * dP"),
    "dk_unscaled": ("dK[b, :, c, :] += (dS.T @ q) * scale", "dK[b, :, c, :] += dS.T @ q"),
    "dq_uses_values": ("dQ[b, :, h, :] = (dS @ Kc) * scale", "dQ[b, :, h, :] = (dS @ Vc) * scale"),
    "dv_untransposed_probs": ("dV[b, :, c, :] += P.T @ dy", "dV[b, :, c, :] += P @ dy"),
    "upstream_not_gated": ("dY = dYg * gv ", "dY = dYg "),
    "gate_grad_uses_gated_output": ("dgv = dYg * Y ", "dgv = dYg * Y * gv "),
    "headwise_mean_not_sum": ("dg = dgv.sum(axis=-1)                      # one gate",
                              "dg = dgv.mean(axis=-1)  # one gate"),
    "gqa_interleaved": ("c = h // G", "c = h % Hkv"),
    "dw_not_summed_over_batch": ("dW = X.reshape(B * S, -1).T @ dZ.reshape(B * S, -1)", "dW = X[0].T @ dZ[0]"),
    "bwd_mask_excludes_self": ("<= (np.arange(S) + off)[:, None]", "< (np.arange(S) + off)[:, None]"),
}


def load_bwd_mutant(name):
    with open(BWD_SRC) as f:
        src = f.read().replace("from .gated_sdpa import", "from oracle.gated_sdpa import")
    if name is not None:
        old, new = BWD_MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_bwd_mutant_{name}")
    exec(compile(src, f"<bwd mutant {name}>", "exec"), mod.__dict__)
    return mod


def bwd_pins_pass(orc):
    """Central differences of the brute-force forward on tiny shapes, every mode."""
    rng = np.random.default_rng(17)
    h = 1e-5
    try:
        for (B, S, Hq, Hkv, D, dm, mode) in [(2, 3, 4, 2, 2, 3, "elementwise"),
                                             (2, 3, 4, 2, 2, 3, "headwise")]:
            N = Hq * D if mode == "elementwise" else Hq
            t = dict(X=rng.standard_normal((B, S, dm)), W=rng.standard_normal((dm, N)),
                     Q=rng.standard_normal((B, S, Hq, D)), K=rng.standard_normal((B, S, Hkv, D)),
                     V=rng.standard_normal((B, S, Hkv, D)))
            dYg = rng.standard_normal((B, S, Hq, D))
            got = orc.gated_sdpa_backward(t["X"], t["W"], t["Q"], t["K"], t["V"], dYg, mode)

            def loss():
                Yg = np.array(brute.gated_sdpa(t["X"], t["W"], t["Q"], t["K"], t["V"], mode))
                return math.fsum((Yg * dYg).ravel())
            for name in ("Q", "K", "V", "X", "W"):
                arr = t[name]
                for idx in np.ndindex(arr.shape):
                    keep = arr[idx]
                    arr[idx] = keep + h
                    lp = loss()
                    arr[idx] = keep - h
                    lm = loss()
                    arr[idx] = keep
                    if not abs((lp - lm) / (2 * h) - got["d" + name][idx]) <= 1e-6:
                        return False
    except Exception:
        return False
    return True


def test_unmutated_backward_copy_passes():
    assert bwd_pins_pass(load_bwd_mutant(None))


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    assert not bwd_pins_pass(load_bwd_mutant(name))


# --------------------------------------------------------------- first-token attention
DIAG_SRC = os.path.join(os.path.dirname(SRC), "diagnostics.py")
DIAG_MUTANTS = {
    "fattn_unscaled": ("/ np.sqrt(D)", ""),
    "fattn_interleaved_gqa": ("K[:, 0, h // G, :]", "K[:, 0, h % Hkv, :]"),
    "fattn_last_key": ("K[:, 0, h // G, :]", "K[:, -1, h // G, :]"),
    "fattn_log_not_exp": ("np.exp(s0 - lse[:, h, r])", "(s0 - lse[:, h, r])"),
    "fattn_mean_over_heads_only": ("F.mean(axis=(0, 2))", "F.mean(axis=(0, 1))[:Hq]"),
}


def load_diag_mutant(name):
    with open(DIAG_SRC) as f:
        src = f.read().replace("from .gated_sdpa import", "from oracle.gated_sdpa import")
    if name is not None:
        old, new = DIAG_MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_diag_mutant_{name}")
    exec(compile(src, f"<diag mutant {name}>", "exec"), mod.__dict__)
    return mod


def diag_pins_pass(orc):
    """Brute-force loops on a tiny GQA shape (per-row shares and per-head means)."""
    rng = np.random.default_rng(23)
    B, S, Hq, Hkv, D = 2, 7, 4, 2, 3
    Q, K, V = (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)),
               rng.standard_normal((B, S, Hkv, D)))
    try:
        F, head_mean, mean = orc.first_token_attention(Q, K, V)
    except Exception:
        return False
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                s = [math.fsum(Q[b, i, h, d] * K[b, j, h // G, d] for d in range(D)) / math.sqrt(D)
                     for j in range(i + 1)]
                want = math.exp(s[0]) / math.fsum(math.exp(x) for x in s)
                if not abs(F[b, h, i] - want) <= 1e-12:
                    return False
    want_h = [math.fsum(F[b, h, i] for b in range(B) for i in range(S)) / (B * S) for h in range(Hq)]
    return (np.shape(head_mean) == (Hq,) and np.allclose(head_mean, want_h, rtol=0, atol=1e-14)
            and abs(mean - math.fsum(want_h) / Hq) <= 1e-14)


def test_unmutated_diagnostics_copy_passes():
    assert diag_pins_pass(load_diag_mutant(None))


@pytest.mark.parametrize("name", sorted(DIAG_MUTANTS))
def test_diagnostics_mutant_is_caught(name):
    assert not diag_pins_pass(load_diag_mutant(name))


# --------------------------------------------------------------- fused input projection
PROJ_SRC = os.path.join(os.path.dirname(SRC), "projection.py")
PROJ_MUTANTS = {
    "proj_heads_transposed": ("np.asarray(Wq, dtype=np.float64)).reshape(B, S, Hq, D)",
                              "np.asarray(Wq, dtype=np.float64)).reshape(B, S, D, Hq).transpose(0, 1, 3, 2)"),
    "proj_keys_from_values": ("K = (X @ np.asarray(Wk,", "K = (X @ np.asarray(Wv,"),
    "proj_gate_without_sigmoid": ("G = None if W is None else sigmoid(gate_scores(X, W))",
                                  "G = None if W is None else gate_scores(X, W)"),
    "proj_weights_transposed": ("V = (X @ np.asarray(Wv, dtype=np.float64))",
                                "V = (X @ np.asarray(Wv, dtype=np.float64).T.T[:, ::-1])"),
}


def load_proj_mutant(name):
    with open(PROJ_SRC) as f:
        src = f.read().replace("from .gated_sdpa import", "from oracle.gated_sdpa import")
    if name is not None:
        old, new = PROJ_MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_proj_mutant_{name}")
    exec(compile(src, f"<proj mutant {name}>", "exec"), mod.__dict__)
    return mod


def proj_pins_pass(orc):
    """Brute-force loops on a tiny GQA shape."""
    rng = np.random.default_rng(29)
    B, S, dm, Hq, Hkv, D, N = 2, 3, 5, 4, 2, 3, 6
    X = rng.standard_normal((B, S, dm))
    Wq, Wk, Wv, W = (rng.standard_normal((dm, w)) for w in (Hq * D, Hkv * D, Hkv * D, N))
    try:
        Q, K, V, G = orc.project_qkvg(X, Wq, Wk, Wv, W, Hq, Hkv, D)
    except Exception:
        return False
    for b in range(B):
        for i in range(S):
            for h in range(Hq):
                for d in range(D):
                    if abs(Q[b, i, h, d] - math.fsum(X[b, i, k] * Wq[k, h * D + d] for k in range(dm))) > 1e-12:
                        return False
            for c in range(Hkv):
                for d in range(D):
                    if abs(K[b, i, c, d] - math.fsum(X[b, i, k] * Wk[k, c * D + d] for k in range(dm))) > 1e-12:
                        return False
                    if abs(V[b, i, c, d] - math.fsum(X[b, i, k] * Wv[k, c * D + d] for k in range(dm))) > 1e-12:
                        return False
            for n in range(N):
                z = math.fsum(X[b, i, k] * W[k, n] for k in range(dm))
                if abs(G[b, i, n] - 1 / (1 + math.exp(-z))) > 1e-14:
                    return False
    return True


def test_unmutated_projection_copy_passes():
    assert proj_pins_pass(load_proj_mutant(None))


@pytest.mark.parametrize("name", sorted(PROJ_MUTANTS))
def test_projection_mutant_is_caught(name):
    assert not proj_pins_pass(load_proj_mutant(name))


# --------------------------------------------------------------- gating variants
VAR_SRC = os.path.join(os.path.dirname(SRC), "variants.py")
VAR_MUTANTS = {
    "ns_sigmoid_half_only": ("return 0.5 + 0.5 * sigmoid(Z)", "return 0.5 * sigmoid(Z)"),
    "silu_without_input": ("return Z * sigmoid(Z)", "return sigmoid(Z)"),
    "shared_over_dims_not_heads": ("return a.reshape(B, S, Hq, D).sum(axis=2, keepdims=True) / Hq",
                                   "return a.reshape(B, S, Hq, D).sum(axis=3, keepdims=True) / D"),
    "shared_first_head_only": ("return a.reshape(B, S, Hq, D).sum(axis=2, keepdims=True) / Hq",
                               "return a.reshape(B, S, Hq, D)[:, :, :1]"),
    "shared_averages_logits": ("    g = gate_layout(activation(gate_scores(X, W), act), Hq, D, mode)\n",
                               "    g = activation(gate_layout(gate_scores(X, W), Hq, D, mode), act)\n"),
    "rms_over_heads": ("np.mean(Y * Y, axis=-1, keepdims=True)", "np.mean(Y * Y, axis=-2, keepdims=True)"),
    "additive_as_multiplicative": ("        return Y + g\n", "        return Y * g\n"),
    "norm_after_gate": ("    if norm == \"rms\":\n        Y = rms_norm_heads(Y)\n", "    if norm == \"rms\":\n        Y = Y\n"),
    "value_gate_uses_query_heads": ("return V * gate_layout(g, Hkv, D, mode)", "return V * gate_layout(g, Hkv, D, mode)[:, ::-1]"),
}


def load_var_mutant(name):
    with open(VAR_SRC) as f:
        src = f.read().replace("from .gated_sdpa import", "from oracle.gated_sdpa import")
    if name is not None:
        old, new = VAR_MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not unique/present"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_var_mutant_{name}")
    exec(compile(src, f"<variant mutant {name}>", "exec"), mod.__dict__)
    return mod


def var_pins_pass(orc):
    """Brute-force loops over the variant cases, and the G2 value gate by loops."""
    from test_oracle_variants import CASES, brute_variant, draw, sig
    try:
        for mode, act, combine, norm in CASES:
            B, S, Hq, Hkv, D, dm = 2, 4, 4, 2, 3, 4
            N = {"elementwise": Hq * D, "headwise": Hq, "shared": Hq * D, "none": 1}[mode]
            t = draw(np.random.default_rng(11), B, S, Hq, Hkv, D, dm, N)
            got = orc.gated_sdpa_variant(t["X"], t["W"], t["Q"], t["K"], t["V"], mode, act, combine, norm)
            if not np.max(np.abs(got - brute_variant(t, mode, act, combine, norm))) <= 1e-12:
                return False
        t = draw(np.random.default_rng(12), 1, 4, 4, 2, 3, 4, 6)
        Vg = orc.value_gate(t["X"], t["W"], t["V"], "elementwise")
        for j in range(4):
            for c in range(2):
                for d in range(3):
                    z = math.fsum(t["X"][0, j, k] * t["W"][k, c * 3 + d] for k in range(4))
                    if abs(Vg[0, j, c, d] - t["V"][0, j, c, d] * sig(z)) > 1e-14:
                        return False
    except Exception:
        return False
    return True


def test_unmutated_variants_copy_passes():
    assert var_pins_pass(load_var_mutant(None))


@pytest.mark.parametrize("name", sorted(VAR_MUTANTS))
def test_variants_mutant_is_caught(name):
    assert not var_pins_pass(load_var_mutant(name))
