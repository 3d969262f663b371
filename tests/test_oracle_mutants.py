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
