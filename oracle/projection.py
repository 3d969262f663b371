"""fp64 oracle for the fused input projection — test infrastructure only.

The attention layer's first stage ("GatedAttention [2025]" §1.2.1: the QKV
linear projections Q = X·W_Q, K = X·W_K, V = X·W_V) together with the G1 gate
scores it shares its input with (§1.2.2: σ(X·W_θ)).  Head h of Q takes columns
h·D .. h·D + D − 1 of X·W_Q (the per-head split of the same section), likewise
K and V with the key/value heads.
"""
import numpy as np

from .gated_sdpa import gate_scores, sigmoid


def project_qkvg(X, Wq, Wk, Wv, W, Hq, Hkv, D):
    """Q [B,S,Hq,D], K and V [B,S,Hkv,D], and G = σ(X·W_θ) [B,S,N] (None when W
    is None), all float64.  X: [B, S, d_model]; Wq [d_model, Hq·D]; Wk, Wv
    [d_model, Hkv·D]; W [d_model, N]."""
    X = np.asarray(X, dtype=np.float64)
    B, S, _ = X.shape
    Q = (X @ np.asarray(Wq, dtype=np.float64)).reshape(B, S, Hq, D)
    K = (X @ np.asarray(Wk, dtype=np.float64)).reshape(B, S, Hkv, D)
    V = (X @ np.asarray(Wv, dtype=np.float64)).reshape(B, S, Hkv, D)
    G = None if W is None else sigmoid(gate_scores(X, W))
    return Q, K, V, G
