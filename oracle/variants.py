"""fp64 oracle for the gating variants of the design space — test infrastructure only.

The "GatedAttention [2025]" page's §1.2.2 lays out the axes a gate can vary
along, with G1 (SDPA output) as the main position:

  * head-specific or head-shared scores (item (3)): head-shared gives every
    query head the same gating score of width d_k per token.  The §1.3.2
    Table 1 discussion (observation (ii)) says how it is formed: the n×q×d_k
    gating scores are averaged over the q query heads into an n×d_k score.
    The gating score is the activated value act(X·W_θ) (the quantity §1.2.2
    calls the score and multiplies into Y), so the average is taken after the
    activation, and W_θ keeps the elementwise width q·d_k ("10 · 门控" §3.2,
    Table 1 row 12 prices head-shared at 201 M, the same as row 5);
  * multiplicative, Y' = Y ⊙ act(X·W_θ), or additive, Y' = Y + act(X·W_θ)
    (item (4));
  * the activation (item (5)): sigmoid (for multiplicative), SiLU(x) = x·σ(x)
    (unbounded, so only additive), or the identity; §1.4.2 (iv) adds the
    non-sparse NS-sigmoid 0.5 + 0.5·σ(x), whose range is [0.5, 1];
  * §1.4.1 replaces or precedes the gate with an RMSNorm of each head's SDPA
    output before concatenation (Table 3 row 5);
  * G2 places the gate on the value map instead: V' = V ⊙ σ(X·W_v) per
    key/value head, then attention over V'.

Readings of what the pages leave open (listed in the design notes): the
RMSNorm has unit weight and ε = 1e-6 (the pages give neither, and count the
norm as adding next to no parameters); norm and gate together apply the norm
first; the G2 gate columns follow the G1 convention with key/value heads
(c·D + d, or c).
"""
import numpy as np

from .gated_sdpa import gate_scores, sigmoid, sdpa

ACTIVATIONS = ("identity", "sigmoid", "ns_sigmoid", "silu")
RMS_EPS = 1e-6


def activation(Z, act):
    """The gate activation applied to the logits Z = X·W_θ."""
    Z = np.asarray(Z, dtype=np.float64)
    if act == "identity":
        return Z
    if act == "sigmoid":
        return sigmoid(Z)
    if act == "ns_sigmoid":
        return 0.5 + 0.5 * sigmoid(Z)
    if act == "silu":
        return Z * sigmoid(Z)
    raise ValueError(act)


def gate_width(mode, Hq, D):
    """Columns of W_θ (per layer: d_model × gate_width parameters) each layout
    consumes: q·d_k for elementwise and for head-shared (whose n×q×d_k scores
    are then averaged over the q heads), q for headwise."""
    if mode in ("elementwise", "shared"):
        return Hq * D
    if mode == "headwise":
        return Hq
    raise ValueError(mode)


def gate_layout(a, Hq, D, mode):
    """Activated scores [B, S, N] arranged to broadcast against Y [B, S, Hq, D]:
    elementwise N = Hq·D -> [B, S, Hq, D]; headwise N = Hq -> [B, S, Hq, 1];
    shared N = Hq·D -> [B, S, 1, D], the mean over the Hq heads of the
    elementwise arrangement (one vector for every head)."""
    B, S, N = a.shape
    assert N == gate_width(mode, Hq, D)
    if mode == "elementwise":
        return a.reshape(B, S, Hq, D)
    if mode == "headwise":
        return a.reshape(B, S, Hq, 1)
    # shared: mean over the query-head axis of the [.., q, d_k] scores
    return a.reshape(B, S, Hq, D).sum(axis=2, keepdims=True) / Hq


def rms_norm_heads(Y, eps=RMS_EPS):
    """Per-head RMSNorm over the head dimension, unit weight: y / sqrt(mean_d y² + ε)."""
    Y = np.asarray(Y, dtype=np.float64)
    return Y / np.sqrt(np.mean(Y * Y, axis=-1, keepdims=True) + eps)


def gated_sdpa_variant(X, W, Q, K, V, mode, act="sigmoid", combine="mul", norm=None, rows=None):
    """Y' for one point of the G1 design space (float64).

    mode in {"none", "elementwise", "headwise", "shared"}; act in ACTIVATIONS;
    combine in {"mul", "add"}; norm in {None, "rms"}.  With mode "none" the
    result is the (optionally normalised) SDPA output.  With ``rows`` only
    those query rows are evaluated and returned ([B, len(rows), Hq, D]).
    K and V may hold more keys than Q has rows (query i at position
    i + Skv - S): one decode step is S = 1 against the whole cache, and the
    gate then sits at the decode merge.
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Y = sdpa(Q, K, V, rows=rows)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        Y = Y[:, rows]
        X = np.asarray(X, dtype=np.float64)[:, rows] if X is not None else None
    if norm == "rms":
        Y = rms_norm_heads(Y)
    elif norm is not None:
        raise ValueError(norm)
    if mode == "none":
        return Y
    g = gate_layout(activation(gate_scores(X, W), act), Hq, D, mode)
    if combine == "mul":
        return Y * g
    if combine == "add":
        return Y + g
    raise ValueError(combine)


def value_gate(X, Wv, V, mode):
    """G2: V' = V ⊙ σ(X·W_v) with one score per (key/value head, dim) (elementwise,
    column c·D + d) or per key/value head (headwise, column c).  X: [B, S, d_model];
    V: [B, S, Hkv, D]."""
    V = np.asarray(V, dtype=np.float64)
    B, S, Hkv, D = V.shape
    g = sigmoid(gate_scores(X, Wv))
    return V * gate_layout(g, Hkv, D, mode)


def value_gated_sdpa(X, Wv, Q, K, V, mode):
    """Causal SDPA over the gated values V' (G2 position)."""
    return sdpa(Q, K, value_gate(X, Wv, V, mode))
