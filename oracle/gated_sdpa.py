"""fp64 numpy oracle for G1 gated SDPA — test infrastructure only (see package doc).

Notation follows the "GatedAttention [2025]" page: X is the gate input (hidden
states after pre-normalisation), W_θ the gate weight, Q, K, V the per-head
projections, d_k the head dimension (called D here), Y the SDPA output and Y'
the gated output.  Layouts: X [B, S, d_model]; W_θ [d_model, N] so that the gate
logits are X·W_θ; Q [B, S, Hq, D]; K, V [B, Skv, Hkv, D]; Y, Y' [B, S, Hq, D].

Readings of points the pages leave open (each listed in the design notes):
  * causal: query i (at absolute position i + Skv - S) sees keys j <= its
    position, itself included ("GatedAttention [2025]" §1.4.1 sums j = 0..i);
  * GQA: query head h reads key/value head h // (Hq / Hkv) (contiguous groups);
  * elementwise gate column for (head h, dim d) is h*D + d; headwise column is h
    ("10 · 门控" §3.2 snippet views the projection as [.., n_h, d_h] / [.., n_h, 1]);
  * no gate bias ("GatedAttention [2025]" §1.2.2 equation has none; the §3.2
    snippet on "10 · 门控" sets bias=False).
"""
import numpy as np


def gate_scores(X, W):
    """Gate logits Z = X·W_θ ("GatedAttention [2025]" §1.2.2 gating equation).

    X: [..., d_model]; W: [d_model, N]  ->  Z: [..., N], float64.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return X @ W


def sigmoid(Z):
    """Logistic sigmoid σ(z) = 1/(1+e^{-z}), the default activation
    ("GatedAttention [2025]" §1.2.2, item (5) and the closing default).

    For z < 0 it is evaluated as e^{z}/(1+e^{z}), the same value without
    overflowing e^{-z}.
    """
    Z = np.asarray(Z, dtype=np.float64)
    out = np.empty_like(Z)
    pos = Z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-Z[pos]))
    ez = np.exp(Z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def gate_values(g, Hq, D, mode):
    """Arrange gate scores per head, ready to multiply the SDPA output.

    g: [B, S, N] scores in (0, 1).  Elementwise: N = Hq*D, column h*D + d gates
    (head h, dim d) -> [B, S, Hq, D].  Headwise: N = Hq, one scalar per head per
    token -> [B, S, Hq, 1] ("GatedAttention [2025]" §1.2.2 granularity (2)).
    """
    B, S, N = g.shape
    if mode == "elementwise":
        assert N == Hq * D
        return g.reshape(B, S, Hq, D)
    if mode == "headwise":
        assert N == Hq
        return g.reshape(B, S, Hq, 1)
    raise ValueError(mode)


def sdpa(Q, K, V, rows=None, return_lse=False, return_probs=False, block=512):
    """Causal multi-head SDPA, Y = softmax(Q·Kᵀ/√d_k)·V per head
    ("GatedAttention [2025]" §1.2.1 SDPA equation, causal per §1.4.1).

    Q: [B, S, Hq, D]; K, V: [B, Skv, Hkv, D] with Skv >= S.  Query i sits at
    absolute position i + (Skv - S) and attends to keys j <= that position.
    Query head h uses key/value head h // (Hq // Hkv).

    rows: optional 1-D array of query indices to evaluate (others are returned
    as NaN).  Rows are evaluated in blocks of ``block`` independent rows; each
    row's softmax is over its whole visible prefix.

    Returns Y [B, S, Hq, D] (float64); with return_lse also the per-row
    log-sum-exp of the scaled scores [B, Hq, S]; with return_probs the full
    probability matrix [B, Hq, S, Skv] (tiny shapes only).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    assert K.shape == (B, Skv, Hkv, D) and V.shape == K.shape
    assert Hq % Hkv == 0 and Skv >= S
    G = Hq // Hkv
    off = Skv - S
    scale = 1.0 / np.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    Y = np.full((B, S, Hq, D), np.nan)
    lse = np.full((B, Hq, S), np.nan) if return_lse else None
    P_all = np.zeros((B, Hq, S, Skv)) if return_probs else None
    for b in range(B):
        for c in range(Hkv):                       # one key/value head ...
            heads = np.arange(c * G, (c + 1) * G)  # ... and the query heads of its group
            Kc = K[b, :, c, :]                     # [Skv, D]
            Vc = V[b, :, c, :]
            for s0 in range(0, len(rows), block):
                r = rows[s0:s0 + block]
                pos = r + off                      # absolute positions of these queries
                n_keys = int(pos.max()) + 1        # keys beyond every row's position are masked anyway
                q = Q[b][r][:, heads, :]           # [R, G, D]
                q = np.transpose(q, (1, 0, 2))     # [G, R, D]
                s = (q @ Kc[:n_keys].T) * scale    # [G, R, n_keys]  scaled dot products
                visible = np.arange(n_keys)[None, :] <= pos[:, None]   # causal: j <= position
                s = np.where(visible[None], s, -np.inf)
                m = s.max(axis=-1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=-1, keepdims=True)
                P = p / l                          # softmax: rows non-negative, summing to 1
                y = P @ Vc[:n_keys]                # [G, R, D]
                Y[b, r[:, None], heads[None, :], :] = np.transpose(y, (1, 0, 2))
                if return_lse:
                    lse[b, heads[:, None], r[None, :]] = (m + np.log(l))[..., 0]
                if return_probs:
                    P_all[b, heads[:, None], r[None, :], :n_keys] = P
    out = [Y]
    if return_lse:
        out.append(lse)
    if return_probs:
        out.append(P_all)
    return out[0] if len(out) == 1 else tuple(out)


def gated_sdpa(X, W, Q, K, V, mode, rows=None, return_gate=False):
    """G1 gated attention: Y' = Y ⊙ σ(X·W_θ) with Y the causal SDPA output, the
    gate applied per head before the heads are concatenated
    ("GatedAttention [2025]" §1.2.2 gating equation; "10 · 门控" §3.2 position
    table, G1 row, and the GatedAttentionOutput snippet).

    X: [B, S, d_model]; W: [d_model, N]; mode in {"elementwise", "headwise",
    "none"} ("none" returns plain SDPA).  Returns Y' [B, S, Hq, D] float64 (and
    the gate scores [B, S, N] when return_gate).
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Y = sdpa(Q, K, V, rows=rows)
    if mode == "none":
        return (Y, None) if return_gate else Y
    X = np.asarray(X, dtype=np.float64)
    if rows is not None:
        r = np.asarray(rows, dtype=np.int64)
        g = np.full((B, S, np.asarray(W).shape[1]), np.nan)
        g[:, r, :] = sigmoid(gate_scores(X[:, r, :], W))
    else:
        g = sigmoid(gate_scores(X, W))
    Yg = Y * gate_values(g, Hq, D, mode)
    return (Yg, g) if return_gate else Yg


def gated_decode(X, W, Q, Kc, Vc, mode, return_gate=False):
    """One decode step: a single query token per batch against a KV cache of
    length L that already holds that token (so it attends to all L keys).

    The cache is the "GatedAttention [2025]" §1.3.1 GQA explainer's KV cache.
    X: [B, 1, d_model]; Q: [B, 1, Hq, D]; Kc, Vc: [B, L, Hkv, D].  This is the
    same definition as ``gated_sdpa`` with S = 1 and Skv = L.
    """
    return gated_sdpa(X, W, Q, Kc, Vc, mode, return_gate=return_gate)


def gate_param_count(d_model, Hq, D, mode):
    """Extra parameters one layer's G1 gate adds: the W_θ entries.

    Elementwise gates have shape n×q×d_k, so W_θ is d_model × (q·d_k); headwise
    gates have shape n×q, so W_θ is d_model × q ("10 · 门控" §3.2, Table 1
    excerpt, shape column).
    """
    if mode == "elementwise":
        return d_model * Hq * D
    if mode == "headwise":
        return d_model * Hq
    raise ValueError(mode)
