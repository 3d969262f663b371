"""fp64 numpy oracle for the backward of G1 gated SDPA — test infrastructure only.

The gradients are the chain rule applied to the plain forward definition
(``oracle.gated_sdpa``).  For an upstream gradient dY' of the gated output:

  gate branch ("Gated Attention如何用1%的参数量…" page, §2.2 gradient analysis:
  the gate's gradient is the upstream gradient times the context, and the
  gate input's gradient multiplies that by σ'(z) = σ(z)(1 − σ(z))):
      dY  = dY' ⊙ g                    (gradient reaching the SDPA output)
      dg  = dY' ⊙ Y                    (elementwise; headwise sums over the head dim)
      dZ  = dg ⊙ g ⊙ (1 − g)
      dX  = dZ · W_θᵀ,   dW_θ = Xᵀ · dZ
  SDPA branch (derivative of the "GatedAttention [2025]" §1.2.1 SDPA equation,
  causal per §1.4.1, GQA per §1.3.1):
      P = softmax(S), S = Q·Kᵀ/√D
      dV = Pᵀ · dY,  dP = dY · Vᵀ,  dS = P ⊙ (dP − rowsum(dP ⊙ P))
      dQ = dS · K/√D,  dK = dSᵀ · Q/√D
  with dK and dV summed over the query heads of each key/value group.

Every quantity is evaluated in float64 on the inputs as given.
"""
import numpy as np

from .gated_sdpa import gate_scores, sigmoid, gate_values, sdpa


def sdpa_backward(Q, K, V, dY):
    """Gradients (dQ, dK, dV) of Y = causal SDPA(Q, K, V) for the upstream
    gradient dY, in float64.

    Q, dY: [B, S, Hq, D]; K, V: [B, Skv, Hkv, D] with Skv >= S (query i sits at
    absolute position i + Skv - S).  One query head at a time, full score
    matrices: meant for shapes where S·Skv fits in memory.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    assert dY.shape == Q.shape and K.shape == (B, Skv, Hkv, D) and V.shape == K.shape
    assert Hq % Hkv == 0 and Skv >= S
    G = Hq // Hkv
    off = Skv - S
    scale = 1.0 / np.sqrt(D)
    visible = np.arange(Skv)[None, :] <= (np.arange(S) + off)[:, None]   # [S, Skv]
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            c = h // G
            q, dy = Q[b, :, h, :], dY[b, :, h, :]
            Kc, Vc = K[b, :, c, :], V[b, :, c, :]
            s = np.where(visible, (q @ Kc.T) * scale, -np.inf)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            P = p / p.sum(axis=-1, keepdims=True)
            dV[b, :, c, :] += P.T @ dy
            dP = dy @ Vc.T
            dS = P * (dP - (dP * P).sum(axis=-1, keepdims=True))
            dQ[b, :, h, :] = (dS @ Kc) * scale
            dK[b, :, c, :] += (dS.T @ q) * scale
    return dQ, dK, dV


def gated_sdpa_backward(X, W, Q, K, V, dYg, mode):
    """Gradients of Y' = SDPA(Q, K, V) ⊙ σ(X·W_θ) for the upstream gradient dYg.

    Returns a dict with dQ, dK, dV (shapes of Q, K, V) and, unless mode is
    "none", dX [B, S, d_model] and dW [d_model, N]; all float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    dYg = np.asarray(dYg, dtype=np.float64)
    B, S, Hq, D = Q.shape
    if mode == "none":
        dQ, dK, dV = sdpa_backward(Q, K, V, dYg)
        return {"dQ": dQ, "dK": dK, "dV": dV, "dX": None, "dW": None}
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Y = sdpa(Q, K, V)
    g = sigmoid(gate_scores(X, W))                 # [B, S, N]
    gv = gate_values(g, Hq, D, mode)               # [B, S, Hq, D] or [B, S, Hq, 1]
    dY = dYg * gv                                  # through the product, to Y
    dgv = dYg * Y                                  # to the gate, per (head, dim)
    if mode == "headwise":
        dg = dgv.sum(axis=-1)                      # one gate per head: sum over the dims it scales
    else:
        dg = dgv.reshape(B, S, Hq * D)
    dZ = dg * g * (1.0 - g)                        # through σ
    dX = dZ @ W.T
    dW = X.reshape(B * S, -1).T @ dZ.reshape(B * S, -1)
    dQ, dK, dV = sdpa_backward(Q, K, V, dY)
    return {"dQ": dQ, "dK": dK, "dV": dV, "dX": dX, "dW": dW}


def gated_sdpa_backward_sampled(X, W, Q, K, V, dYg, mode, kv_heads, rows):
    """Part of ``gated_sdpa_backward``'s result, for shapes where all of it is too
    costly: the same chain rule, evaluated only for

      * the key/value heads ``kv_heads``: dK and dV of those heads and dQ of every
        query head in their groups (all rows);
      * the dW_θ columns those query heads' gates use (all d_model rows);
      * the dX rows ``rows`` (every column).

    Returns a dict with q_heads, dQ [B, S, len(q_heads), D], dK and dV
    [B, S, len(kv_heads), D], w_cols, dW [d_model, len(w_cols)] and dX
    [B, len(rows), d_model] (the last three None for mode "none"); float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dYg = np.asarray(dYg, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    kv_heads = np.asarray(kv_heads, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    q_heads = np.concatenate([np.arange(c * G, (c + 1) * G) for c in kv_heads])
    gated = mode != "none"
    per = D if mode == "elementwise" else 1          # gate columns per query head
    out = {"q_heads": q_heads, "dQ": np.zeros((B, S, len(q_heads), D)),
           "dK": np.zeros((B, S, len(kv_heads), D)), "dV": np.zeros((B, S, len(kv_heads), D)),
           "w_cols": None, "dW": None, "dX": None}
    if gated:
        X = np.asarray(X, dtype=np.float64)
        W = np.asarray(W, dtype=np.float64)
        w_cols = (q_heads[:, None] * per + np.arange(per)[None, :]).ravel()
        g_cols = sigmoid(gate_scores(X, W[:, w_cols]))   # gates of the sampled heads, every row
        out["w_cols"] = w_cols
        out["dW"] = np.zeros((X.shape[-1], len(w_cols)))
    for i, c in enumerate(kv_heads):
        hq = slice(c * G, (c + 1) * G)                   # query heads of this group
        loc = slice(i * G, (i + 1) * G)                  # their place in the output
        cols = slice(i * G * per, (i + 1) * G * per)
        Kc, Vc = K[:, :, c:c + 1], V[:, :, c:c + 1]
        dY = dYg[:, :, hq]
        if gated:
            g = g_cols[:, :, cols]                       # [B, S, G*per]
            dY = dY * g.reshape(B, S, G, per)            # through the product, to Y
        dq, dk, dv = sdpa_backward(Q[:, :, hq], Kc, Vc, dY)
        out["dQ"][:, :, loc] = dq
        out["dK"][:, :, i] = dk[:, :, 0]
        out["dV"][:, :, i] = dv[:, :, 0]
        if gated:
            Y = sdpa(Q[:, :, hq], Kc, Vc)                # [B, S, G, D]
            dgv = dYg[:, :, hq] * Y                      # to the gate, per (head, dim)
            dg = dgv.sum(axis=-1) if mode == "headwise" else dgv.reshape(B, S, G * D)
            dZ = dg * g * (1.0 - g)                      # through σ
            out["dW"][:, cols] = X.reshape(B * S, -1).T @ dZ.reshape(B * S, -1)
    if gated:
        Yr = sdpa(Q, K, V, rows=rows)[:, rows]           # [B, R, Hq, D]
        gr = sigmoid(gate_scores(X[:, rows], W))         # [B, R, N]
        dgv = dYg[:, rows] * Yr
        dg = dgv.sum(axis=-1) if mode == "headwise" else dgv.reshape(B, len(rows), Hq * D)
        dZ = dg * gr * (1.0 - gr)
        out["dX"] = dZ @ W.T
    return out
