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
