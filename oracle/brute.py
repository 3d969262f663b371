"""Brute-force G1 gated SDPA in pure Python loops — test infrastructure only.

A second, independent statement of the definition for tiny shapes (a few
thousand score entries at most), used to pin the numpy oracle.  Scalars only:
``math.exp``, ``math.fsum``, nested loops, no numpy arithmetic.  The pieces are
the "GatedAttention [2025]" page's: SDPA equation (§1.2.1), causal prefix
(§1.4.1), gating equation and sigmoid (§1.2.2), GQA grouping (§1.3.1).
"""
import math


def _nested(a):
    return a.tolist() if hasattr(a, "tolist") else a


def gated_sdpa(X, W, Q, K, V, mode):
    """Return Y' as nested lists [B][S][Hq][D] (floats).

    X [B][S][dm]; W [dm][N]; Q [B][S][Hq][D]; K, V [B][Skv][Hkv][D].
    """
    X, W, Q, K, V = map(_nested, (X, W, Q, K, V))
    B, S, Hq, D = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    Skv, Hkv = len(K[0]), len(K[0][0])
    group = Hq // Hkv
    dm = len(W)
    N = len(W[0])
    out = []
    for b in range(B):
        out_b = []
        for i in range(S):
            pos = i + (Skv - S)
            # gate for this token: sigma(x_i . W[:, n]) for every column n
            gate = []
            for n in range(N):
                z = math.fsum(X[b][i][k] * W[k][n] for k in range(dm))
                gate.append(1.0 / (1.0 + math.exp(-z)) if z >= 0 else
                            math.exp(z) / (1.0 + math.exp(z)))
            out_i = []
            for h in range(Hq):
                c = h // group
                scores = []
                for j in range(pos + 1):
                    dot = math.fsum(Q[b][i][h][d] * K[b][j][c][d] for d in range(D))
                    scores.append(dot / math.sqrt(D))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = math.fsum(w)
                row = []
                for d in range(D):
                    y = math.fsum(w[j] * V[b][j][c][d] for j in range(pos + 1)) / tot
                    if mode == "elementwise":
                        y *= gate[h * D + d]
                    elif mode == "headwise":
                        y *= gate[h]
                    row.append(y)
                out_i.append(row)
            out_b.append(out_i)
        out.append(out_b)
    return out
