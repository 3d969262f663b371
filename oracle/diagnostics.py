"""fp64 oracle for the first-token attention diagnostic — test infrastructure only.

The share of attention a query row gives the first token ("GatedAttention
[2025]" §1.4.3, the F-Attn column of Table 4; "10 · 门控" §3.4, the average
attention on token 0 before and after gating): for query head h and row i,

    F[b, h, i] = P_{i,0} = exp(s_{i,0}) / Σ_{j<=i} exp(s_{i,j}),   s_{i,j} = q_i·k_j / √D,

the causal softmax probability of key 0 (self included, so row 0 gives 1).
The pages average it over heads (and rows); ``first_token_attention`` also
returns per-head means over batches and rows, and the mean of those.
"""
import numpy as np

from .gated_sdpa import sdpa


def first_token_attention(Q, K, V, rows=None):
    """F [B, Hq, S], per-head means [Hq] and their mean, in float64.

    Q: [B, S, Hq, D]; K, V: [B, S, Hkv, D] (V only fixes the call to the
    plain SDPA, whose per-row log-sum-exp is the softmax denominator).  With
    ``rows`` only those query rows are evaluated (the others are NaN) and the
    means are None.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    r = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    _, lse = sdpa(Q, K, V, rows=r, return_lse=True)         # ln Σ_{j<=i} exp(s_ij)   [B, Hq, S]
    F = np.full((B, Hq, S), np.nan)
    for h in range(Hq):
        k0 = K[:, 0, h // G, :]                             # [B, D]: key 0 of this head's group
        s0 = np.einsum("bsd,bd->bs", Q[:, r, h, :], k0) / np.sqrt(D)
        F[:, h, r] = np.exp(s0 - lse[:, h, r])
    if rows is not None:
        return F, None, None
    head_mean = F.mean(axis=(0, 2))
    return F, head_mean, float(head_mean.mean())
