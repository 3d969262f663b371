"""Oracle for SDPA-output (G1) gated attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 CPU statement of what the hot path computes, written from
the pages, used to judge the HIP path.  Only ``tests/``, ``smoke()`` in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import it;
the library and its Python binding never do, and this package imports nothing
from them.

Sources (page titles; sections):
  * "GatedAttention [2025]" (huaxiaozhuan.com, a translation of *Gated Attention
    for Large Language Models: Non-linearity, Sparsity, and Attention-Sink-Free*):
    §1.2.1 SDPA equation and multi-head concatenation; §1.2.2 gating equation
    Y' = Y ⊙ σ(X W_θ), granularity (headwise / elementwise), default activation
    σ(x) = 1/(1+e^{-x}); §1.3.1 GQA explainer; §1.4.1 per-head output equation
    (causal prefix sum j = 0..i).
  * "10 · 门控" (llm-infra-atlas): §3.2 position table (G1: after SDPA, per head,
    before concat) and the GatedAttentionOutput snippet (bias-free projection,
    view of the gate as [B, T, n_h, d_h] or [B, T, n_h, 1]).

Every function here is pinned by tests in ``tests/test_oracle.py``,
``tests/test_oracle_backward.py``, ``tests/test_oracle_diagnostics.py``,
``tests/test_oracle_projection.py`` and ``tests/test_oracle_variants.py`` (brute-force loops, central differences of the
brute-force forward, a library SDPA and a library autodiff in float64, closed
forms and invariants); none is "parity unpinned".

The backward (``backward.py``) is the chain rule on the plain forward; its gate
branch follows the "Gated Attention如何用1%的参数量…" page, §2.2 gradient analysis.
``variants.py`` holds the gating variants of the design space (§1.2.2 items
(3)-(5), NS-sigmoid of §1.4.2, the per-head RMSNorm of §1.4.1, G2 value
gating), pinned in ``tests/test_oracle_variants.py``.
``projection.py`` holds the fused input projection (§1.2.1 QKV projections plus the
gate scores), pinned in ``tests/test_oracle_projection.py``.
``diagnostics.py`` holds the first-token attention share ("GatedAttention [2025]"
§1.4.3, F-Attn; "10 · 门控" §3.4), pinned in ``tests/test_oracle_diagnostics.py``.
"""
from .gated_sdpa import (
    gate_scores, sigmoid, gate_values, sdpa, gated_sdpa, gated_decode,
    gate_param_count,
)
from .backward import sdpa_backward, gated_sdpa_backward, gated_sdpa_backward_sampled
from .diagnostics import first_token_attention
from .projection import project_qkvg
from . import variants
from . import brute

__all__ = ["gate_scores", "sigmoid", "gate_values", "sdpa", "gated_sdpa", "gated_decode",
           "gate_param_count", "sdpa_backward", "gated_sdpa_backward",
           "gated_sdpa_backward_sampled", "first_token_attention", "project_qkvg", "variants", "brute"]
