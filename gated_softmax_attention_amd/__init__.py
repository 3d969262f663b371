"""gated_softmax_attention_amd — SDPA-output (G1) gated attention for AMD MI355X (gfx950).

Thin Python binding over libgsa.so (see include/gsa.h).  Every step of the
computation runs in the library's HIP kernels; this module only checks tensor
properties, allocates outputs with torch and passes device pointers and the
current HIP stream.  There is no CPU or PyTorch fallback: calls fail loudly
when the library is missing or no GPU is present.
"""
from .ops import (gate_logits, gate_logits_workspace_bytes, gated_decode_workspace_bytes, forward, forward_lse, decode, gated_attention, gated_decode,
                  decode_workspace_bytes, decode_num_splits, decode_noalloc, noalloc_scratch_bytes, backward, backward_workspace_bytes,
                  first_token_attention, project_qkvg, forward_variant, decode_variant, value_gate,
                  gate_head_mean, gated_attention_variant, gate_width, forward_value_gated,
                  MODES, LAYOUTS, ACTIVATIONS)
from ._lib import GsaError, load as load_library, LIB_PATH

__all__ = ["gate_logits", "gate_logits_workspace_bytes", "gated_decode_workspace_bytes", "forward", "forward_lse", "decode", "gated_attention", "gated_decode",
           "decode_workspace_bytes", "decode_num_splits", "decode_noalloc", "noalloc_scratch_bytes", "backward",
           "backward_workspace_bytes", "first_token_attention", "project_qkvg", "forward_variant",
           "decode_variant", "value_gate", "gate_head_mean", "gated_attention_variant", "gate_width", "forward_value_gated", "MODES", "LAYOUTS", "ACTIVATIONS", "GsaError",
           "load_library", "LIB_PATH"]
