"""The Python binding refuses a gate or an output it cannot hand to the kernels
(wrong width for the gate layout, wrong dtype, wrong device, wrong shape)
before any launch.  The C ABI only sees pointers, so these checks are the only
guard against a kernel reading past the end of G.  The tensors here live on the
CPU: every refusal must come from the gate / output checks, which run before
the binding asks for device pointers (a CPU tensor that passed them would be
refused as "must be a GPU tensor" instead)."""
import pytest
import torch

import gated_softmax_attention_amd as gsa

B, S, Hq, Hkv, D, DM = 2, 16, 4, 2, 64, 32


def qkv(dtype=torch.bfloat16):
    Q = torch.zeros((B, S, Hq, D), dtype=dtype)
    K = torch.zeros((B, S, Hkv, D), dtype=dtype)
    return Q, K, K.clone()


def gate(n_cols, rows=B * S, dtype=torch.float32):
    return torch.zeros((rows, n_cols), dtype=dtype)


def refused(fn, *a, match, **kw):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **kw)


def reaches_pointer_check(fn, *a, **kw):
    """Arguments that pass every shape check stop at the device-pointer check."""
    with pytest.raises(ValueError, match="GPU tensor"):
        fn(*a, **kw)


def test_forward_gate_width_dtype_and_presence():
    Q, K, V = qkv()
    refused(gsa.forward, Q, K, V, gate(Hq), "elementwise", match="elementwise")        # headwise width
    refused(gsa.forward, Q, K, V, gate(Hq * D), "headwise", match="headwise")          # elementwise width
    refused(gsa.forward, Q, K, V, gate(Hq * D, dtype=torch.bfloat16), "elementwise", match="float32")
    refused(gsa.forward, Q, K, V, gate(Hq * D, rows=B * S - 1), "elementwise", match="rows")
    refused(gsa.forward, Q, K, V, None, "elementwise", match="required")
    refused(gsa.forward, Q, K, V, gate(Hq), "none", match="None")
    refused(gsa.forward, Q, K, V, gate(Hq), "shared", match="mode")
    reaches_pointer_check(gsa.forward, Q, K, V, gate(Hq * D), "elementwise")
    reaches_pointer_check(gsa.forward, Q, K, V, gate(Hq), "headwise")


def test_forward_output_checks():
    Q, K, V = qkv()
    G = gate(Hq * D)
    refused(gsa.forward, Q, K, V, G, "elementwise", Y=torch.zeros((B, S, Hq, D - 1), dtype=Q.dtype), match="Y")
    refused(gsa.forward, Q, K, V, G, "elementwise", Y=torch.zeros((B, S, Hq, D), dtype=torch.float32), match="Y")
    refused(gsa.forward_lse, Q, K, V, gate(Hq * D + 1), "elementwise", match="elementwise")
    reaches_pointer_check(gsa.forward, Q, K, V, G, "elementwise", Y=torch.zeros_like(Q))


def test_decode_gate_and_output():
    Q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16)
    Kc = torch.zeros((B, 40, Hkv, D), dtype=torch.bfloat16)
    refused(gsa.decode, Q, Kc, Kc, gate(Hq, rows=B), "elementwise", match="elementwise")
    refused(gsa.decode, Q, Kc, Kc, gate(Hq * D, rows=B * S), "elementwise", match="rows")
    refused(gsa.decode, Q, Kc, Kc, gate(Hq, rows=B, dtype=torch.float64), "headwise", match="float32")
    refused(gsa.decode_noalloc, Q, Kc, Kc, gate(Hq, rows=B), "headwise", None, match="allocates nothing")
    refused(gsa.decode_noalloc, Q, Kc, Kc, gate(Hq, rows=B), "headwise", torch.zeros((B, Hq, D)), match="Y")
    reaches_pointer_check(gsa.decode, Q, Kc, Kc, gate(Hq, rows=B), "headwise")


def test_variant_layouts():
    Q, K, V = qkv()
    refused(gsa.forward_variant, Q, K, V, gate(Hq * D), "shared", match="shared")       # not yet head-averaged
    refused(gsa.forward_variant, Q, K, V, gate(D), "elementwise", match="elementwise")
    refused(gsa.forward_variant, Q, K, V, gate(D), "none", match="None")
    reaches_pointer_check(gsa.forward_variant, Q, K, V, gate(D), "shared")
    Qd = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16)
    Kc = torch.zeros((B, 40, Hkv, D), dtype=torch.bfloat16)
    refused(gsa.decode_variant, Qd, Kc, Kc, gate(Hq * D, rows=B), "shared", match="shared")
    reaches_pointer_check(gsa.decode_variant, Qd, Kc, Kc, gate(D, rows=B), "shared")


def test_value_gate_and_head_mean():
    V = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16)
    refused(gsa.value_gate, V, gate(Hq * D), "elementwise", match="elementwise")         # query-head width
    refused(gsa.value_gate, V, gate(Hkv * D), "headwise", match="headwise")
    refused(gsa.value_gate, V, gate(Hkv * D), "shared", match="layout")
    refused(gsa.value_gate, V, gate(Hkv), "headwise", Vout=torch.zeros((B, S, Hkv, D)), match="Vout")
    reaches_pointer_check(gsa.value_gate, V, gate(Hkv), "headwise")
    refused(gsa.gate_head_mean, gate(Hq * D + 4), Hq, D, match="rows")
    refused(gsa.gate_head_mean, gate(Hq * D, dtype=torch.bfloat16), Hq, D, match="float32")


def test_whole_path_weight_and_rows():
    Q, K, V = qkv()
    X = torch.zeros((B, S, DM), dtype=torch.bfloat16)
    refused(gsa.gated_attention, X, torch.zeros((DM, Hq)), Q, K, V, "elementwise", match="W must be")
    refused(gsa.gated_attention, X, torch.zeros((DM, Hq * D)), Q, K, V, "headwise", match="W must be")
    refused(gsa.gated_attention, X[:, :-1], torch.zeros((DM, Hq)), Q, K, V, "headwise", match="token rows")
    refused(gsa.gated_attention, X, torch.zeros((DM + 1, Hq)), Q, K, V, "headwise", match="W must be")
    Qd = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16)
    Kc = torch.zeros((B, 40, Hkv, D), dtype=torch.bfloat16)
    refused(gsa.gated_decode, X, torch.zeros((DM, Hq)), Qd, Kc, Kc, "headwise", match="token rows")
    refused(gsa.gated_attention_variant, X, torch.zeros((DM, D)), Q, K, V, "shared", match="W must be")


def test_backward_gate_checks():
    Q, K, V = qkv()
    X = torch.zeros((B, S, DM), dtype=torch.bfloat16)
    LSE = torch.zeros((B, Hq, S))
    refused(gsa.backward, X, torch.zeros((DM, Hq * D), dtype=torch.bfloat16), gate(Hq), Q, K, V, Q, LSE, Q,
            "elementwise", match="elementwise")
    refused(gsa.backward, X, torch.zeros((DM, Hq), dtype=torch.bfloat16), gate(Hq), Q, K, V, Q, LSE, Q,
            "elementwise", match="elementwise")
    refused(gsa.backward, X, torch.zeros((DM, Hq), dtype=torch.bfloat16), gate(Hq), Q, K, V, Q, LSE, Q,
            "none", match="None")
