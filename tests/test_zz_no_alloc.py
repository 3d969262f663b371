"""gsa_decode_noalloc (decode without a caller workspace, for callers that
cannot allocate) against gsa_decode, both called through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, so the
second runs on the scratch the first left behind.  Each output must equal
gsa_decode's on the same inputs and split count bit for bit (the two share their
kernels), and both must be within the bf16 bar of the fp64 oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_softmax_attention_amd import _lib
from synth import CONFIGS, make_inputs
from helpers import TOL, f64, report, oracle_decode_by_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def call_both(lib, inp, mode, num_splits):
    """gsa_decode (with a workspace) and gsa_decode_noalloc on the same inputs."""
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    B, _, Hq, D = Q.shape
    L, Hkv = K.shape[1], K.shape[2]
    G = None
    if mode != "none":
        G = torch.empty((B, inp["W"].shape[1]), dtype=torch.float32, device=DEV)
        _lib.check(lib.gsa_gate_logits(ptr(inp["X"]), ptr(inp["W"]), ptr(G), B, inp["X"].shape[-1],
                                       G.shape[1], _lib.GSA_BF16, _lib.GSA_ACT_SIGMOID, None))
    mcode = {"none": _lib.GSA_GATE_NONE, "elementwise": _lib.GSA_GATE_ELEMENTWISE,
             "headwise": _lib.GSA_GATE_HEADWISE}[mode]
    need = lib.gsa_decode_workspace_bytes(B, L, Hq, Hkv, D, num_splits)
    assert need <= lib.gsa_noalloc_scratch_bytes()
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y_ref = torch.full_like(Q, float("nan"))
    y_na = torch.full_like(Q, float("nan"))
    _lib.check(lib.gsa_decode(ptr(Q), ptr(K), ptr(V), ptr(G), ptr(y_ref), B, L, Hq, Hkv, D, mcode,
                              _lib.GSA_BF16, num_splits, ptr(ws), need, None))
    _lib.check(lib.gsa_decode_noalloc(ptr(Q), ptr(K), ptr(V), ptr(G), ptr(y_na), B, L, Hq, Hkv, D, mcode,
                                      _lib.GSA_BF16, num_splits, None))
    torch.cuda.synchronize()
    return y_ref, y_na


def check_pair(inp, mode, y_ref, y_na, what):
    a = y_ref.view(torch.int16).cpu().numpy()
    b = y_na.view(torch.int16).cpu().numpy()
    assert not torch.isnan(y_na.float()).any(), f"{what}: output not fully written"
    assert np.array_equal(a, b), f"{what}: {int((a != b).sum())} elements differ from gsa_decode"
    # every batch against the oracle (the full-size call: all 64 batches)
    want = oracle_decode_by_batch(inp, mode)
    report(f64(y_na), want, TOL["bf16"], what)


def test_noalloc_matches_decode_on_two_calls():
    lib = _lib.load()
    torch.cuda.set_device(0)
    # first call: the full decode workload (64 batches, a 16384-key cache, 32/8 heads,
    # D 128) with the automatic split count, as the bench times it
    big = CONFIGS["decode"]
    print(f"case 1: decode B{big.B} L{big.L} {big.Hq}/{big.Hkv}x{big.D} elementwise, auto splits", flush=True)
    inp = make_inputs(big, seed=0, device=DEV)
    y_ref, y_na = call_both(lib, inp, "elementwise", 0)
    check_pair(inp, "elementwise", y_ref, y_na, "noalloc decode, full size")
    del inp, y_ref, y_na
    torch.cuda.empty_cache()
    # second call, smaller: fewer batches, a short ragged cache, another head layout
    # and an explicit split count, so its partial records sit where the first
    # call's stale ones are
    small = big.with_(name="noalloc_small", B=3, L=1000, Hq=8, Hkv=2, D=64, d_model=256, mode="headwise")
    print(f"case 2: decode B{small.B} L{small.L} {small.Hq}/{small.Hkv}x{small.D} headwise, 5 splits",
          flush=True)
    inp = make_inputs(small, seed=3, device=DEV)
    y_ref, y_na = call_both(lib, inp, "headwise", 5)
    check_pair(inp, "headwise", y_ref, y_na, "noalloc decode, second smaller call")


def test_noalloc_refuses_partials_beyond_the_scratch():
    lib = _lib.load()
    cap = lib.gsa_noalloc_scratch_bytes()
    # 64 batches x 32 heads x 8 splits x 132 floats x 4 B = 8.65 MB > 8 MiB
    assert lib.gsa_decode_workspace_bytes(64, 16384, 32, 8, 128, 8) > cap
    Q = torch.zeros((64, 1, 32, 128), dtype=torch.bfloat16, device=DEV)
    status = lib.gsa_decode_noalloc(ptr(Q), ptr(Q), ptr(Q), None, ptr(Q), 64, 16384, 32, 8, 128,
                                    _lib.GSA_GATE_NONE, _lib.GSA_BF16, 8, None)
    assert status == _lib.GSA_ERR_WORKSPACE
    assert b"scratch" in lib.gsa_last_error_message()
