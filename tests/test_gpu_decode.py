"""Split-K gated decode on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs
from helpers import TOL, f64, report, guarded_empty, guard_ok, oracle_decode_by_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dec_cfg(B, L, Hq, Hkv, D, mode, dtype, dm=64):
    return CONFIGS["decode"].with_(name="d", B=B, L=L, Hq=Hq, Hkv=Hkv, D=D, mode=mode, dtype=dtype,
                                   d_model=dm)


def run(inp, mode, num_splits=0):
    Q = inp["Q"]
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    Y, g = guarded_empty(tuple(Q.shape), Q.dtype, DEV)
    gsa.decode(Q, inp["K"], inp["V"], G, mode, num_splits=num_splits, Y=Y)
    torch.cuda.synchronize()
    assert guard_ok(g)
    return Y, G


def oracle_decode(inp, mode, batches=None):
    bs = slice(None) if batches is None else batches
    return oracle.gated_decode(f64(inp["X"][bs]), f64(inp["W"]), f64(inp["Q"][bs]), f64(inp["K"][bs]),
                               f64(inp["V"][bs]), mode)


CASES = []
# (Hkv a multiple of 4 takes the 4-heads-per-workgroup split kernel; with
# groups of 6, 8 and 12 query heads it also serves 2 or 3 quads, the last partial)
for (B, L, Hq, Hkv) in [(1, 1, 4, 1), (2, 15, 4, 4), (3, 16, 8, 2), (2, 63, 8, 1), (1, 1025, 32, 8),
                        (2, 3000, 16, 2), (4, 777, 12, 2), (1, 4096, 4, 4), (2, 1500, 32, 4), (1, 700, 48, 4),
                        (3, 333, 24, 4), (1, 2000, 16, 16)]:
    for D in (128, 64):
        for mode in ("elementwise", "headwise"):
            CASES.append((B, L, Hq, Hkv, D, mode))
CASES.append((2, 500, 8, 2, 128, "none"))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,L,Hq,Hkv,D,mode", CASES)
def test_small_decode(B, L, Hq, Hkv, D, mode, dtype):
    inp = make_inputs(dec_cfg(B, L, Hq, Hkv, D, mode, dtype), seed=L + Hq, device=DEV)
    Y, _ = run(inp, mode)
    report(f64(Y), oracle_decode(inp, mode), TOL[dtype], f"{dtype} B{B} L{L} {Hq}/{Hkv} D{D} {mode}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 8)])   # one key/value head per split workgroup, and four
@pytest.mark.parametrize("ns", [1, 2, 3, 7, 16, 64])
def test_split_counts_agree(ns, Hq, Hkv):
    inp = make_inputs(dec_cfg(2, 2049, Hq, Hkv, 128, "elementwise", "bf16"), seed=9, device=DEV)
    want = oracle_decode(inp, "elementwise")
    Y, _ = run(inp, "elementwise", num_splits=ns)
    report(f64(Y), want, TOL["bf16"], f"{Hq}/{Hkv} heads, splits {ns} (effective "
           f"{gsa.decode_num_splits(2, 2049, Hq, Hkv, 128, ns)})")


def test_decode_matches_last_prefill_row():
    """Decode of token L-1 against the cache equals row L-1 of the prefill forward."""
    L = 700
    cfg = CONFIGS["tiny_fp32"].with_(name="p", B=2, S=L, Hq=8, Hkv=2, D=128, d_model=64,
                                     mode="elementwise", dtype="bf16")
    inp = make_inputs(cfg, seed=5, device=DEV)
    G = gsa.gate_logits(inp["X"], inp["W"])
    Yp = gsa.forward(inp["Q"], inp["K"], inp["V"], G, "elementwise")
    dec = {"X": inp["X"][:, -1:].contiguous(), "W": inp["W"], "Q": inp["Q"][:, -1:].contiguous(),
           "K": inp["K"], "V": inp["V"]}
    Yd, _ = run(dec, "elementwise")
    report(f64(Yd), f64(Yp[:, -1:]), TOL["bf16"], "decode vs prefill last row")
    report(f64(Yd), oracle_decode(dec, "elementwise"), TOL["bf16"], "decode vs oracle")


def test_saturated_gate_decode_equals_ungated_bitwise():
    inp = make_inputs(dec_cfg(2, 1000, 8, 2, 128, "elementwise", "bf16"), seed=2, device=DEV)
    inp["W"].zero_()
    inp["W"][0, :] = 1.0
    inp["X"][..., 0] = 40.0
    Yg, G = run(inp, "elementwise")
    assert bool((G == 1.0).all())
    Yn, _ = run(inp, "none")
    assert torch.equal(Yg.view(torch.int16), Yn.view(torch.int16))


def test_full_size_decode_config():
    """The decode workload (B 64, L 16384, 32/8 heads, elementwise gate) with the
    automatic split count the bench uses: every batch against the oracle."""
    cfg = CONFIGS["decode"]
    print("  decode: generating inputs", flush=True)
    inp = make_inputs(cfg, seed=0, device=DEV)
    Y, _ = run(inp, cfg.mode)
    assert not torch.isnan(Y.float()).any()
    report(f64(Y), oracle_decode_by_batch(inp, cfg.mode), TOL["bf16"], f"decode full size, all {cfg.B} batches")


def test_decode_long_cache():
    """A 262144-long cache (one batch, 32/8 heads, elementwise gate)."""
    cfg = dec_cfg(1, 262144, 32, 8, 128, "elementwise", "bf16")
    inp = make_inputs(cfg, seed=9, device=DEV)
    Y, _ = run(inp, "elementwise")
    report(f64(Y), oracle_decode(inp, "elementwise"), TOL["bf16"], "decode L=262144")


# --------------------------------------------------------------- the whole decode step in one call
@pytest.mark.parametrize("B,L,Hq,Hkv,D,mode,dtype,dm", [
    (64, 16384, 32, 8, 128, "elementwise", "bf16", 4096),   # the decode workload: split-K gate
    (8, 3000, 16, 2, 128, "elementwise", "bf16", 2048),     # split-K gate, fewer batches
    (3, 777, 8, 2, 128, "elementwise", "bf16", 1096),       # ragged d_model tile
    (4, 1000, 8, 2, 128, "headwise", "bf16", 2048),         # one-pass gate (32 columns)
    (2, 500, 8, 2, 64, "elementwise", "bf16", 2048),        # D 64
    (2, 300, 4, 2, 128, "elementwise", "fp32", 256),        # float32
    (2, 300, 4, 2, 128, "none", "bf16", 64),
])
def test_gated_decode_one_call(B, L, Hq, Hkv, D, mode, dtype, dm):
    """gsa_gated_decode against the two calls it stands for (the gate with a
    workspace, then the decode), bitwise, and against the oracle, every batch."""
    cfg = dec_cfg(B, L, Hq, Hkv, D, mode, dtype, dm=dm)
    print(f"  gated decode B{B} L{L} {Hq}/{Hkv}x{D} {mode} {dtype} dm{dm}", flush=True)
    if (B, L) in ((64, 16384), (8, 3000)):
        # few gate rows: the workspace also holds the split-K gate parts
        dws = gsa.decode_workspace_bytes(B, L, Hq, Hkv, D)
        gate_area = gsa.gated_decode_workspace_bytes(B, L, Hq, Hkv, D, dm, mode) - (dws + 255) // 256 * 256
        assert gate_area > B * Hq * D * 4
    inp = make_inputs(cfg, seed=B + L, device=DEV)
    X = None if mode == "none" else inp["X"].reshape(B, dm)
    W = None if mode == "none" else inp["W"]
    Y, guard = guarded_empty(tuple(inp["Q"].shape), inp["Q"].dtype, DEV)
    gsa.gated_decode(X, W, inp["Q"], inp["K"], inp["V"], mode, Y=Y)
    G = None if mode == "none" else gsa.gate_logits(X, W, workspace=True)
    Y2 = gsa.decode(inp["Q"], inp["K"], inp["V"], G, mode)
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Y"
    itype = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(Y.view(itype), Y2.view(itype))
    report(f64(Y), oracle_decode_by_batch(inp, mode), TOL[dtype], f"gated decode {mode} {dtype} B{B} L{L}")


def test_decode_at_the_per_batch_size_limit():
    """The largest cache a batch may hold: the kernels address one batch's K and
    V with 32-bit byte offsets, so L·Hkv·D·4 must stay below 2 GiB.  Here
    L = 2^22 − 8 keys of one 128-dim key/value head (just under the limit), two
    batches, so the second batch's cache starts past 2 GiB into K and V; every
    output against the oracle.  One more key per batch (L = 2^22) is refused."""
    L = (1 << 22) - 8
    cfg = dec_cfg(2, L, 4, 1, 128, "headwise", "bf16", dm=256)
    print(f"  decode B2 L{L} 4/1x128 headwise: generating inputs", flush=True)
    inp = make_inputs(cfg, seed=17, device=DEV)
    # one key per batch that query head 0 attends to almost entirely (key L-3 of
    # batch 1 lies within 2 KB of the end of the cache), so head 0's output is
    # close to that key's value row and a wrong offset shows as an O(1) error
    for b, kb in ((0, (1 << 21) + 5), (1, L - 3)):
        inp["K"][b, kb, 0] = (inp["Q"][b, 0, 0].float() * 4).to(torch.bfloat16)
    Y, _ = run(inp, "headwise")
    assert not torch.isnan(Y.float()).any()
    print("  oracle, one batch at a time", flush=True)
    want = oracle_decode_by_batch(inp, "headwise")
    report(f64(Y), want, TOL["bf16"], f"decode L={L}, 2 batches")
    assert float(np.abs(want[:, 0, 0]).max()) > 0.5   # head 0 really follows its planted key
    del inp, Y
    torch.cuda.empty_cache()
    big = torch.empty((1, 1 << 22, 1, 128), dtype=torch.bfloat16, device=DEV)
    Q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gsa.GsaError) as err:
        gsa.decode(Q, big, big, None, "none")
    assert "exceeds" in str(err.value)
