"""The gate design-space variants on the GPU against the fp64 oracle: gate
activations (gsa_gate_logits), the head-shared gate (gsa_gate_head_mean: the
mean over the heads of the activated elementwise scores), layouts / combine /
norm (gsa_forward_variant) and G2 value gating (gsa_value_gate + gsa_forward)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import variants as ov
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs
from helpers import TOL, f64, report, sample_rows, guarded_empty, guard_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw_xw(M, dm, N, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    X = torch.randn(M, dm, generator=g, device=DEV).to(dtype)
    W = (torch.randn(dm, N, generator=g, device=DEV) * (3.0 / math.sqrt(dm))).to(dtype)   # logits ~ N(0, 9)
    return X, W


@pytest.mark.parametrize("act", ["identity", "sigmoid", "ns_sigmoid", "silu"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("M,dm,N", [(37, 64, 5), (300, 2048, 256), (64, 4096, 32)])
def test_gate_activations(M, dm, N, dtype, act):
    X, W = draw_xw(M, dm, N, dtype, seed=M + N)
    G = gsa.gate_logits(X, W, activation=act)
    torch.cuda.synchronize()
    want = ov.activation(oracle.gate_scores(f64(X), f64(W)), act)
    # float32 accumulation of at most 4096 exact products: relative 1e-5 of the
    # logits' scale; the activations are 1-Lipschitz up to |z| (SiLU)
    tol = 1e-4 * max(1.0, float(np.abs(want).max()))
    report(G.cpu().numpy(), want, tol, f"{act} {M}x{dm}x{N}")


@pytest.mark.parametrize("act", ["sigmoid", "identity", "silu"])
@pytest.mark.parametrize("M,Hq,D", [(1, 1, 4), (37, 4, 64), (8192, 16, 128), (64, 32, 128), (5, 3, 12)])
def test_gate_head_mean(M, Hq, D, act):
    """Gs = mean over the Hq heads of the activated scores, against the oracle's
    head-shared layout (float32 sums of Hq values: relative error ≤ Hq·2^-24)."""
    dm = 64
    X, W = draw_xw(M, dm, Hq * D, torch.bfloat16, seed=M + Hq)
    G = gsa.gate_logits(X, W, activation=act)
    Gs, guard = guarded_empty((M, D), torch.float32, DEV)
    gsa.gate_head_mean(G, Hq, D, Gs=Gs)
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Gs"
    a = ov.activation(oracle.gate_scores(f64(X), f64(W)), act)[None]          # [1, M, Hq*D]
    want = ov.gate_layout(a, Hq, D, "shared").reshape(M, D)
    tol = 1e-4 * max(1.0, float(np.abs(a).max()))
    report(Gs.cpu().numpy(), want, tol, f"head mean {act} M{M} Hq{Hq} D{D}")


@pytest.mark.parametrize("Hq", [2, 8])
def test_head_mean_of_identical_heads(Hq):
    """With the same weight block for every head, every head's score is the same
    float32 value x, and the gate is the mean of Hq copies of x.  For two heads
    x + x = 2x and 2x / 2 = x exactly, so head-shared equals the head bitwise;
    summing more copies in order rounds (3x needs one more bit), so for eight
    the mean is within 8·2^-24 of x relatively."""
    D, M, dm = 64, 300, 128
    X, W = draw_xw(M, dm, D, torch.bfloat16, seed=4)
    G = gsa.gate_logits(X, W.repeat(1, Hq))
    Gs = gsa.gate_head_mean(G, Hq, D)
    torch.cuda.synchronize()
    x = G[:, :D]
    for h in range(1, Hq):
        assert torch.equal(G[:, h * D:(h + 1) * D], x)       # the GEMM gives every head block the same values
    if Hq == 2:
        assert torch.equal(Gs, x)
    else:
        assert float(((Gs - x).abs() / x.abs()).max()) <= Hq * 2.0 ** -24


ACT_FOR = {("mul", "elementwise"): "sigmoid", ("mul", "headwise"): "ns_sigmoid", ("mul", "shared"): "sigmoid",
           ("add", "elementwise"): "silu", ("add", "headwise"): "sigmoid", ("add", "shared"): "identity"}
CASES = [(layout, combine, norm) for layout in ("elementwise", "headwise", "shared")
         for combine in ("mul", "add") for norm in (None, "rms")] + [("none", "mul", "rms")]


def gate_width(layout, Hq, D):
    """Columns of W_θ: head-shared uses the elementwise width and averages the
    activated scores over the heads (gsa_gate_head_mean)."""
    return {"elementwise": Hq * D, "headwise": Hq, "shared": Hq * D, "none": 0}[layout]


def gate_for(X, W, layout, act, Hq, D):
    G = gsa.gate_logits(X, W, activation=act)
    return gsa.gate_head_mean(G, Hq, D) if layout == "shared" else G


def run_variant(cfg, layout, combine, norm, seed, rows=None):
    inp = make_inputs(cfg.with_(mode="none"), seed=seed, device=DEV)
    N = gate_width(layout, cfg.Hq, cfg.D)
    act = ACT_FOR.get((combine, layout), "sigmoid")
    G = W = None
    if N:
        gx = torch.Generator(device=DEV).manual_seed(seed + 5)
        W = (torch.randn(cfg.d_model, N, generator=gx, device=DEV) / math.sqrt(cfg.d_model)).to(inp["X"].dtype)
        G = gate_for(inp["X"], W, layout, act, cfg.Hq, cfg.D)
    Y = gsa.forward_variant(inp["Q"], inp["K"], inp["V"], G, layout, combine, norm)
    torch.cuda.synchronize()
    want = ov.gated_sdpa_variant(f64(inp["X"]), None if W is None else f64(W), f64(inp["Q"]), f64(inp["K"]),
                                 f64(inp["V"]), layout, act, combine, norm, rows=rows)
    got = f64(Y) if rows is None else f64(Y[:, rows])
    return got, want, act


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("layout,combine,norm", CASES)
def test_forward_variant_small(layout, combine, norm, dtype):
    for (B, S, Hq, Hkv, D) in [(2, 129, 8, 2, 128), (1, 200, 4, 4, 64)]:
        cfg = CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, d_model=64)
        got, want, act = run_variant(cfg, layout, combine, norm, seed=S + Hq)
        # bf16: one rounding of an output of magnitude up to a few units
        tol = TOL[dtype] * max(1.0, float(np.abs(want).max()) / 4)
        report(got, want, tol, f"{dtype} {layout}/{combine}/{norm}/{act} B{B} S{S} {Hq}/{Hkv} D{D}")


def test_default_variant_equals_forward_bitwise():
    cfg = CONFIGS["tiny_fp32"].with_(name="t", B=2, S=300, Hq=8, Hkv=2, D=128, dtype="bf16", d_model=64,
                                     mode="elementwise")
    inp = make_inputs(cfg, seed=3, device=DEV)
    G = gsa.gate_logits(inp["X"], inp["W"])
    a = gsa.forward(inp["Q"], inp["K"], inp["V"], G, "elementwise")
    b = gsa.forward_variant(inp["Q"], inp["K"], inp["V"], G, "elementwise", "mul", None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("layout", ["elementwise", "headwise"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_value_gating_g2(layout, dtype):
    cfg = CONFIGS["tiny_fp32"].with_(name="t", B=2, S=257, Hq=8, Hkv=2, D=128, dtype=dtype, d_model=64,
                                     mode="none")
    inp = make_inputs(cfg, seed=11, device=DEV)
    N = cfg.Hkv * cfg.D if layout == "elementwise" else cfg.Hkv
    gx = torch.Generator(device=DEV).manual_seed(12)
    Wv = (torch.randn(cfg.d_model, N, generator=gx, device=DEV) / math.sqrt(cfg.d_model)).to(inp["X"].dtype)
    Gv = gsa.gate_logits(inp["X"], Wv)
    Vg = gsa.value_gate(inp["V"], Gv, layout)
    Y = gsa.forward(inp["Q"], inp["K"], Vg, None, "none")
    torch.cuda.synchronize()
    want_v = ov.value_gate(f64(inp["X"]), f64(Wv), f64(inp["V"]), layout)
    # the gated values are rounded once to the value dtype
    report(f64(Vg), want_v, 2.0 ** -8 * float(np.abs(want_v).max()) if dtype == "bf16" else 1e-6,
           f"V' {dtype} {layout}")
    want = ov.value_gated_sdpa(f64(inp["X"]), f64(Wv), f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]), layout)
    report(f64(Y), want, TOL[dtype], f"G2 {dtype} {layout}")


def value_gate_inputs(cfg, layout, seed):
    inp = make_inputs(cfg.with_(mode="none"), seed=seed, device=DEV)
    N = cfg.Hkv * cfg.D if layout == "elementwise" else cfg.Hkv
    gx = torch.Generator(device=DEV).manual_seed(seed + 1)
    Wv = (torch.randn(cfg.d_model, N, generator=gx, device=DEV) / math.sqrt(cfg.d_model)).to(inp["X"].dtype)
    return inp, Wv, gsa.gate_logits(inp["X"], Wv)


G2_CASES = [(2, 257, 8, 2, 128), (1, 200, 4, 4, 64), (1, 64, 8, 1, 128), (2, 1000, 16, 4, 128), (1, 129, 2, 2, 64)]


@pytest.mark.parametrize("layout", ["elementwise", "headwise"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", G2_CASES)
def test_value_gating_in_the_forward(B, S, Hq, Hkv, D, dtype, layout):
    """G2 gated as the forward stages its value tiles (gsa_forward_value_gated)
    against the oracle's SDPA over V ⊙ σ(X·W_v), and bitwise equal to the
    separate pass (V' = V ⊙ g rounded once, then the ungated forward): the
    same rounded V' enters the same arithmetic."""
    cfg = CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, d_model=64)
    inp, Wv, Gv = value_gate_inputs(cfg, layout, seed=S + Hq + D)
    Y, guard = guarded_empty(tuple(inp["Q"].shape), inp["Q"].dtype, DEV)
    gsa.forward_value_gated(inp["Q"], inp["K"], inp["V"], Gv, layout, Y=Y)
    Y2 = gsa.forward(inp["Q"], inp["K"], gsa.value_gate(inp["V"], Gv, layout), None, "none")
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Y"
    itype = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(Y.view(itype), Y2.view(itype))
    want = ov.value_gated_sdpa(f64(inp["X"]), f64(Wv), f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]), layout)
    report(f64(Y), want, TOL[dtype], f"G2 in the forward {dtype} {layout} B{B} S{S} {Hq}/{Hkv} D{D}")


@pytest.mark.parametrize("name,layout", [("dense_prefill", "elementwise"), ("gqa_prefill", "headwise")])
def test_value_gating_in_the_forward_full_size(name, layout):
    """The dense (B 2, S 4096, 16/16 heads) and GQA (B 1, S 8192, 32/4 heads)
    prefill shapes with a G2 gate: every output element against the oracle, the
    LSE against the oracle's, and bitwise equal to the separate pass."""
    cfg = CONFIGS[name]
    inp, Wv, Gv = value_gate_inputs(cfg, layout, seed=0)
    LSE = torch.empty((cfg.B, cfg.Hq, cfg.S), dtype=torch.float32, device=DEV)
    Y, LSE = gsa.forward_value_gated(inp["Q"], inp["K"], inp["V"], Gv, layout, LSE=LSE)
    Y2 = gsa.forward(inp["Q"], inp["K"], gsa.value_gate(inp["V"], Gv, layout), None, "none")
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    Vg = ov.value_gate(f64(inp["X"]), f64(Wv), f64(inp["V"]), layout)
    want, lse = oracle.sdpa(f64(inp["Q"]), f64(inp["K"]), Vg, return_lse=True)
    report(f64(Y), want, TOL["bf16"], f"{name} G2 {layout} every element")
    report(LSE.cpu().numpy(), lse, 4e-3, f"{name} G2 LSE")


@pytest.mark.parametrize("name,layout,combine,norm", [("dense_prefill", "shared", "add", "rms"),
                                                     ("dense_prefill", "headwise", "mul", "rms"),
                                                     ("gqa_prefill", "shared", "add", "rms"),
                                                     ("gqa_prefill", "elementwise", "add", None)])
def test_forward_variant_full_size_sampled(name, layout, combine, norm):
    """Full-size prefill workloads (gqa_prefill: S 8192, 32/4 heads, d_model
    4096) through the design-space epilogue, checked on sampled rows."""
    cfg = CONFIGS[name]
    rows = sample_rows(cfg.S)
    got, want, act = run_variant(cfg, layout, combine, norm, seed=0, rows=rows)
    report(got, want, TOL["bf16"] * max(1.0, float(np.abs(want).max()) / 4),
           f"{name} {layout}/{combine}/{norm}/{act} sampled rows")


def run_decode_variant(B, L, Hq, Hkv, D, dtype, layout, combine, norm, seed, num_splits=0):
    cfg = CONFIGS["decode"].with_(name="d", B=B, L=L, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, d_model=64, mode="none")
    inp = make_inputs(cfg, seed=seed, device=DEV)
    N = gate_width(layout, Hq, D)
    act = ACT_FOR.get((combine, layout), "sigmoid")
    G = W = None
    if N:
        gx = torch.Generator(device=DEV).manual_seed(seed + 5)
        W = (torch.randn(cfg.d_model, N, generator=gx, device=DEV) / math.sqrt(cfg.d_model)).to(inp["X"].dtype)
        G = gate_for(inp["X"].reshape(B, cfg.d_model), W, layout, act, Hq, D)
    Y, guard = guarded_empty(tuple(inp["Q"].shape), inp["Q"].dtype, DEV)
    gsa.decode_variant(inp["Q"], inp["K"], inp["V"], G, layout, combine, norm, num_splits=num_splits, Y=Y)
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Y"
    want = ov.gated_sdpa_variant(f64(inp["X"]), None if W is None else f64(W), f64(inp["Q"]), f64(inp["K"]),
                                 f64(inp["V"]), layout, act, combine, norm)
    return f64(Y), want, act


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("layout,combine,norm", CASES)
def test_decode_variant_small(layout, combine, norm, dtype):
    for (B, L, Hq, Hkv, D) in [(3, 777, 8, 2, 128), (2, 65, 4, 4, 64), (1, 1, 4, 1, 128)]:
        got, want, act = run_decode_variant(B, L, Hq, Hkv, D, dtype, layout, combine, norm, seed=L + Hq)
        tol = TOL[dtype] * max(1.0, float(np.abs(want).max()) / 4)
        report(got, want, tol, f"decode {dtype} {layout}/{combine}/{norm}/{act} B{B} L{L} {Hq}/{Hkv} D{D}")


@pytest.mark.parametrize("ns", [1, 3, 16])
def test_decode_variant_split_counts(ns):
    # the RMS norm is taken after the split partials are merged: any split
    # count gives the same head-wide normaliser
    got, want, act = run_decode_variant(2, 2049, 8, 2, 128, "bf16", "shared", "add", "rms", seed=21, num_splits=ns)
    report(got, want, TOL["bf16"] * max(1.0, float(np.abs(want).max()) / 4), f"decode variant splits {ns}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["elementwise", "headwise", "none"])
def test_default_decode_variant_equals_decode_bitwise(mode, dtype):
    cfg = CONFIGS["decode"].with_(name="d", B=3, L=1500, Hq=16, Hkv=4, D=128, dtype=dtype, d_model=64, mode=mode)
    inp = make_inputs(cfg, seed=4, device=DEV)
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    a = gsa.decode(inp["Q"], inp["K"], inp["V"], G, mode)
    b = gsa.decode_variant(inp["Q"], inp["K"], inp["V"], G, mode, "mul", None)
    torch.cuda.synchronize()
    itype = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(a.view(itype), b.view(itype))


@pytest.mark.parametrize("layout,combine,norm", [("shared", "add", "rms"), ("headwise", "mul", None)])
def test_decode_variant_full_size_sampled(layout, combine, norm):
    """The decode workload (B 64, L 16384, 32/8 heads) in the launch bench.py
    times, checked on sampled batches against the oracle."""
    cfg = CONFIGS["decode"].with_(mode="none")
    print("  decode variant: generating inputs", flush=True)
    inp = make_inputs(cfg, seed=2, device=DEV)
    N = gate_width(layout, cfg.Hq, cfg.D)
    act = ACT_FOR[(combine, layout)]
    gx = torch.Generator(device=DEV).manual_seed(7)
    W = (torch.randn(cfg.d_model, N, generator=gx, device=DEV) / math.sqrt(cfg.d_model)).to(inp["X"].dtype)
    G = gate_for(inp["X"].reshape(cfg.B, cfg.d_model), W, layout, act, cfg.Hq, cfg.D)
    Y = gsa.decode_variant(inp["Q"], inp["K"], inp["V"], G, layout, combine, norm)
    torch.cuda.synchronize()
    assert not torch.isnan(Y.float()).any()
    bs = [0, 31, 63]
    want = ov.gated_sdpa_variant(f64(inp["X"][bs]), f64(W), f64(inp["Q"][bs]), f64(inp["K"][bs]),
                                 f64(inp["V"][bs]), layout, act, combine, norm)
    report(f64(Y[bs]), want, TOL["bf16"] * max(1.0, float(np.abs(want).max()) / 4),
           f"decode full size {layout}/{combine}/{norm}, batches {bs}")
