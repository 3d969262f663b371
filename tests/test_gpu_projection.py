"""Fused input projection (gsa_project_qkvg) on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs, make_projection
from helpers import f64, report, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_bf16(got, want, label):
    """Q, K and V are rounded once to bf16 from float32 accumulators: within
    2^-8·|ref| (half an ulp at the bottom of a binade, the round-to-nearest
    bound) plus 1e-4 for the float32 accumulation, of the exact value."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    excess = np.abs(got - want) - (2.0 ** -8 * np.abs(want) + 1e-4)
    i = np.unravel_index(int(np.argmax(excess)), excess.shape)
    print(f"  {label}: max_abs={np.abs(got - want).max():.3e} worst_excess={excess[i]:.3e} at {i}", flush=True)
    assert excess[i] <= 0, f"{label}: {got[i]} vs {want[i]}"


def run(cfg, seed, rows=None):
    inp = make_inputs(cfg, seed=seed, device=DEV)
    W = None if cfg.mode == "none" else inp["W"]
    pw = make_projection(cfg, W, seed=seed, device=DEV)
    ng = 0 if W is None else W.shape[1]
    Q, K, V, G = gsa.project_qkvg(inp["X"], pw["Wcat"], cfg.Hq, cfg.Hkv, cfg.D, ng)
    torch.cuda.synchronize()
    X = f64(inp["X"]) if rows is None else f64(inp["X"][:, rows])
    Qr, Kr, Vr, Gr = oracle.project_qkvg(X, f64(pw["Wq"]), f64(pw["Wk"]), f64(pw["Wv"]),
                                         None if W is None else f64(W), cfg.Hq, cfg.Hkv, cfg.D)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, rows])
    label = f"{cfg.name} B{cfg.B} S{cfg.S} dm{cfg.d_model} {cfg.Hq}/{cfg.Hkv} D{cfg.D} {cfg.mode}"
    check_bf16(f64(sel(Q)), Qr, f"Q {label}")
    check_bf16(f64(sel(K)), Kr, f"K {label}")
    check_bf16(f64(sel(V)), Vr, f"V {label}")
    if W is None:
        assert G is None
    else:
        Gv = G.view(cfg.B, cfg.S, -1)
        report(sel(Gv).cpu().numpy(), Gr, 1e-4, f"G {label}")
    return inp, G


def small_cfg(B, S, dm, Hq, Hkv, D, mode):
    return CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, d_model=dm, Hq=Hq, Hkv=Hkv, D=D, mode=mode,
                                      dtype="bf16")


@pytest.mark.parametrize("B,S,dm,Hq,Hkv,D,mode", [
    (1, 1, 64, 8, 8, 64, "headwise"), (1, 37, 136, 4, 2, 64, "elementwise"), (2, 129, 256, 8, 1, 128, "headwise"),
    (1, 300, 512, 16, 2, 128, "elementwise"), (2, 257, 64, 2, 2, 128, "none"), (1, 520, 1024, 8, 8, 64, "headwise")])
def test_projection_small(B, S, dm, Hq, Hkv, D, mode):
    run(small_cfg(B, S, dm, Hq, Hkv, D, mode), seed=S + dm)


def test_projection_gate_equals_gate_logits_bitwise():
    """With an elementwise gate the gate columns go through the same large-tile
    kernel and summation order as gsa_gate_logits."""
    cfg = small_cfg(1, 512, 512, 4, 2, 128, "elementwise")
    inp, G = run(cfg, seed=3)
    G2 = gsa.gate_logits(inp["X"], inp["W"])
    torch.cuda.synchronize()
    assert torch.equal(G, G2)


@pytest.mark.parametrize("name", ["dense_prefill", "gqa_prefill"])
def test_projection_full_size_sampled(name):
    cfg = CONFIGS[name]
    run(cfg, seed=0, rows=sample_rows(cfg.S))
