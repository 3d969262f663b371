"""Gate projection σ(X·W_θ) on the GPU against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import variants as ov
import gated_softmax_attention_amd as gsa
from helpers import f64, report, guarded_empty, guard_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw(M, dm, N, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    X = torch.randn(M, dm, generator=g, device=DEV).to(dtype)
    W = (torch.randn(dm, N, generator=g, device=DEV) / math.sqrt(dm)).to(dtype)
    return X, W


SHAPES = [(1, 8, 1), (37, 64, 5), (130, 136, 129), (257, 256, 256), (64, 4096, 32),
          (300, 2048, 200), (128, 256, 256), (8192, 64, 8)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("M,dm,N", SHAPES)
def test_gate_scores_and_logits(M, dm, N, dtype):
    X, W = draw(M, dm, N, dtype, seed=M + dm + N)
    G, guard = guarded_empty((M, N), torch.float32, DEV)
    gsa.gate_logits(X, W, G=G)
    Z, guard2 = guarded_empty((M, N), torch.float32, DEV)
    gsa.gate_logits(X, W, G=Z, apply_sigmoid=False)
    torch.cuda.synchronize()
    assert guard_ok(guard) and guard_ok(guard2)
    z_ref = oracle.gate_scores(f64(X), f64(W))
    report(Z.cpu().numpy(), z_ref, 1e-4, f"logits {M}x{dm}x{N}")
    report(G.cpu().numpy(), oracle.sigmoid(z_ref), 1e-4, f"gate {M}x{dm}x{N}")


def test_gate_saturation_and_half_are_exact():
    M, dm, N = 65, 64, 40
    X = torch.zeros(M, dm, device=DEV, dtype=torch.bfloat16)
    W = torch.zeros(dm, N, device=DEV, dtype=torch.bfloat16)
    X[:, 0] = 40.0
    W[0, :] = 1.0
    G = gsa.gate_logits(X, W)
    assert bool((G == 1.0).all())
    G0 = gsa.gate_logits(X, torch.zeros_like(W))
    assert bool((G0 == 0.5).all())
    X[:, 0] = -40.0
    Gn = gsa.gate_logits(X, W).cpu().numpy()
    assert np.all(np.abs(Gn - math.exp(-40.0)) <= 1e-3 * math.exp(-40.0))


# --------------------------------------------------------------- split-K path for few rows
SPLITK = [(64, 4096, 4096), (1, 2048, 64), (37, 2000, 520), (128, 2048, 1024), (64, 4096, 136), (100, 3080, 4096)]


@pytest.mark.parametrize("act", ["sigmoid", "identity", "silu"])
@pytest.mark.parametrize("M,dm,N", SPLITK)
def test_gate_split_k(M, dm, N, act):
    """gsa_gate_logits_ws on few-row shapes (the decode gate: 64 rows, d_model =
    N = 4096): partial logits over d_model parts, added in part order, then the
    activation.  Against the oracle (float32 accumulation of exact products:
    1e-4 of the logits' scale), bitwise reproducible across calls, and within
    the same bar of the one-pass kernel."""
    X, W = draw(M, dm, N, torch.bfloat16, seed=M * 7 + N)
    need = gsa.gate_logits_workspace_bytes(M, dm, N)
    assert need > 0, "this shape should take the split-K path"
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)   # stale contents do not matter
    G, guard = guarded_empty((M, N), torch.float32, DEV)
    gsa.gate_logits(X, W, G=G, activation=act, workspace=ws)
    G2 = gsa.gate_logits(X, W, activation=act, workspace=ws)
    G1 = gsa.gate_logits(X, W, activation=act)                  # the one-pass kernel
    torch.cuda.synchronize()
    assert guard_ok(guard)
    assert torch.equal(G, G2)
    want = ov.activation(oracle.gate_scores(f64(X), f64(W)), act)
    tol = 1e-4 * max(1.0, float(np.abs(want).max()))
    report(G.cpu().numpy(), want, tol, f"split-K {act} {M}x{dm}x{N}")
    report(G.cpu().numpy(), G1.cpu().numpy(), 2 * tol, f"split-K vs one-pass {act} {M}x{dm}x{N}")


def test_gate_split_k_workspace_rules():
    assert gsa.gate_logits_workspace_bytes(8192, 2048, 2048) == 0       # enough tiles: one pass
    assert gsa.gate_logits_workspace_bytes(64, 4096, 32) == 0           # too narrow for 64-column tiles
    assert gsa.gate_logits_workspace_bytes(64, 4096, 4096) == 4 * 64 * 4096 * 4
    X, W = draw(64, 4096, 4096, torch.bfloat16, seed=3)
    with pytest.raises(gsa.GsaError, match="WORKSPACE"):
        gsa.gate_logits(X, W, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    # a shape without the split-K path ignores the workspace: same as gsa_gate_logits
    X2, W2 = draw(300, 256, 256, torch.bfloat16, seed=4)
    a = gsa.gate_logits(X2, W2, workspace=True)
    b = gsa.gate_logits(X2, W2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
