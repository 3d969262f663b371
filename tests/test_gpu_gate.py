"""Gate projection σ(X·W_θ) on the GPU against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
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
