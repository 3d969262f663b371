"""First-token attention share on the GPU (gsa_first_token_attention) against
the fp64 oracle on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs
from helpers import f64, report, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# F = exp(s_0 - LSE): an LSE error e changes F by the factor e^{±e}, and F <= 1,
# so the bar is the forward LSE bar (bf16 4e-3, fp32 1e-4).
F_TOL = {"bf16": 4e-3, "fp32": 1e-4}


def small_cfg(B, S, Hq, Hkv, D, dtype, sink=1.0):
    return CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mode="none", dtype=dtype,
                                      d_model=64, sink_scale=sink)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,S,Hq,Hkv,D,sink", [
    (1, 1, 2, 1, 128, 1.0), (2, 129, 4, 2, 128, 1.0), (1, 300, 8, 8, 64, 8.0), (2, 257, 16, 2, 128, 8.0),
    (1, 511, 4, 1, 64, 1.0)])
def test_first_token_share_small(B, S, Hq, Hkv, D, sink, dtype):
    cfg = small_cfg(B, S, Hq, Hkv, D, dtype, sink)
    inp = make_inputs(cfg, seed=S + Hq, device=DEV)
    _, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], None, "none")
    F, means = gsa.first_token_attention(inp["Q"], inp["K"], LSE)
    torch.cuda.synchronize()
    Fw, hm, m = oracle.first_token_attention(f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]))
    label = f"{dtype} B{B} S{S} {Hq}/{Hkv} D{D} sink{sink}"
    report(F.cpu().numpy(), Fw, F_TOL[dtype], f"F {label}")
    report(means.cpu().numpy(), np.append(hm, m), F_TOL[dtype], f"means {label}")


def test_first_token_share_is_deterministic():
    cfg = small_cfg(2, 300, 8, 2, 128, "bf16", 8.0)
    inp = make_inputs(cfg, seed=4, device=DEV)
    _, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], None, "none")
    a = gsa.first_token_attention(inp["Q"], inp["K"], LSE)
    b = gsa.first_token_attention(inp["Q"], inp["K"], LSE)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_first_token_share_long_prefill_full_size_sampled():
    """The 32k sink-mimicking workload (token-0 keys x8, 16/2 heads), sampled rows."""
    cfg = CONFIGS["long_prefill"]
    inp = make_inputs(cfg, seed=0, device=DEV)
    G = gsa.gate_logits(inp["X"], inp["W"])
    _, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, cfg.mode)
    F, means = gsa.first_token_attention(inp["Q"], inp["K"], LSE)
    torch.cuda.synchronize()
    rows = sample_rows(cfg.S)
    Fw, _, _ = oracle.first_token_attention(f64(inp["Q"][:, :]), f64(inp["K"]), f64(inp["V"]), rows=rows)
    report(F[:, :, rows].cpu().numpy(), Fw[:, :, rows], F_TOL["bf16"], "F long_prefill sampled rows")
    # (the means' reduction is checked exactly against the oracle at the small sizes)
    hm = means.cpu().numpy().astype(np.float64)
    assert np.all((hm > 0) & (hm < 1))
    print(f"  long_prefill mean first-token share: {means[-1].item():.4f}", flush=True)
