"""Forward, decode and backward on the GPU against the fp64 oracle for shapes
drawn at random (from a fixed seed, so the list is the same on every run):
odd lengths, GQA groups of 1 to 8, both head sizes, every gate mode, gate
widths and d_model off the kernels' tile sizes.  The hand-picked cases in the
other files cover the boundaries one knows of; these cover combinations
nobody listed."""
import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs, make_grad
from helpers import TOL, f64, report, guarded_empty, guard_ok

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
_rng = np.random.RandomState(20261202)


def _heads():
    hkv = int(_rng.choice([1, 2, 3, 4]))
    return hkv * int(_rng.choice([1, 2, 4, 8])), hkv


FWD = []
for _ in range(14):
    Hq, Hkv = _heads()
    FWD.append((int(_rng.randint(1, 4)), int(_rng.randint(1, 420)), Hq, Hkv, int(_rng.choice([64, 128])),
                str(_rng.choice(["elementwise", "headwise", "none"])), str(_rng.choice(["bf16", "bf16", "fp32"])),
                int(_rng.choice([40, 64, 136, 256]))))
DEC = []
for _ in range(8):
    Hq, Hkv = _heads()
    DEC.append((int(_rng.randint(1, 6)), int(_rng.randint(1, 2500)), Hq, Hkv, int(_rng.choice([64, 128])),
                str(_rng.choice(["elementwise", "headwise", "none"])), str(_rng.choice(["bf16", "fp32"]))))
BWD = []
for _ in range(8):
    Hkv = int(_rng.choice([1, 2, 4]))
    Hq = Hkv * int(_rng.choice([1, 2, 4, 8]))
    mode = str(_rng.choice(["elementwise", "headwise", "none"]))
    if mode == "headwise" and Hq % 8:
        mode = "elementwise"          # the backward needs gate widths that are multiples of 8
    BWD.append((int(_rng.randint(1, 3)), int(_rng.randint(1, 330)), Hq, Hkv, int(_rng.choice([64, 128])), mode,
                int(_rng.choice([64, 136, 256]))))


def _cfg(base, **kw):
    return CONFIGS[base].with_(name="r", **kw)


@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode,dtype,dm", FWD)
def test_forward_random_shape(B, S, Hq, Hkv, D, mode, dtype, dm):
    cfg = _cfg("tiny_fp32", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mode=mode, dtype=dtype, d_model=dm)
    inp = make_inputs(cfg, seed=S * 7 + Hq, device=DEV)
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    Y, guard = guarded_empty(tuple(inp["Q"].shape), inp["Q"].dtype, DEV)
    gsa.forward(inp["Q"], inp["K"], inp["V"], G, mode, Y=Y)
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Y"
    want = oracle.gated_sdpa(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]), mode)
    report(f64(Y), want, TOL[dtype], f"fwd B{B} S{S} {Hq}/{Hkv} D{D} {mode} {dtype} dm{dm}")


@pytest.mark.parametrize("B,L,Hq,Hkv,D,mode,dtype", DEC)
def test_decode_random_shape(B, L, Hq, Hkv, D, mode, dtype):
    cfg = _cfg("decode", B=B, L=L, Hq=Hq, Hkv=Hkv, D=D, mode=mode, dtype=dtype, d_model=64)
    inp = make_inputs(cfg, seed=L + 3 * Hq, device=DEV)
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    Y, guard = guarded_empty(tuple(inp["Q"].shape), inp["Q"].dtype, DEV)
    gsa.decode(inp["Q"], inp["K"], inp["V"], G, mode, Y=Y)
    torch.cuda.synchronize()
    assert guard_ok(guard), "write past the end of Y"
    want = oracle.gated_decode(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]), mode)
    report(f64(Y), want, TOL[dtype], f"decode B{B} L{L} {Hq}/{Hkv} D{D} {mode} {dtype}")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode,dm", BWD)
def test_backward_random_shape(B, S, Hq, Hkv, D, mode, dm):
    cfg = _cfg("tiny_fp32", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mode=mode, dtype="bf16", d_model=dm)
    inp = make_inputs(cfg, seed=S * 5 + Hq, device=DEV)
    dY = make_grad(cfg, seed=S * 5 + Hq, device=DEV)
    gated = mode != "none"
    G = gsa.gate_logits(inp["X"], inp["W"]) if gated else None
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, mode)
    out = gsa.backward(inp["X"] if gated else None, inp["W"] if gated else None, G, inp["Q"], inp["K"],
                       inp["V"], Y, LSE, dY, mode)
    torch.cuda.synchronize()
    ref = oracle.gated_sdpa_backward(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]),
                                     f64(inp["V"]), f64(dY), mode)
    for n in ["dQ", "dK", "dV"] + (["dX", "dW"] if gated else []):
        want = ref[n]
        got = f64(out[n]).reshape(want.shape)
        rms = float(np.sqrt(np.mean(np.square(want)))) if want.size else 0.0
        # the backward's bar: bf16 2e-2 scaled by the gradient's RMS, plus the
        # RNE rounding of each bf16 output element (2^-8 of its magnitude)
        report(got, want, TOL["bf16"] * max(1.0, rms), f"bwd B{B} S{S} {Hq}/{Hkv} D{D} {mode} dm{dm} {n}",
               rel=2.0 ** -8)
        nrm = float(np.linalg.norm(want))
        if nrm > 0:
            assert float(np.linalg.norm(got - want)) / nrm <= 1e-2, n
