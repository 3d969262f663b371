"""Backward of the gated path on the GPU (forward LSE output, gsa_backward)
against the fp64 oracle on the same bf16 inputs, plus bit-exact causality."""
import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs, make_grad
from helpers import TOL, f64, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small_cfg(B, S, Hq, Hkv, D, mode, dtype="bf16", dm=64):
    return CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mode=mode,
                                      dtype=dtype, d_model=dm)


# --------------------------------------------------------------- LSE from the forward
LSE_TOL = {"fp32": 1e-4, "bf16": 4e-3}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode", [
    (1, 1, 2, 1, 128, "elementwise"), (2, 129, 4, 2, 128, "headwise"), (1, 300, 8, 8, 64, "elementwise"),
    (1, 200, 16, 2, 128, "none"), (1, 511, 2, 2, 64, "headwise")])
def test_forward_lse(B, S, Hq, Hkv, D, mode, dtype):
    cfg = small_cfg(B, S, Hq, Hkv, D, mode, dtype)
    inp = make_inputs(cfg, seed=S + 11 * Hq, device=DEV)
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    Y0 = gsa.forward(inp["Q"], inp["K"], inp["V"], G, mode)
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, mode)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16) if Y0.dtype == torch.bfloat16 else Y0,
                       Y.view(torch.int16) if Y.dtype == torch.bfloat16 else Y), "forward_lse changed Y"
    _, lse = oracle.sdpa(f64(inp["Q"]), f64(inp["K"]), f64(inp["V"]), return_lse=True)
    report(LSE.cpu().numpy(), lse, LSE_TOL[dtype], f"LSE {dtype} B{B} S{S} {Hq}/{Hkv} D{D}")


# --------------------------------------------------------------- gsa_backward vs the oracle
def bwd_tol(ref):
    """The bf16 bar (2e-2 max-abs) scaled by the gradient's RMS when that exceeds 1:
    every bf16 rounding on the way (g·dY', P, dS, dZ and the output) is relative.
    Used with BWD_REL: an element far above the RMS also carries the RNE
    rounding of its own bf16 output, up to 2^-8 of its magnitude."""
    rms = float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0.0
    return TOL["bf16"] * max(1.0, rms)


BWD_REL = 2.0 ** -8


def run_backward(inp, dY, mode):
    gated = mode != "none"
    G = gsa.gate_logits(inp["X"], inp["W"]) if gated else None
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, mode)
    X = inp["X"] if gated else None
    W = inp["W"] if gated else None
    out = gsa.backward(X, W, G, inp["Q"], inp["K"], inp["V"], Y, LSE, dY, mode)
    torch.cuda.synchronize()
    return out


def check_against_oracle(inp, dY, mode, label):
    out = run_backward(inp, dY, mode)
    ref = oracle.gated_sdpa_backward(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]),
                                     f64(inp["V"]), f64(dY), mode)
    names = ["dQ", "dK", "dV"] + (["dX", "dW"] if mode != "none" else [])
    for n in names:
        want = ref[n]
        got = f64(out[n]).reshape(want.shape)
        report(got, want, bwd_tol(want), f"{label} {n}", rel=BWD_REL)
        nrm = float(np.linalg.norm(want))
        if nrm > 0:   # (a single key makes dQ exactly zero: then only the max-abs bar applies)
            rel = float(np.linalg.norm(got - want)) / nrm
            print(f"  {label} {n}: rms_ref={np.sqrt(np.mean(want ** 2)):.3e} rel_fro={rel:.3e}", flush=True)
            assert rel <= 1e-2, f"{label} {n}: relative Frobenius error {rel:.3e}"
    if mode == "none":
        assert out["dX"] is None and out["dW"] is None


BWD_CASES = []
for D in (128, 64):
    for (B, S, Hq, Hkv, mode) in [(1, 1, 8, 1, "elementwise"), (2, 7, 8, 8, "headwise"),
                                  (1, 64, 2, 2, "elementwise"), (1, 65, 8, 1, "headwise"),
                                  (2, 129, 4, 2, "elementwise"), (1, 200, 16, 2, "headwise"),
                                  (1, 300, 8, 8, "elementwise"), (1, 257, 4, 2, "none")]:
        BWD_CASES.append((B, S, Hq, Hkv, D, mode))


@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode", BWD_CASES)
def test_backward_small_shapes(B, S, Hq, Hkv, D, mode):
    cfg = small_cfg(B, S, Hq, Hkv, D, mode)
    seed = 5 * S + Hq + D
    inp = make_inputs(cfg, seed=seed, device=DEV)
    dY = make_grad(cfg, seed=seed, device=DEV)
    check_against_oracle(inp, dY, mode, f"B{B} S{S} {Hq}/{Hkv} D{D} {mode}")


@pytest.mark.parametrize("dm,mode", [(200, "elementwise"), (136, "headwise"), (1024, "elementwise")])
def test_backward_gate_widths(dm, mode):
    """d_model and token counts that are not multiples of the 128-wide GEMM tiles."""
    cfg = small_cfg(1, 333, 8, 2, 64, mode, dm=dm)
    inp = make_inputs(cfg, seed=dm, device=DEV)
    dY = make_grad(cfg, seed=dm, device=DEV)
    check_against_oracle(inp, dY, mode, f"dm{dm} {mode}")


@pytest.mark.parametrize("S,Hq,Hkv,D,dm", [(512, 2, 2, 128, 512), (1024, 4, 2, 64, 256)])
def test_backward_large_tile_gemms(S, Hq, Hkv, D, dm):
    """Token count, d_model and gate width all multiples of 256: dX and dW_θ take
    the 256 x 256 tile products, dW_θ with 2 and 4 token chunks of partial sums."""
    cfg = small_cfg(1, S, Hq, Hkv, D, "elementwise", dm=dm)
    inp = make_inputs(cfg, seed=S + dm, device=DEV)
    dY = make_grad(cfg, seed=S + dm, device=DEV)
    check_against_oracle(inp, dY, "elementwise", f"S{S} {Hq}/{Hkv} D{D} dm{dm}")


@pytest.mark.parametrize("S,Hq,Hkv", [(8192, 2, 2), (8200, 2, 1)])
def test_backward_long_rows(S, Hq, Hkv):
    """S >= 8192 at D = 128: dK/dV run in eight-wave workgroups of 256 keys,
    whole groups (S 8192, MHA) and sliced ones with float32 partials and a
    ragged last key tile (S 8200, two query heads per key/value head)."""
    cfg = small_cfg(1, S, Hq, Hkv, 128, "elementwise")
    inp = make_inputs(cfg, seed=S, device=DEV)
    dY = make_grad(cfg, seed=S, device=DEV)
    check_against_oracle(inp, dY, "elementwise", f"S{S} {Hq}/{Hkv} D128")


def test_backward_rejects_unsupported():
    cfg = small_cfg(1, 16, 4, 4, 64, "headwise")          # headwise gate width 4: not a multiple of 8
    inp = make_inputs(cfg, seed=1, device=DEV)
    dY = make_grad(cfg, seed=1, device=DEV)
    G = gsa.gate_logits(inp["X"], inp["W"])
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, "headwise")
    with pytest.raises(gsa.GsaError, match="multiples of 8"):
        gsa.backward(inp["X"], inp["W"], G, inp["Q"], inp["K"], inp["V"], Y, LSE, dY, "headwise")
    cfg32 = small_cfg(1, 16, 2, 2, 64, "none", dtype="fp32")
    i32 = make_inputs(cfg32, seed=1, device=DEV)
    Y32, L32 = gsa.forward_lse(i32["Q"], i32["K"], i32["V"], None, "none")
    with pytest.raises(gsa.GsaError, match="BF16"):
        gsa.backward(None, None, None, i32["Q"], i32["K"], i32["V"], Y32, L32, Y32, "none")


# --------------------------------------------------------------- bit-exact causality
def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


def _redraw(t, gen):
    """Seeded N(0,1) values of t's shape and dtype."""
    return torch.randn(tuple(t.shape), generator=gen, device=t.device, dtype=torch.float32).to(t.dtype)


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
def test_backward_causality_bitwise(mode):
    """dQ of rows <= c ignores every token after c; dK, dV of keys > c ignore every
    query row <= c (Q, dY and X of those rows), bit for bit."""
    cfg = small_cfg(2, 300, 8, 2, 128, mode)
    inp = make_inputs(cfg, seed=77, device=DEV)
    dY = make_grad(cfg, seed=77, device=DEV)
    base = run_backward(inp, dY, mode)
    c = 130
    gen = torch.Generator(device=DEV)
    gen.manual_seed(78)
    fut = {k: v.clone() for k, v in inp.items()}
    for k in ("Q", "K", "V", "X"):
        fut[k][:, c + 1:] = _redraw(fut[k][:, c + 1:], gen)
    dYf = dY.clone()
    dYf[:, c + 1:] = -dYf[:, c + 1:]
    a = run_backward(fut, dYf, mode)
    assert torch.equal(_bits(base["dQ"][:, :c + 1]), _bits(a["dQ"][:, :c + 1]))
    past = {k: v.clone() for k, v in inp.items()}
    past["Q"][:, :c + 1] = _redraw(past["Q"][:, :c + 1], gen)
    dYp = dY.clone()
    dYp[:, :c + 1] = 2 * dYp[:, :c + 1]
    p = run_backward(past, dYp, mode)
    for n in ("dK", "dV"):
        assert torch.equal(_bits(base[n][:, c + 1:]), _bits(p[n][:, c + 1:])), n


def test_backward_is_deterministic():
    cfg = small_cfg(1, 257, 8, 2, 128, "elementwise", dm=256)
    inp = make_inputs(cfg, seed=9, device=DEV)
    dY = make_grad(cfg, seed=9, device=DEV)
    a = run_backward(inp, dY, "elementwise")
    b = run_backward(inp, dY, "elementwise")
    for n in ("dQ", "dK", "dV", "dX"):
        assert torch.equal(_bits(a[n]), _bits(b[n])), n
    assert torch.equal(a["dW"].cpu(), b["dW"].cpu())


# --------------------------------------------------------------- full workload size, sampled
@pytest.mark.parametrize("name", ["dense_prefill", "gqa_prefill"])
def test_backward_full_size_sampled(name):
    """gsa_backward on a whole workload, in the launch configuration the bench
    uses for dense_prefill (B 2, S 4096, 16/16 heads, D 128, d_model 2048,
    elementwise gate: one workgroup per key tile and head), and on gqa_prefill
    (B 1, S 8192, 32/4 heads, d_model 4096, headwise gate), where each group's
    eight query heads are cut into slices whose float32 partial dK/dV sums are
    added afterwards.  The oracle computes chosen key/value heads' dQ, dK, dV
    (with every query head of their groups), their dW_θ columns (every token)
    and a sample of dX rows exactly."""
    from helpers import sample_rows
    cfg = CONFIGS[name]
    inp = make_inputs(cfg, seed=0, device=DEV)
    dY = make_grad(cfg, seed=0, device=DEV)
    out = run_backward(inp, dY, cfg.mode)
    kv = [0, cfg.Hkv - 1] if name == "dense_prefill" else [cfg.Hkv - 1]
    rows = sample_rows(cfg.S)
    ref = oracle.gated_sdpa_backward_sampled(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]),
                                             f64(inp["V"]), f64(dY), cfg.mode, kv, rows)
    qh = torch.as_tensor(ref["q_heads"])
    pieces = {
        "dQ": f64(out["dQ"][:, :, qh.to(DEV)]),
        "dK": f64(out["dK"][:, :, kv]),
        "dV": f64(out["dV"][:, :, kv]),
        "dW": f64(out["dW"][:, torch.as_tensor(ref["w_cols"]).to(DEV)]),
        "dX": f64(out["dX"][:, torch.as_tensor(rows).to(DEV)]),
    }
    for n, got in pieces.items():
        want = ref[n]
        report(got, want, bwd_tol(want), f"{name} {n}", rel=BWD_REL)
        rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        print(f"  {name} {n}: rel_fro={rel:.3e}", flush=True)
        assert rel <= 1e-2


# --------------------------------------------------------------- stream order: side stream and graph capture
def test_backward_graph_replay_matches_eager():
    """On an MHA shape (key/value grid not sliced) the eager call runs dQ and dX
    on the library's side stream; captured into a graph, every kernel runs in
    sequence on the capturing stream.  Every replay, with eager work and
    synchronisations between the replays, must give the eager call's bits."""
    cfg = small_cfg(2, 640, 4, 4, 128, "elementwise", dm=256)
    inp = make_inputs(cfg, seed=21, device=DEV)
    dY = make_grad(cfg, seed=21, device=DEV)
    G = gsa.gate_logits(inp["X"], inp["W"])
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, "elementwise")
    args = (inp["X"], inp["W"], G, inp["Q"], inp["K"], inp["V"], Y, LSE, dY, "elementwise")
    eager = gsa.backward(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, as torch advises
        gsa.backward(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = gsa.backward(*args)
    dY2 = -dY
    for rep in range(3):
        other = gsa.backward(*args[:8], dY2, "elementwise")   # eager work between replays
        torch.cuda.synchronize()
        for n in ("dQ", "dK", "dV", "dX"):
            captured[n].zero_()
        graph.replay()
        torch.cuda.synchronize()
        for n in ("dQ", "dK", "dV", "dX"):
            assert torch.equal(_bits(captured[n]), _bits(eager[n])), (rep, n)
        assert torch.equal(captured["dW"].cpu(), eager["dW"].cpu()), rep
        assert not torch.equal(_bits(other["dQ"]), _bits(eager["dQ"]))


def test_backward_on_a_user_stream_orders_its_work():
    """Called on a stream of the caller's, the backward's side-stream kernels are
    joined back to it: work the caller enqueues next on that stream sees the
    finished gradients (copies made right after the call, with no
    synchronisation, equal the gradients of a call on the default stream)."""
    cfg = small_cfg(2, 1100, 8, 8, 128, "elementwise", dm=512)
    inp = make_inputs(cfg, seed=33, device=DEV)
    dY = make_grad(cfg, seed=33, device=DEV)
    ref = run_backward(inp, dY, "elementwise")
    G = gsa.gate_logits(inp["X"], inp["W"])
    Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, "elementwise")
    torch.cuda.synchronize()
    user = torch.cuda.Stream()
    with torch.cuda.stream(user):
        out = gsa.backward(inp["X"], inp["W"], G, inp["Q"], inp["K"], inp["V"], Y, LSE, dY, "elementwise")
        copies = {n: out[n].clone() for n in ("dQ", "dK", "dV", "dX", "dW")}
    torch.cuda.synchronize()
    for n in ("dQ", "dK", "dV", "dX"):
        assert torch.equal(_bits(copies[n]), _bits(ref[n])), n
    assert torch.equal(copies["dW"].cpu(), ref["dW"].cpu())


def test_backward_from_two_host_threads():
    """Two host threads, each with its own stream and inputs, call the backward
    at the same time (the library's side stream and events are shared per
    device, guarded by a lock): each thread's gradients equal those of a call
    made alone, bit for bit."""
    import threading
    cfgs = [small_cfg(2, 700, 8, 8, 128, "elementwise", dm=256), small_cfg(1, 900, 8, 8, 128, "headwise", dm=256)]
    cases = []
    for i, cfg in enumerate(cfgs):
        inp = make_inputs(cfg, seed=50 + i, device=DEV)
        dY = make_grad(cfg, seed=50 + i, device=DEV)
        ref = run_backward(inp, dY, cfg.mode)
        G = gsa.gate_logits(inp["X"], inp["W"])
        Y, LSE = gsa.forward_lse(inp["Q"], inp["K"], inp["V"], G, cfg.mode)
        cases.append((cfg, inp, dY, G, Y, LSE, ref))
    torch.cuda.synchronize()
    results, errors = [None, None], []

    def worker(i):
        try:
            cfg, inp, dY, G, Y, LSE, _ = cases[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(5):
                    out = gsa.backward(inp["X"], inp["W"], G, inp["Q"], inp["K"], inp["V"], Y, LSE, dY, cfg.mode)
                    outs.append({n: out[n].clone() for n in ("dQ", "dK", "dV", "dX", "dW")})
            s.synchronize()
            results[i] = outs
        except Exception as e:   # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (_, _, _, _, _, _, ref) in enumerate(cases):
        for out in results[i]:
            for n in ("dQ", "dK", "dV", "dX"):
                assert torch.equal(_bits(out[n]), _bits(ref[n])), (i, n)
            assert torch.equal(out["dW"].cpu(), ref["dW"].cpu()), i
