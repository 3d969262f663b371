"""Benchmark of the gated SDPA hot path on one MI355X.

One step of the headline = the whole prefill path on the bf16 dense-prefill
workload (batch 2, seq 4096, d_model 2048, 16 query / 16 key-value heads, head
dim 128, elementwise gate): gsa_gate_logits (σ(X·W_θ)) then gsa_forward (causal
gated SDPA).  Every other workload gets its own entry under "workloads": the
GQA prefill (batch 1, seq 8192, 32/4 heads, headwise gate), the 32k prefill
(seq 32768, 16/2 heads, token-0 keys ×8) and the decode step (batch 64, one
token against a 16384-long KV cache, 32/8 heads).  Inputs are seeded synthetic
tensors already resident in HBM.

Timing protocol, the same for every workload:
  * clock settle: the workload's own step runs for --settle seconds (the chip
    needs about 0.1 s of such load to reach its working clock); the length is
    printed as clock_settle_s;
  * --warmup untimed steps, then exactly --steps steps between two HIP events
    on the stream the library launches on (mean = ms_per_step);
  * --steps back-to-back launches of the dominant kernel alone, again between
    two events: its average launch duration, from which roofline.achieved and
    roofline.frac follow;
  * --blocks further blocks of steps (and of kernel launches), each between two
    events: the median and min of the block means.

Also reported: the backward of the prefill path, the fused Q/K/V/gate
projection, the gate design-space variants, the first-token attention
diagnostic, and the fp64 oracle timed on the host cores for every workload
(a process pool over independent (batch, key/value head, query-row range)
pieces), which also gives each workload's max-abs error against the GPU output.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_softmax_attention_amd", "csrc")
PREFILL = ("dense_prefill", "gqa_prefill", "long_prefill")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--settle", type=float, default=0.3,
                   help="seconds of the workload's own step run before warm-up (clock settle)")
    p.add_argument("--blocks", type=int, default=9, help="timed blocks for the median and min")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="oracle time budget per workload; above it a stratified row sample is timed")
    p.add_argument("--only", choices=list(PREFILL) + ["decode", "backward", "diagnostic", "projection", "variants"],
                   default=None, help="run one workload's GPU part only (for profiling)")
    p.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    p.add_argument("--no-others", action="store_true", help="skip the gqa_prefill and long_prefill workloads")
    p.add_argument("--no-backward", action="store_true", help="skip the backward workload")
    p.add_argument("--no-projection", action="store_true", help="skip the fused input projection")
    p.add_argument("--no-variants", action="store_true", help="skip the gate design-space variants")
    p.add_argument("--no-diagnostic", action="store_true",
                   help="skip the first-token attention diagnostic on the long_prefill workload")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run only a plain device copy of this many MiB (HBM counter calibration)")
    return p.parse_args()


def src_hash(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, sources):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != src_hash(*sources):
        return None
    return rec.get("bytes_per_launch")


def _events_ms(fn, n, torch):
    """Mean duration of n back-to-back calls, from two events on the current
    stream (the one the library launches on)."""
    st = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(st)
    for _ in range(n):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def _median(xs):
    ys = sorted(xs)
    m = len(ys) // 2
    return ys[m] if len(ys) % 2 else 0.5 * (ys[m - 1] + ys[m])


def measure(step, kernel, args, torch):
    """The timing protocol of the module docstring.  kernel=None when the step is
    the timed unit itself."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < args.settle:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = _events_ms(step, args.steps, torch)          # the timed region: exactly --steps steps
    wall = time.perf_counter() - wall0
    per_block = max(2, args.steps // 4)
    blocks = [_events_ms(step, per_block, torch) for _ in range(args.blocks)]
    out = {"ms": ms, "median_ms": _median(blocks), "min_ms": min(blocks), "wall_s": wall,
           "settle_s": settle_s, "settle_steps": n, "block_steps": per_block, "blocks": args.blocks}
    if kernel is not None:
        out["kernel_ms"] = _events_ms(kernel, args.steps, torch)
        kb = [_events_ms(kernel, per_block, torch) for _ in range(args.blocks)]
        out["kernel_median_ms"] = _median(kb)
        out["kernel_min_ms"] = min(kb)
    return out


def timing_fields(m):
    return {"statistic": "mean over the timed steps (value, ms_per_step)", "median_ms": m["median_ms"],
            "min_ms": m["min_ms"], "blocks": m["blocks"], "steps_per_block": m["block_steps"],
            "clock_settle_s": round(m["settle_s"], 3), "clock_settle_steps": m["settle_steps"]}


def host_u16(t):
    """A device tensor's raw 16-bit (bf16) or 32-bit (float32) contents on the host."""
    import numpy as np
    t = t.detach().contiguous()
    if t.element_size() == 2:
        import torch
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def prefill_bench(args, torch, gsa, cfg, keep_host=False):
    """One prefill workload: step = gate GEMM + gated forward; dominant kernel =
    the forward.  With keep_host the inputs and the GPU output are copied to
    the host (raw bf16 bits) for the oracle leg."""
    from synth import make_inputs
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    G = torch.empty((cfg.B * cfg.S, cfg.N), dtype=torch.float32, device="cuda:0")
    Y = torch.empty_like(Q)

    def step():
        gsa.gate_logits(X, W, G=G)
        gsa.forward(Q, K, V, G, cfg.mode, Y=Y)

    def kernel_only():
        gsa.forward(Q, K, V, G, cfg.mode, Y=Y)

    m = measure(step, kernel_only, args, torch)
    if torch.isnan(Y.float()).any():
        raise RuntimeError(f"NaN in the {cfg.name} output")
    flops = cfg.total_flops()
    fwd_flops = cfg.attention_flops()
    achieved = fwd_flops / (m["kernel_ms"] * 1e-3) / 1e12
    tflops = flops / (m["ms"] * 1e-3) / 1e12
    r = {
        "workload": cfg.name,
        "metric": "gated causal SDPA TFLOP/s (gate GEMM + gated forward, % of bf16 MFMA peak)",
        "value": tflops, "unit": "TFLOP/s", "ms_per_step": m["ms"],
        "pct_of_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "timing": timing_fields(m),
        "config": {"workload": cfg.name, "B": cfg.B, "S": cfg.S, "d_model": cfg.d_model, "Hq": cfg.Hq,
                   "Hkv": cfg.Hkv, "D": cfg.D, "mode": cfg.mode, "causal": True,
                   "token0_key_scale": cfg.sink_scale, "flops_per_step": flops},
        "roofline": {
            "kernel": f"attn_fwd_bf16_kernel<{cfg.D}, {cfg.mode}>",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(f"attn_fwd_{cfg.name}", ["attn_fwd.hip", "common.h"]),
            "avg_launch_ms": m["kernel_ms"], "median_launch_ms": m["kernel_median_ms"],
            "min_launch_ms": m["kernel_min_ms"], "algorithmic_flops_per_launch": fwd_flops,
        },
        "gate_ms_per_step": m["ms"] - m["kernel_ms"],
    }
    host = None
    if keep_host:
        host = {k: host_u16(inp[k]) for k in "XWQKV"}
        host["Y"] = host_u16(Y)
    return r, host


def decode_bench(args, torch, gsa, cfg, keep_batches=0):
    """The decode workload: step = gate GEMM for the new tokens + gsa_decode
    (split + merge); dominant kernels = the decode call.  keep_batches > 0
    copies that many batches' inputs and output to the host for the oracle leg."""
    from synth import make_inputs
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    G = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device="cuda:0")
    Y = torch.empty_like(Q)
    ns = gsa.decode_num_splits(cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.D)
    X2 = X.reshape(cfg.B, cfg.d_model)
    ws = torch.empty(gsa.gated_decode_workspace_bytes(cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.D, cfg.d_model, cfg.mode),
                     dtype=torch.uint8, device="cuda:0")

    # one call: the gate σ(X·W_θ) (split-K over d_model for the B rows) into
    # the workspace, then the split and merge kernels of the decode
    def step():
        gsa.gated_decode(X2, W, Q, K, V, cfg.mode, Y=Y, workspace=ws)

    # the decode call alone (split + merge, the dominant kernels), on the same gate
    dws = torch.empty(gsa.decode_workspace_bytes(cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.D), dtype=torch.uint8,
                      device="cuda:0")
    G = gsa.gate_logits(X2, W, workspace=True)

    def kernel_only():
        gsa.decode(Q, K, V, G, cfg.mode, Y=Y, workspace=dws)

    m = measure(step, kernel_only, args, torch)
    if torch.isnan(Y.float()).any():
        raise RuntimeError("NaN in decode output")
    nbytes = cfg.decode_bytes()
    # what the decode call itself must move: the cache, q, the fp32 gate and y
    kv = nbytes["kv"] + nbytes["q"] + cfg.B * cfg.N * 4 + nbytes["y"]
    achieved = kv / (m["kernel_ms"] * 1e-3) / 1e9
    gbs = nbytes["total"] / (m["ms"] * 1e-3) / 1e9
    r = {
        "workload": "decode", "metric": "gated decode GB/s (gate GEMM + decode, % of HBM peak)",
        "value": gbs, "unit": "GB/s", "ms_per_step": m["ms"], "pct_of_peak": 100.0 * gbs / PEAK_HBM_GBS,
        "timing": timing_fields(m),
        "config": {"workload": "decode", "B": cfg.B, "L": cfg.L, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "d_model": cfg.d_model, "mode": cfg.mode, "num_splits": ns, "bytes_per_step": nbytes["total"]},
        "roofline": {
            # the library takes 4 key/value heads per split workgroup when 4 divides Hkv
            "kernel": (f"decode_split_bf16_kernel<{cfg.D}, {4 if cfg.Hkv % 4 == 0 else 1}> + "
                       f"decode_merge_bf16_kernel<{cfg.D}> (one gsa_decode call)"),
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic("decode_split", ["attn_decode.hip", "common.h"]),
            "avg_launch_ms": m["kernel_ms"], "median_launch_ms": m["kernel_median_ms"],
            "min_launch_ms": m["kernel_min_ms"], "algorithmic_bytes_per_launch": kv,
        },
        "gate_ms_per_step": m["ms"] - m["kernel_ms"],
    }
    host = None
    if keep_batches:
        nb = min(keep_batches, cfg.B)
        host = {k: host_u16(inp[k][:nb]) for k in "XQKV"}
        host["W"] = host_u16(W)
        host["Y"] = host_u16(Y[:nb])
    return r, host


def backward_bench(args, torch, gsa, cfg):
    """gsa_backward on the prefill workload, from the forward's resident outputs
    (G, Y', LSE) and a seeded upstream gradient.  The timed unit is the whole
    call (prep, dQ, dK/dV, dX and dW kernels); its rocprofv3 split is in profiles/."""
    from synth import make_inputs, make_grad
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    dY = make_grad(cfg, seed=0, device="cuda:0")
    G = gsa.gate_logits(X, W)
    Y, LSE = gsa.forward_lse(Q, K, V, G, cfg.mode)
    ws = torch.empty(gsa.backward_workspace_bytes(cfg.B, cfg.S, cfg.Hq, cfg.Hkv, cfg.D, cfg.d_model,
                                                  cfg.mode), dtype=torch.uint8, device="cuda:0")
    holder = {}

    def step():
        holder["g"] = gsa.backward(X, W, G, Q, K, V, Y, LSE, dY, cfg.mode, workspace=ws)

    # the timed unit is the whole call, so there is no separate kernel-only pass
    m = measure(step, None, args, torch)
    ms = m["ms"]
    for n in ("dQ", "dK", "dV", "dX", "dW"):
        if not torch.isfinite(holder["g"][n][:64].float()).all():
            raise RuntimeError(f"non-finite {n}")
    flops = cfg.backward_flops()
    achieved = flops / (ms * 1e-3) / 1e12
    return {
        "workload": cfg.name, "metric": "gated causal SDPA backward TFLOP/s (% of bf16 MFMA peak)",
        "value": achieved, "unit": "TFLOP/s", "ms_per_step": ms,
        "pct_of_peak": 100.0 * achieved / PEAK_BF16_TFLOPS, "timing": timing_fields(m),
        "config": {"B": cfg.B, "S": cfg.S, "d_model": cfg.d_model, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "D": cfg.D, "mode": cfg.mode, "causal": True, "flops_per_step": flops},
        "roofline": {
            "kernel": "gsa_backward (prep + dQ + dK/dV + dX + dW kernels)", "bound": "mfma",
            "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            # HBM bytes of one call, all its kernels summed
            "traffic": measured_traffic("backward", ["attn_bwd.hip", "gemm_bwd.hip", "common.h"]),
            "avg_launch_ms": ms,
            "algorithmic_flops_per_launch": flops,
        },
    }


def projection_bench(args, torch, gsa, cfg):
    """gsa_project_qkvg: Q, K, V and σ(X·W_θ) from one GEMM over X on the prefill
    workload (W = [W_Q | W_K | W_V | W_θ]).  MFMA-bound: 2·M·d_model·N flop."""
    from synth import make_inputs, make_projection
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    pw = make_projection(cfg, inp["W"], seed=0, device="cuda:0")
    X, Wcat = inp["X"], pw["Wcat"]
    ng = inp["W"].shape[1]
    del inp, pw
    holder = {}

    def step():
        holder["r"] = gsa.project_qkvg(X, Wcat, cfg.Hq, cfg.Hkv, cfg.D, ng)

    m = measure(step, None, args, torch)
    ms = m["ms"]
    M, N = cfg.B * cfg.S, Wcat.shape[1]
    flops = 2 * M * cfg.d_model * N
    achieved = flops / (ms * 1e-3) / 1e12
    return {
        "workload": cfg.name, "metric": "fused Q/K/V/gate projection TFLOP/s (% of bf16 MFMA peak)",
        "value": achieved, "unit": "TFLOP/s", "ms_per_step": ms, "pct_of_peak": 100.0 * achieved / PEAK_BF16_TFLOPS,
        "timing": timing_fields(m),
        "config": {"M": M, "d_model": cfg.d_model, "N": N, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "gate_width": ng, "flops_per_step": flops},
        "roofline": {
            "kernel": "gate_gemm_bf16_big_kernel<true> (routing epilogue)", "bound": "mfma", "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
            "avg_launch_ms": ms, "algorithmic_flops_per_launch": flops,
        },
    }


def variants_bench(args, torch, gsa, cfg):
    """Design-space variants on the prefill workload, each timed as its whole step:
    gate GEMM with the variant's activation, then gsa_forward_variant; and the
    G2 value gate (gsa_value_gate, HBM-bound) as GB/s."""
    from synth import make_inputs
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    Y = torch.empty_like(Q)
    out = {}
    cases = [("elementwise", "sigmoid", "mul", None), ("elementwise", "ns_sigmoid", "mul", "rms"),
             ("elementwise", "silu", "add", None), ("shared", "sigmoid", "mul", None)]
    for layout, act, combine, norm in cases:
        # head-shared uses the elementwise-width W_θ and averages the activated
        # scores over the heads (gsa_gate_head_mean) before the forward
        Wl = W
        G = torch.empty((cfg.B * cfg.S, Wl.shape[1]), dtype=torch.float32, device="cuda:0")
        Gs = torch.empty((cfg.B * cfg.S, cfg.D), dtype=torch.float32, device="cuda:0") if layout == "shared" else G

        def step():
            gsa.gate_logits(X, Wl, G=G, activation=act)
            if layout == "shared":
                gsa.gate_head_mean(G, cfg.Hq, cfg.D, Gs=Gs)
            gsa.forward_variant(Q, K, V, Gs, layout, combine, norm, Y=Y)

        m = measure(step, None, args, torch)
        ms = m["ms"]
        flops = cfg.attention_flops() + 2 * cfg.B * cfg.S * cfg.d_model * Wl.shape[1]
        out[f"{layout}/{act}/{combine}/{norm or 'no-norm'}"] = {
            "ms_per_step": ms, "median_ms": m["median_ms"], "min_ms": m["min_ms"],
            "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "flops_per_step": flops}
    Nv = cfg.Hkv * cfg.D
    Gv = torch.rand((cfg.B * cfg.S, Nv), dtype=torch.float32, device="cuda:0")
    Vo = torch.empty_like(V)

    def vstep():
        gsa.value_gate(V, Gv, "elementwise", Vout=Vo)

    # G2 whole steps: the value gate σ(X·W_v) then attention over V ⊙ g, gated as
    # the forward stages its value tiles, against the separate V' pass
    Wv = W[:, :Nv].contiguous()
    Gvs = torch.empty((cfg.B * cfg.S, Nv), dtype=torch.float32, device="cuda:0")
    Vp = torch.empty_like(V)

    def g2_fused():
        gsa.gate_logits(X, Wv, G=Gvs)
        gsa.forward_value_gated(Q, K, V, Gvs, "elementwise", Y=Y)

    def g2_separate():
        gsa.gate_logits(X, Wv, G=Gvs)
        gsa.value_gate(V, Gvs, "elementwise", Vout=Vp)
        gsa.forward(Q, K, Vp, None, "none", Y=Y)

    g2_flops = cfg.attention_flops() + 2 * cfg.B * cfg.S * cfg.d_model * Nv
    for key, fn in (("g2_value_gate_in_forward", g2_fused), ("g2_value_gate_separate_pass", g2_separate)):
        m = measure(fn, None, args, torch)
        out[key] = {"ms_per_step": m["ms"], "median_ms": m["median_ms"], "min_ms": m["min_ms"],
                    "value": g2_flops / (m["ms"] * 1e-3) / 1e12, "unit": "TFLOP/s", "flops_per_step": g2_flops}
    m = measure(vstep, None, args, torch)
    ms = m["ms"]
    nbytes = 2 * V.numel() * V.element_size() + Gv.numel() * 4
    # back-to-back calls keep this 134 MB working set in the 256 MB last-level
    # cache, so the rate is not an HBM figure and carries no HBM roofline
    out["value_gate_elementwise"] = {
        "ms_per_step": ms, "median_ms": m["median_ms"], "min_ms": m["min_ms"],
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
        "bytes_per_step": nbytes, "kernel": "value_gate_kernel",
        "note": "working set resident in the last-level cache across back-to-back calls: not an HBM rate"}
    return {"workload": cfg.name, "cases": out}


def diagnostic_bench(args, torch, gsa, cfg):
    """gsa_first_token_attention (F = exp(q_i·k_0/√D − LSE_i) per head and row, plus
    per-head means) on the long_prefill workload, whose token-0 keys are scaled ×8
    to mimic an attention sink.  HBM-bound: Q is read once, LSE read and F
    written once."""
    from synth import make_inputs
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    G = gsa.gate_logits(X, W)
    _, LSE = gsa.forward_lse(Q, K, V, G, cfg.mode)
    del G, X
    holder = {}

    def step():
        holder["r"] = gsa.first_token_attention(Q, K, LSE)

    m = measure(step, None, args, torch)
    ms = m["ms"]
    F, means = holder["r"]
    e = cfg.elem_bytes()
    rows = cfg.B * cfg.Hq * cfg.S
    nbytes = rows * cfg.D * e + rows * 4 * 2 + cfg.B * cfg.Hkv * cfg.D * e
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": cfg.name, "metric": "first-token attention share, GB/s (% of HBM peak)",
        "value": achieved, "unit": "GB/s", "ms_per_step": ms, "timing": timing_fields(m),
        "mean_first_token_share": float(means[-1].item()),
        "config": {"B": cfg.B, "S": cfg.S, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "token0_key_scale": cfg.sink_scale},
        "roofline": {
            "kernel": "first_token_share_kernel (+ head means)", "bound": "hbm", "achieved": achieved,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic("first_token", ["attn_diag.hip", "common.h"]),
            "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes,
        },
    }


# ------------------------------------------------------------------ oracle leg
# The fp64 oracle, as it stands, timed on the host cores.  A workload splits
# into independent pieces (batch b, key/value head c with its group of query
# heads, a range of query rows); each piece is the same definition on a
# sub-problem (those queries against keys 0 .. their last position), evaluated
# by one oracle call in a worker process.  Workers are fresh interpreters
# (spawn) that import numpy and the oracle only, never the GPU; inputs reach
# them as memory-mapped files of raw bf16 bits (in /dev/shm when it has room),
# and each writes its rows of the float64 output into a shared mapped file.

_MAPS = {}


def _mapped(path, mode="r"):
    import numpy as np
    key = (path, mode)
    if key not in _MAPS:
        _MAPS[key] = np.load(path, mmap_mode=mode)
    return _MAPS[key]


_READY = None


def _pool_init(barrier=None):
    global _READY
    _READY = barrier
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)      # one BLAS thread per worker: the pool supplies the parallelism
    except Exception:  # pragma: no cover
        pass


def _pool_ready(_):
    """Imports the oracle, then waits for every worker at the barrier: a worker
    held there takes no second task, so each worker runs one of these and all
    have started before the timing begins."""
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = -1
    if _READY is not None:
        _READY.wait(timeout=300)
    return os.getpid(), threads


def _bf16_to_f64(u):
    """Exact widening of raw bf16 bits (uint16) to float64; float32 arrays are widened as they are."""
    import numpy as np
    if u.dtype == np.float32:
        return u.astype(np.float64)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _oracle_piece(t):
    """Oracle output of query rows [q0, q1) of batch b for the query heads of
    key/value head c, against keys [0, k1): the last query sits at key k1 - 1
    (prefill: k1 = q1; decode: one query against the whole cache)."""
    import oracle
    d = t["dir"]
    b, c, q0, q1, k1, G, D, mode = (t[k] for k in ("b", "c", "q0", "q1", "k1", "G", "D", "mode"))
    cols = slice(c * G * D, (c + 1) * G * D) if mode == "elementwise" else slice(c * G, (c + 1) * G)
    X = _bf16_to_f64(_mapped(os.path.join(d, "X.npy"))[b:b + 1, q0:q1])
    W = _bf16_to_f64(_mapped(os.path.join(d, "W.npy"))[:, cols])
    Q = _bf16_to_f64(_mapped(os.path.join(d, "Q.npy"))[b:b + 1, q0:q1, c * G:(c + 1) * G])
    K = _bf16_to_f64(_mapped(os.path.join(d, "K.npy"))[b:b + 1, :k1, c:c + 1])
    V = _bf16_to_f64(_mapped(os.path.join(d, "V.npy"))[b:b + 1, :k1, c:c + 1])
    y = oracle.gated_sdpa(X, W, Q, K, V, mode)
    out = _mapped(os.path.join(d, "out.npy"), "r+")
    out[b, q0:q1, c * G:(c + 1) * G] = y[0]
    out.flush()
    return None


def _row_ranges(S, n, max_rows):
    """Contiguous query-row ranges with about equal causal work (row i costs
    i + 1 pairs), none longer than max_rows."""
    import math
    cuts = sorted({min(S, max(1, round(S * math.sqrt(k / n)))) for k in range(1, n + 1)} | {S})
    ranges, r0 = [], 0
    for r1 in cuts:
        while r1 - r0 > max_rows:
            ranges.append((r0, r0 + max_rows))
            r0 += max_rows
        if r1 > r0:
            ranges.append((r0, r1))
            r0 = r1
    return ranges


def _pieces(cfg, nb, d):
    G = cfg.Hq // cfg.Hkv
    base = {"dir": d, "G": G, "D": cfg.D, "mode": cfg.mode}
    out = []
    if cfg.decode:
        for b in range(nb):
            for c in range(cfg.Hkv):
                out.append(dict(base, b=b, c=c, q0=0, q1=1, k1=cfg.L))
        return out
    for r0, r1 in _row_ranges(cfg.S, 64, 256):
        for b in range(nb):
            for c in range(cfg.Hkv):
                out.append(dict(base, b=b, c=c, q0=r0, q1=r1, k1=r1))
    return out


def _piece_flops(cfg, t):
    """Algorithmic flops of a piece: causal pairs × 4·D per query head, plus its
    gate columns' share of the gate GEMM."""
    G = cfg.Hq // cfg.Hkv
    rows = t["q1"] - t["q0"]
    if cfg.decode:
        pairs = cfg.L
    else:
        pairs = (t["q1"] * (t["q1"] + 1) - t["q0"] * (t["q0"] + 1)) // 2
    ncol = G * cfg.D if cfg.mode == "elementwise" else G
    return 4 * cfg.D * G * pairs + 2 * rows * cfg.d_model * ncol


def cpu_baseline(args, runs, pool_size):
    """Time the oracle per workload on `pool_size` worker processes and compare its
    output with the GPU's.  runs: {name: (cfg, host arrays, GPU entry)}.  When a
    workload's whole oracle would take longer than --cpu-seconds (estimated from
    a calibration pass over a sixteenth of the pieces), a stratified subset of pieces is
    timed and the full time is extrapolated by the ratio of algorithmic flops
    (for prefill: the causal pairs Σ(i+1) plus the gate rows)."""
    import multiprocessing as mp
    import shutil
    import tempfile
    import numpy as np
    per = {}
    ctx = mp.get_context("spawn")
    # one BLAS / OpenMP thread per worker, set before the workers start (the
    # pool supplies the parallelism; hosts may export a larger thread count)
    thread_vars = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in thread_vars}
    os.environ.update({k: "1" for k in thread_vars})
    try:
        barrier = ctx.Barrier(pool_size)
        pool = ctx.Pool(pool_size, initializer=_pool_init, initargs=(barrier,))
        # interpreter start-up and imports, outside the timing: one task per worker
        ready = pool.map(_pool_ready, range(pool_size), chunksize=1)
        print(f"# oracle pool: {len({p for p, _ in ready})} workers, BLAS threads per worker "
              f"{sorted({t for _, t in ready})}", file=sys.stderr, flush=True)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    with pool:
        for name, (cfg, host, gpu) in runs.items():
            need = sum(host[k].nbytes for k in "XWQKVY") * 5      # inputs + float64 output, with margin
            shm_ok = os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > need
            d = tempfile.mkdtemp(prefix="gsa_oracle_", dir="/dev/shm" if shm_ok else None)
            try:
                for k in "XWQKV":
                    np.save(os.path.join(d, f"{k}.npy"), host[k])
                nb = host["Q"].shape[0]
                S_out = 1 if cfg.decode else cfg.S
                out = np.lib.format.open_memmap(os.path.join(d, "out.npy"), mode="w+", dtype=np.float64,
                                                shape=(nb, S_out, cfg.Hq, cfg.D))
                out[:] = np.nan
                out.flush()
                pieces = _pieces(cfg, nb, d)
                total = sum(_piece_flops(cfg, t) for t in pieces)
                # calibration: every 16th piece once to bring the workers' mappings in,
                # then the next interleaved sixteenth for the rate estimate
                pool.map(_oracle_piece, pieces[::16], chunksize=1)
                cal = pieces[8::16] or pieces[:1]
                t0 = time.perf_counter()
                pool.map(_oracle_piece, cal, chunksize=1)
                t_cal = time.perf_counter() - t0
                est = t_cal * total / sum(_piece_flops(cfg, t) for t in cal)
                if est <= args.cpu_seconds:
                    run, extrap = pieces, False
                else:
                    # every step-th piece; at least two per worker so the pool stays busy
                    step = max(1, min(int(np.ceil(est / args.cpu_seconds)), len(pieces) // (2 * pool_size)))
                    run, extrap = pieces[step // 2::step], step > 1
                t0 = time.perf_counter()
                pool.map(_oracle_piece, run, chunksize=1)
                dt = time.perf_counter() - t0
                done = sum(_piece_flops(cfg, t) for t in run)
                want = np.load(os.path.join(d, "out.npy"), mmap_mode="r")
                mask = ~np.isnan(want)                              # the elements the timed pieces wrote
                got = _bf16_to_f64(host["Y"])
                err = np.abs(got[mask] - want[mask])
                full_s = dt * total / done
                # the workload's whole algorithmic work (all batches, when only
                # some were copied to the host) at the measured oracle rate
                work_total = cfg.total_flops() if not cfg.decode else None
                entry = {
                    "oracle_cpu_s": dt, "oracle_cpu_s_full": full_s * (cfg.B / nb),
                    "extrapolated": bool(extrap or nb < cfg.B), "host_cores": pool_size,
                    "fraction_timed": done / total * nb / cfg.B,
                    "pieces_timed": len(run), "pieces_total": len(pieces) * cfg.B // nb,
                    "max_abs_err": float(err.max()), "elements_compared": int(mask.sum()),
                    "batches_on_host": nb,
                }
                if cfg.decode:
                    gbytes = cfg.decode_bytes()["total"]
                    entry.update({"value": gbytes / entry["oracle_cpu_s_full"] / 1e9, "unit": "GB/s",
                                  "gpu_time_us": gpu["ms_per_step"] * 1e3, "gpu_gbps": gpu["value"],
                                  "gpu_pct_hbm": gpu["pct_of_peak"]})
                else:
                    entry.update({"value": work_total / entry["oracle_cpu_s_full"] / 1e12, "unit": "TFLOP/s",
                                  "gpu_time_us": gpu["ms_per_step"] * 1e3, "gpu_tflops": gpu["value"],
                                  "gpu_pct_bf16_peak": gpu["pct_of_peak"]})
                per[name] = entry
                print(f"# oracle {name}: {dt:.2f} s on {pool_size} processes for {entry['fraction_timed']:.3f} "
                      f"of the work; max-abs vs GPU {entry['max_abs_err']:.3e}", file=sys.stderr, flush=True)
                del out, want
                _MAPS.clear()
            finally:
                shutil.rmtree(d, ignore_errors=True)
    return per


def copy_calibration(mib, torch):
    n = mib * (1 << 20)
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    x.fill_(1)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, torch)
        return
    from gated_softmax_attention_amd.build import ensure_built
    ensure_built()   # load what is built; build only when nothing is
    import gated_softmax_attention_amd as gsa
    from synth import CONFIGS
    gsa.load_library()
    torch.cuda.set_device(0)
    common = dict(n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True, scaling="weak",
                  vs_baseline=None, dtype="bf16", data="synthetic")

    single = {"backward": backward_bench, "projection": projection_bench, "variants": variants_bench}
    if args.only in single:
        print(json.dumps(dict(single[args.only](args, torch, gsa, CONFIGS["dense_prefill"]), **common)), flush=True)
        return
    if args.only == "diagnostic":
        print(json.dumps(dict(diagnostic_bench(args, torch, gsa, CONFIGS["long_prefill"]), **common)), flush=True)
        return
    if args.only == "decode":
        r, _ = decode_bench(args, torch, gsa, CONFIGS["decode"])
        print(json.dumps(dict(r, **common)), flush=True)
        return
    if args.only in PREFILL:
        r, _ = prefill_bench(args, torch, gsa, CONFIGS[args.only])
        print(json.dumps(dict(r, **common)), flush=True)
        return

    want_cpu = not args.no_cpu_baseline
    workloads, hosts = {}, {}
    names = ["dense_prefill"] + ([] if args.no_others else ["gqa_prefill", "long_prefill"])
    for name in names:
        r, host = prefill_bench(args, torch, gsa, CONFIGS[name], keep_host=want_cpu)
        torch.cuda.empty_cache()
        print(f"# {name}: {r['ms_per_step']:.4f} ms/step (median {r['timing']['median_ms']:.4f}, min "
              f"{r['timing']['min_ms']:.4f}), {r['value']:.1f} TFLOP/s; forward "
              f"{r['roofline']['avg_launch_ms']:.4f} ms = {r['roofline']['achieved']:.1f} TFLOP/s "
              f"({100 * r['roofline']['frac']:.1f}%)", file=sys.stderr, flush=True)
        workloads[name], hosts[name] = r, host
    if not args.no_decode:
        r, host = decode_bench(args, torch, gsa, CONFIGS["decode"], keep_batches=16 if want_cpu else 0)
        torch.cuda.empty_cache()
        print(f"# decode: {r['ms_per_step']:.4f} ms/step, {r['value']:.1f} GB/s; decode call "
              f"{r['roofline']['avg_launch_ms']:.4f} ms = {r['roofline']['achieved']:.1f} GB/s",
              file=sys.stderr, flush=True)
        workloads["decode"], hosts["decode"] = r, host
    head = workloads["dense_prefill"]
    out = {
        "metric": "gated causal SDPA fwd TFLOP/s (gate GEMM + gated forward, % of bf16 MFMA peak)",
        "value": head["value"], "unit": "TFLOP/s", "ms_per_step": head["ms_per_step"], **common,
        "pct_of_peak": head["pct_of_peak"], "timing": head["timing"], "config": head["config"],
        "roofline": head["roofline"], "gate_ms_per_step": head["gate_ms_per_step"],
        "workloads": workloads,
    }
    if not args.no_backward:
        out["backward"] = backward_bench(args, torch, gsa, CONFIGS["dense_prefill"])
        torch.cuda.empty_cache()
        print(f"# backward: {out['backward']['ms_per_step']:.4f} ms/step, {out['backward']['value']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
    if not args.no_projection:
        out["projection"] = projection_bench(args, torch, gsa, CONFIGS["dense_prefill"])
        torch.cuda.empty_cache()
        print(f"# projection: {out['projection']['ms_per_step'] * 1e3:.1f} us, "
              f"{out['projection']['value']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_variants:
        vr = variants_bench(args, torch, gsa, CONFIGS["dense_prefill"])
        torch.cuda.empty_cache()
        print("# variants: " + ", ".join(f"{k} {v['value']:.0f} {v['unit']}" for k, v in vr["cases"].items()),
              file=sys.stderr, flush=True)
        out["variants"] = vr
    if not args.no_diagnostic:
        dg = diagnostic_bench(args, torch, gsa, CONFIGS["long_prefill"])
        torch.cuda.empty_cache()
        print(f"# first-token share (long_prefill): {dg['ms_per_step'] * 1e3:.1f} us, {dg['value']:.0f} GB/s, "
              f"mean share {dg['mean_first_token_share']:.4f}", file=sys.stderr, flush=True)
        out["first_token_attention"] = dg
    if want_cpu:
        pool_size = max(1, min(len(os.sched_getaffinity(0)), 16))
        print(f"# timing the oracle on {pool_size} host processes ...", file=sys.stderr, flush=True)
        runs = {n: (CONFIGS[n], hosts[n], workloads[n]) for n in workloads}
        per = cpu_baseline(args, runs, pool_size)
        h = per["dense_prefill"]
        out["cpu_baseline"] = {
            "value": h["value"], "unit": "TFLOP/s", "cores": pool_size, "kind": "oracle",
            "sample": (f"dense_prefill workload, fp64 numpy oracle on {pool_size} processes (one BLAS thread "
                       f"each) over (batch, key/value head, query-row range) pieces: "
                       + ("the whole workload" if not h["extrapolated"] else
                          f"{h['fraction_timed']:.3f} of its work, extrapolated by algorithmic flops")
                       + f", {h['oracle_cpu_s']:.2f} s; max-abs vs GPU {h['max_abs_err']:.2e}"),
            "per_workload": per,
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
