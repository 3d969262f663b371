"""Benchmark of the gated SDPA hot path on one MI355X.

One step = the whole prefill path on the bf16 dense-prefill workload (batch 2,
seq 4096, d_model 2048, 16 query / 16 key-value heads, head dim 128,
elementwise gate): gsa_gate_logits (σ(X·W_θ)) then gsa_forward (causal gated
SDPA).  Inputs are seeded synthetic tensors already resident in HBM.

Reported (one JSON line): whole-step TFLOP/s; the roofline of the dominant
kernel (the gated forward), timed per launch with HIP events on the stream it
runs on; the decode workload (batch 64, one token against a 16384-long KV
cache, 32/8 heads) as GB/s with its own roofline; the backward of the prefill
path (gsa_backward) as TFLOP/s; the fused Q/K/V/gate projection as TFLOP/s;
the gate design-space variants (activation, layout, combine, norm) as whole
steps, and the G2 value gate as GB/s;
the first-token attention diagnostic on the
32k sink-mimicking workload as GB/s; and the fp64 oracle timed on the host
cores on a bounded sample of the prefill workload.
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


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    # The GPU needs about 0.1 s of this load to reach its working clock: after
    # 5 warm-up steps the dense prefill step measured 0.267 ms, after 500 it
    # measured 0.213 ms; these defaults time the settled rate.
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    p.add_argument("--only", choices=["prefill", "decode", "backward", "diagnostic", "projection", "variants"], default=None,
                   help="run one workload's GPU part only (for profiling)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    p.add_argument("--no-backward", action="store_true", help="skip the backward workload")
    p.add_argument("--no-projection", action="store_true", help="skip the fused input projection")
    p.add_argument("--no-variants", action="store_true", help="skip the gate design-space variants")
    p.add_argument("--no-diagnostic", action="store_true",
                   help="skip the first-token attention diagnostic on the long_prefill workload")
    p.add_argument("--no-others", action="store_true",
                   help="skip the gqa_prefill and long_prefill lines (reported beside the headline)")
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


def time_steps(step, kernel_only, steps, warmup, torch):
    """Warm up, then time exactly `steps` whole steps with events at the two ends
    only (events between kernels add a dispatch gap of several microseconds).
    Then time `steps` back-to-back launches of the dominant kernel alone, again
    with one event pair, for its average launch duration.  All events are
    recorded on the current stream, the one the library launches on."""
    for _ in range(warmup):
        step()
    st = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(st)
    for _ in range(steps):
        step()
    t_end.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    k_start = torch.cuda.Event(enable_timing=True)
    k_end = torch.cuda.Event(enable_timing=True)
    k_start.record(st)
    for _ in range(steps):
        kernel_only()
    k_end.record(st)
    torch.cuda.synchronize()
    return total_ms / steps, k_start.elapsed_time(k_end) / steps, wall


def prefill_bench(args, torch, gsa, cfg):
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

    ms, fwd_ms, wall = time_steps(step, kernel_only, args.steps, args.warmup, torch)
    if torch.isnan(Y[:, :64].float()).any():
        raise RuntimeError("NaN in output")
    flops = cfg.total_flops()
    fwd_flops = cfg.attention_flops()
    achieved = fwd_flops / (fwd_ms * 1e-3) / 1e12
    traffic = measured_traffic(f"attn_fwd_{cfg.name}", ["attn_fwd.hip", "common.h"])
    return {
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "wall_s": wall,
        "roofline": {
            "kernel": f"attn_fwd_bf16_kernel<{cfg.D}, {cfg.mode}>",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
            "avg_launch_ms": fwd_ms, "algorithmic_flops_per_launch": fwd_flops,
        },
        "gate_ms_per_step": ms - fwd_ms,
    }


def decode_bench(args, torch, gsa, cfg):
    from synth import make_inputs
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    G = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device="cuda:0")
    Y = torch.empty_like(Q)
    ns = gsa.decode_num_splits(cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.D)
    ws = torch.empty(gsa.decode_workspace_bytes(cfg.B, cfg.L, cfg.Hq, cfg.Hkv, cfg.D),
                     dtype=torch.uint8, device="cuda:0")

    def step():
        gsa.gate_logits(X, W, G=G)
        gsa.decode(Q, K, V, G, cfg.mode, Y=Y, workspace=ws)

    def kernel_only():
        gsa.decode(Q, K, V, G, cfg.mode, Y=Y, workspace=ws)

    ms, dec_ms, wall = time_steps(step, kernel_only, args.steps, args.warmup, torch)
    if torch.isnan(Y.float()).any():
        raise RuntimeError("NaN in decode output")
    nbytes = cfg.decode_bytes()
    # what the decode call itself must move: the cache, q, the fp32 gate and y
    kv = nbytes["kv"] + nbytes["q"] + cfg.B * cfg.N * 4 + nbytes["y"]
    achieved = kv / (dec_ms * 1e-3) / 1e9
    traffic = measured_traffic("decode_split", ["attn_decode.hip", "common.h"])
    return {
        "workload": "decode", "metric": "decode GB/s (% of HBM peak)",
        "value": nbytes["total"] / (ms * 1e-3) / 1e9, "unit": "GB/s",
        "ms_per_step": ms, "pct_of_peak": 100.0 * nbytes["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "config": {"B": cfg.B, "L": cfg.L, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "d_model": cfg.d_model, "mode": cfg.mode, "num_splits": ns},
        "roofline": {
            "kernel": "gsa_decode (split + merge)", "bound": "hbm", "achieved": achieved,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic, "avg_launch_ms": dec_ms, "algorithmic_bytes_per_launch": kv,
        },
    }


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
    ms, _, wall = time_steps(step, lambda: None, args.steps, args.warmup, torch)
    for n in ("dQ", "dK", "dV", "dX", "dW"):
        if not torch.isfinite(holder["g"][n][:64].float()).all():
            raise RuntimeError(f"non-finite {n}")
    flops = cfg.backward_flops()
    achieved = flops / (ms * 1e-3) / 1e12
    return {
        "workload": cfg.name, "metric": "gated causal SDPA backward TFLOP/s (% of bf16 MFMA peak)",
        "value": achieved, "unit": "TFLOP/s", "ms_per_step": ms,
        "pct_of_peak": 100.0 * achieved / PEAK_BF16_TFLOPS,
        "config": {"B": cfg.B, "S": cfg.S, "d_model": cfg.d_model, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "D": cfg.D, "mode": cfg.mode, "causal": True, "flops_per_step": flops},
        "roofline": {
            "kernel": "gsa_backward (prep + dQ + dK/dV + dX + dW kernels)", "bound": "mfma",
            "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None, "avg_launch_ms": ms,
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

    ms, _, wall = time_steps(step, lambda: None, args.steps, args.warmup, torch)
    M, N = cfg.B * cfg.S, Wcat.shape[1]
    flops = 2 * M * cfg.d_model * N
    achieved = flops / (ms * 1e-3) / 1e12
    return {
        "workload": cfg.name, "metric": "fused Q/K/V/gate projection TFLOP/s (% of bf16 MFMA peak)",
        "value": achieved, "unit": "TFLOP/s", "ms_per_step": ms, "pct_of_peak": 100.0 * achieved / PEAK_BF16_TFLOPS,
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

        ms, _, _ = time_steps(step, lambda: None, args.steps, args.warmup, torch)
        flops = cfg.attention_flops() + 2 * cfg.B * cfg.S * cfg.d_model * Wl.shape[1]
        out[f"{layout}/{act}/{combine}/{norm or 'no-norm'}"] = {
            "ms_per_step": ms, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "flops_per_step": flops}
    Nv = cfg.Hkv * cfg.D
    Gv = torch.rand((cfg.B * cfg.S, Nv), dtype=torch.float32, device="cuda:0")
    Vo = torch.empty_like(V)

    def vstep():
        gsa.value_gate(V, Gv, "elementwise", Vout=Vo)

    ms, _, _ = time_steps(vstep, lambda: None, args.steps, args.warmup, torch)
    nbytes = 2 * V.numel() * V.element_size() + Gv.numel() * 4
    out["value_gate_elementwise"] = {
        "ms_per_step": ms, "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s",
        "roofline": {"kernel": "value_gate_kernel", "bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes}}
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

    ms, _, wall = time_steps(step, lambda: None, args.steps, args.warmup, torch)
    F, means = holder["r"]
    e = cfg.elem_bytes()
    rows = cfg.B * cfg.Hq * cfg.S
    nbytes = rows * cfg.D * e + rows * 4 * 2 + cfg.B * cfg.Hkv * cfg.D * e
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": cfg.name, "metric": "first-token attention share, GB/s (% of HBM peak)",
        "value": achieved, "unit": "GB/s", "ms_per_step": ms,
        "mean_first_token_share": float(means[-1].item()),
        "config": {"B": cfg.B, "S": cfg.S, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "token0_key_scale": cfg.sink_scale},
        "roofline": {
            "kernel": "first_token_share_kernel (+ head means)", "bound": "hbm", "achieved": achieved,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
            "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes,
        },
    }


def cpu_baseline(args, torch, cfg):
    """The fp64 oracle, as it is, on a bounded sample of the prefill workload:
    every query row r with r % stride == 0 (all batches and heads), with the
    smallest power-of-two stride whose estimated time fits --cpu-seconds
    (stride 1 = the whole workload)."""
    import numpy as np
    import oracle
    from synth import make_inputs, to_float64_numpy as f64
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    inp = make_inputs(cfg, seed=0, device="cuda:0")
    a = {k: f64(inp[k]) for k in "XWQKV"}
    del inp

    def run(stride):
        rows = np.arange(0, cfg.S, stride)
        t0 = time.perf_counter()
        oracle.gated_sdpa(a["X"], a["W"], a["Q"], a["K"], a["V"], cfg.mode, rows=rows)
        dt = time.perf_counter() - t0
        pairs = int((rows + 1).sum())
        flops = 4 * cfg.D * cfg.B * cfg.Hq * pairs + 2 * cfg.B * len(rows) * cfg.d_model * cfg.N
        return dt, flops, len(rows)

    dt, fl, n = run(64)                       # calibration on 1/64 of the rows
    stride = 1
    while stride < 64 and dt * (64 / stride) > args.cpu_seconds:
        stride *= 2
    dt, fl, n = run(stride)
    # when the whole workload takes well under the budget, time it repeatedly
    # (up to --cpu-seconds in all) for a steadier figure
    reps = 1
    while stride == 1 and dt / reps * (reps + 1) <= args.cpu_seconds and reps < 8:
        more, _, _ = run(1)
        dt += more
        reps += 1
    return {"value": fl * reps / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": dt,
            "sample": f"dense_prefill workload, query rows i % {stride} == 0 ({n} of {cfg.S} rows, "
                      f"all {cfg.B} batches x {cfg.Hq} heads), {reps} run(s): {fl:.3e} algorithmic flops "
                      f"(gate + causal attention) per run in fp64 numpy"}


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

    pcfg = CONFIGS["dense_prefill"]
    dcfg = CONFIGS["decode"]
    out = None
    if args.only == "variants":
        print(json.dumps(variants_bench(args, torch, gsa, pcfg)), flush=True)
        return
    if args.only == "projection":
        pj = projection_bench(args, torch, gsa, pcfg)
        print(json.dumps(dict(pj, n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True,
                              scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic")), flush=True)
        return
    if args.only == "diagnostic":
        dg = diagnostic_bench(args, torch, gsa, CONFIGS["long_prefill"])
        print(json.dumps(dict(dg, n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True,
                              scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic")), flush=True)
        return
    if args.only == "backward":
        bwd = backward_bench(args, torch, gsa, pcfg)
        print(json.dumps(dict(bwd, n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True,
                              scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic")), flush=True)
        return
    if args.only not in ("decode",):
        pre = prefill_bench(args, torch, gsa, pcfg)
        print(f"# prefill: {pre['ms_per_step']:.4f} ms/step, {pre['tflops']:.1f} TFLOP/s; forward "
              f"{pre['roofline']['avg_launch_ms']:.4f} ms = {pre['roofline']['achieved']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        out = {
            "metric": "gated causal SDPA fwd TFLOP/s (gate GEMM + gated forward, % of bf16 MFMA peak)",
            "value": pre["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": pre["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "pct_of_peak": 100.0 * pre["tflops"] / PEAK_BF16_TFLOPS,
            "config": {"workload": "dense_prefill", "B": pcfg.B, "S": pcfg.S, "d_model": pcfg.d_model,
                       "Hq": pcfg.Hq, "Hkv": pcfg.Hkv, "D": pcfg.D, "mode": pcfg.mode,
                       "causal": True, "flops_per_step": pcfg.total_flops()},
            "roofline": pre["roofline"],
            "gate_ms_per_step": pre["gate_ms_per_step"],
        }
    if not args.no_decode and args.only != "prefill":
        dec = decode_bench(args, torch, gsa, dcfg)
        print(f"# decode: {dec['ms_per_step']:.4f} ms/step, {dec['value']:.1f} GB/s; decode call "
              f"{dec['roofline']['avg_launch_ms']:.4f} ms = {dec['roofline']['achieved']:.1f} GB/s",
              file=sys.stderr, flush=True)
        if out is None:
            out = {"metric": dec["metric"], "value": dec["value"], "unit": "GB/s", "n_gpus": 1,
                   "steps": args.steps, "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
                   "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                   "dtype": "bf16", "data": "synthetic", "config": {"workload": "decode"},
                   "roofline": dec["roofline"]}
        else:
            out["decode"] = dec
    if out is not None and not args.no_backward and args.only is None:
        bwd = backward_bench(args, torch, gsa, pcfg)
        torch.cuda.empty_cache()
        print(f"# backward: {bwd['ms_per_step']:.4f} ms/step, {bwd['value']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        out["backward"] = bwd
    if out is not None and not args.no_projection and args.only is None:
        pj = projection_bench(args, torch, gsa, pcfg)
        torch.cuda.empty_cache()
        print(f"# projection: {pj['ms_per_step']*1e3:.1f} us, {pj['value']:.0f} TFLOP/s", file=sys.stderr,
              flush=True)
        out["projection"] = pj
    if out is not None and not args.no_variants and args.only is None:
        vr = variants_bench(args, torch, gsa, pcfg)
        torch.cuda.empty_cache()
        print("# variants: " + ", ".join(f"{k} {v['value']:.0f} {v['unit']}" for k, v in vr["cases"].items()),
              file=sys.stderr, flush=True)
        out["variants"] = vr
    if out is not None and not args.no_diagnostic and args.only is None:
        dg = diagnostic_bench(args, torch, gsa, CONFIGS["long_prefill"])
        torch.cuda.empty_cache()
        print(f"# first-token share (long_prefill): {dg['ms_per_step']*1e3:.1f} us, {dg['value']:.0f} GB/s, "
              f"mean share {dg['mean_first_token_share']:.4f}", file=sys.stderr, flush=True)
        out["first_token_attention"] = dg
    if out is not None and not args.no_others and args.only is None:
        # the other prefill workloads, each its own gate GEMM + forward step
        others = {}
        for name in ("gqa_prefill", "long_prefill"):
            cfg = CONFIGS[name]
            r = prefill_bench(args, torch, gsa, cfg)
            torch.cuda.empty_cache()
            print(f"# {name}: {r['ms_per_step']:.4f} ms/step, {r['tflops']:.1f} TFLOP/s; forward "
                  f"{r['roofline']['avg_launch_ms']:.4f} ms = {r['roofline']['achieved']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            others[name] = {
                "value": r["tflops"], "unit": "TFLOP/s", "ms_per_step": r["ms_per_step"],
                "pct_of_peak": 100.0 * r["tflops"] / PEAK_BF16_TFLOPS,
                "config": {"B": cfg.B, "S": cfg.S, "d_model": cfg.d_model, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                           "D": cfg.D, "mode": cfg.mode, "causal": True,
                           "flops_per_step": cfg.total_flops()},
                "roofline": r["roofline"], "gate_ms_per_step": r["gate_ms_per_step"],
            }
        out["other_prefill"] = others
    if out is not None and not args.no_cpu_baseline and args.only is None:
        print("# timing the oracle on the host ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args, torch, pcfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
