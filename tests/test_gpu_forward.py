"""Causal gated SDPA forward on the GPU against the fp64 oracle, plus bit-exact
masking / indexing properties."""
import math

import numpy as np
import pytest
import torch

import oracle
import gated_softmax_attention_amd as gsa
from synth import CONFIGS, make_inputs
from helpers import TOL, f64, report, guarded_empty, guard_ok, oracle_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(inp, mode, guard=True):
    Q = inp["Q"]
    G = None if mode == "none" else gsa.gate_logits(inp["X"], inp["W"])
    if guard:
        Y, g = guarded_empty(tuple(Q.shape), Q.dtype, DEV)
    else:
        Y, g = torch.empty_like(Q), None
    gsa.forward(Q, inp["K"], inp["V"], G, mode, Y=Y)
    torch.cuda.synchronize()
    if g is not None:
        assert guard_ok(g), "write past the end of Y"
    return Y, G


def full_oracle(inp, mode):
    return oracle.gated_sdpa(f64(inp["X"]), f64(inp["W"]), f64(inp["Q"]), f64(inp["K"]),
                             f64(inp["V"]), mode)


def small_cfg(B, S, Hq, Hkv, D, mode, dtype, dm=64):
    return CONFIGS["tiny_fp32"].with_(name="t", B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, mode=mode,
                                      dtype=dtype, d_model=dm)


# --------------------------------------------------------------- the tiny fp32 config
@pytest.mark.parametrize("mode", ["elementwise", "headwise", "none"])
def test_tiny_fp32_config(mode):
    cfg = CONFIGS["tiny_fp32"].with_(mode=mode)
    inp = make_inputs(cfg, seed=0, device=DEV)
    Y, _ = run(inp, mode)
    report(f64(Y), full_oracle(inp, mode), TOL["fp32"], f"tiny_fp32 {mode}")


# --------------------------------------------------------------- small shapes, full oracle
CASES = []
for D in (128, 64):
    for (B, S, Hq, Hkv) in [(1, 1, 2, 1), (2, 7, 4, 4), (1, 64, 2, 2), (1, 65, 8, 1), (2, 129, 4, 2),
                            (1, 200, 16, 2), (1, 511, 2, 2), (1, 300, 8, 8)]:
        for mode in ("elementwise", "headwise"):
            CASES.append((B, S, Hq, Hkv, D, mode))
CASES.append((1, 100, 4, 2, 128, "none"))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode", CASES)
def test_small_shapes(B, S, Hq, Hkv, D, mode, dtype):
    cfg = small_cfg(B, S, Hq, Hkv, D, mode, dtype)
    inp = make_inputs(cfg, seed=S * 7 + Hq, device=DEV)
    Y, _ = run(inp, mode)
    report(f64(Y), full_oracle(inp, mode), TOL[dtype], f"{dtype} B{B} S{S} {Hq}/{Hkv} D{D} {mode}")


# --------------------------------------------------------------- bit-exact properties
def bf16_case(S=300, Hq=8, Hkv=2, D=128, B=2, mode="elementwise", seed=3):
    return make_inputs(small_cfg(B, S, Hq, Hkv, D, mode, "bf16"), seed=seed, device=DEV)


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
@pytest.mark.parametrize("D", [128, 64])
def test_row_zero_is_value_times_gate_bitwise(mode, D):
    inp = bf16_case(mode=mode, D=D)
    Y, G = run(inp, mode)
    B, S, Hq, _ = inp["Q"].shape
    grp = Hq // inp["K"].shape[2]
    v0 = inp["V"][:, 0].float().repeat_interleave(grp, dim=1)          # [B, Hq, D]
    g0 = G.view(B, S, -1)[:, 0]
    g0 = g0.view(B, Hq, D) if mode == "elementwise" else g0.view(B, Hq, 1)
    want = (v0 * g0).to(torch.bfloat16)
    assert torch.equal(Y[:, 0].view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("mode", ["elementwise", "headwise"])
def test_saturated_gate_equals_ungated_bitwise(mode):
    inp = bf16_case(mode=mode)
    inp["W"].zero_()
    inp["W"][0, :] = 1.0
    inp["X"][..., 0] = 40.0
    Yg, G = run(inp, mode)
    assert bool((G == 1.0).all())
    Yn, _ = run(inp, "none")
    assert torch.equal(Yg.view(torch.int16), Yn.view(torch.int16))


def test_zero_gate_weight_halves_output_bitwise():
    inp = bf16_case()
    inp["W"].zero_()
    Yg, _ = run(inp, "elementwise")
    Yn, _ = run(inp, "none")
    assert torch.equal(Yg.float(), Yn.float() * 0.5)


@pytest.mark.parametrize("i0", [0, 63, 64, 127, 128, 298])
def test_future_keys_do_not_change_earlier_rows_bitwise(i0):
    inp = bf16_case()
    Y1, _ = run(inp, "elementwise")
    gen = torch.Generator(device=DEV).manual_seed(i0)
    for k in "KV":
        t = inp[k][:, i0 + 1:]
        sgn = torch.where(torch.rand(t.shape, generator=gen, device=DEV) < 0.5, -1.0, 1.0)
        inp[k][:, i0 + 1:] = (1e4 * sgn).to(torch.bfloat16) if k == "K" else (-1e4 * sgn).to(torch.bfloat16)
    Y2, _ = run(inp, "elementwise")
    assert torch.equal(Y1[:, :i0 + 1].view(torch.int16), Y2[:, :i0 + 1].view(torch.int16))
    if i0 + 1 < Y1.shape[1]:
        assert not torch.equal(Y1[:, i0 + 1:], Y2[:, i0 + 1:])


def test_gqa_equals_repeated_kv_mha_bitwise():
    inp = bf16_case(Hq=8, Hkv=2)
    Yg, _ = run(inp, "elementwise")
    rep = dict(inp)
    rep["K"] = inp["K"].repeat_interleave(4, dim=2).contiguous()
    rep["V"] = inp["V"].repeat_interleave(4, dim=2).contiguous()
    Ym, _ = run(rep, "elementwise")
    assert torch.equal(Yg.view(torch.int16), Ym.view(torch.int16))


def test_batch_and_head_permutation_bitwise():
    inp = bf16_case(B=3, Hq=4, Hkv=4)
    Y, _ = run(inp, "elementwise")
    bp = torch.tensor([2, 0, 1], device=DEV)
    hp = torch.tensor([3, 1, 0, 2], device=DEV)
    D = inp["Q"].shape[3]
    per = {
        "X": inp["X"][bp].contiguous(),
        "W": inp["W"].view(-1, 4, D)[:, hp].reshape(inp["W"].shape).contiguous(),
        "Q": inp["Q"][bp][:, :, hp].contiguous(),
        "K": inp["K"][bp][:, :, hp].contiguous(),
        "V": inp["V"][bp][:, :, hp].contiguous(),
    }
    Yp, _ = run(per, "elementwise")
    assert torch.equal(Yp.view(torch.int16), Y[bp][:, :, hp].contiguous().view(torch.int16))


def test_headwise_equals_broadcast_elementwise():
    inp = bf16_case(mode="headwise")
    Yh, _ = run(inp, "headwise")
    D = inp["Q"].shape[3]
    ew = dict(inp)
    ew["W"] = inp["W"].repeat_interleave(D, dim=1).contiguous()
    Ye, _ = run(ew, "elementwise")
    # same gate values (the GEMM's k order does not depend on N) => identical output
    assert torch.equal(Yh.view(torch.int16), Ye.view(torch.int16))


# --------------------------------------------------------------- full-size configs
def check_row0(cfg, inp, Y, G):
    """Row 0 of every (batch, head): a softmax over one key is 1, so the output is
    exactly V[0] times the gate, rounded once (bitwise)."""
    grp = cfg.group
    v0 = inp["V"][:, 0].float().repeat_interleave(grp, dim=1)
    g0 = G.view(cfg.B, cfg.S, -1)[:, 0]
    g0 = g0.view(cfg.B, cfg.Hq, cfg.D) if cfg.mode == "elementwise" else g0.view(cfg.B, cfg.Hq, 1)
    assert torch.equal(Y[:, 0].view(torch.int16), (v0 * g0).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("name", ["dense_prefill", "gqa_prefill", "long_prefill"])
def test_full_size_config_every_element(name):
    """The dense (B 2, S 4096, 16/16 heads, elementwise gate), GQA (B 1, S 8192,
    32/4 heads, headwise gate) and 32k (B 1, S 32768, 16/2 heads, token-0 keys
    ×8, elementwise gate) prefill workloads in the launch the bench times: every
    output element against one oracle evaluation, max-abs ≤ 2e-2; row 0 bitwise."""
    cfg = CONFIGS[name]
    print(f"  {name}: generating inputs", flush=True)
    inp = make_inputs(cfg, seed=0, device=DEV)
    Y, G = run(inp, cfg.mode)
    check_row0(cfg, inp, Y, G)
    print(f"  {name}: oracle over all {cfg.B * cfg.S} rows", flush=True)
    report(f64(Y), full_oracle(inp, cfg.mode), TOL[cfg.dtype], f"{name} every element")


# --------------------------------------------------------------- extremes
def test_long_sequence_near_the_size_limit_sampled():
    """S = 131072 (one batch, 4 query heads on 1 key/value head, headwise gate):
    the last query rows see 131072 keys; sampled rows against the oracle."""
    cfg = CONFIGS["long_prefill"].with_(name="s128k", B=1, S=131072, d_model=64, Hq=4, Hkv=1,
                                        mode="headwise", sink_scale=1.0)
    inp = make_inputs(cfg, seed=5, device=DEV)
    Y, G = run(inp, cfg.mode, guard=False)
    rows = [0, 1, 4095, 65536, 131070, 131071]
    idx = torch.tensor(rows, device=DEV)
    want = oracle_rows(f64(inp["X"][:, idx]), f64(inp["W"]), f64(inp["Q"][:, idx]),
                       f64(inp["K"]), f64(inp["V"]), cfg.mode, rows)
    report(f64(Y[:, idx]), want, TOL["bf16"], "S=131072 sampled rows")
    assert not torch.isnan(Y.float()).any()


def test_forward_at_the_per_batch_size_limit():
    """The largest Q a batch may hold: the kernels address one batch's Q (and
    Y) with 32-bit byte offsets, so S·Hq·D·4 must stay below 2 GiB.  Two batches
    of S = 65528 rows of 64 query heads (8 key/value heads, D 128, headwise
    gate): S·Hq·D·4 is 2^31 − 262144, and the second batch starts 1 GiB into Q
    and Y.  For rows and heads at the largest offsets a key a few positions back
    is made to dominate the row (its key is 4 × the query), so a wrong offset
    shows as an O(1) error; sampled rows of every head against the oracle.
    S = 65536 rows of 64 heads is refused."""
    S = 65528
    cfg = CONFIGS["gqa_prefill"].with_(name="lim", B=2, S=S, d_model=256, Hq=64, Hkv=8, mode="headwise")
    print(f"  forward B2 S{S} 64/8x128 headwise: generating inputs", flush=True)
    inp = make_inputs(cfg, seed=23, device=DEV)
    G = cfg.Hq // cfg.Hkv
    planted = [(S - 1, cfg.Hq - 1), (S - 1, 0), (S // 2, cfg.Hq - 1), (64, 5)]
    for b in range(cfg.B):
        for i, h in planted:
            inp["K"][b, i - 3, h // G] = (inp["Q"][b, i, h].float() * 4).to(torch.bfloat16)
    Y, _ = run(inp, cfg.mode, guard=False)
    assert not torch.isnan(Y.float()).any()
    rows = sorted({0, 1, 64, 127, 128, S // 2, S - 129, S - 2, S - 1})
    idx = torch.tensor(rows, device=DEV)
    print("  oracle on sampled rows", flush=True)
    want = oracle_rows(f64(inp["X"][:, idx]), f64(inp["W"]), f64(inp["Q"][:, idx]),
                       f64(inp["K"]), f64(inp["V"]), cfg.mode, rows)
    report(f64(Y[:, idx]), want, TOL["bf16"], f"S={S}, 64 heads, sampled rows")
    for b in range(cfg.B):   # the planted rows really follow their key
        for i, h in planted:
            assert float(np.abs(want[b, rows.index(i), h]).max()) > 0.5, (b, i, h)
    del inp, Y
    torch.cuda.empty_cache()
    Qbig = torch.empty((1, 65536, 64, 128), dtype=torch.bfloat16, device=DEV)
    Kbig = torch.empty((1, 65536, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gsa.GsaError) as err:
        gsa.forward(Qbig, Kbig, Kbig, None, "none")
    assert "exceeds" in str(err.value)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_scores(dtype):
    """Q and K scaled by 8: scores reach several hundred, rows are nearly one-hot
    and the running maximum moves by large steps."""
    cfg = small_cfg(2, 333, 8, 2, 128, "elementwise", dtype)
    inp = make_inputs(cfg, seed=41, device=DEV)
    for k in ("Q", "K"):
        inp[k] = (inp[k].float() * 8).to(inp[k].dtype)   # exact: a power of two
    Y, _ = run(inp, "elementwise")
    report(f64(Y), full_oracle(inp, "elementwise"), TOL[dtype], f"{dtype} scores x64")
