"""The seeded input generator: determinism, shapes, bf16 rounding, token-0 scaling."""
import math

import numpy as np
import pytest
import torch

from synth import CONFIGS, make_inputs, to_float64_numpy


def rne_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) at the bit level."""
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


SMALL = CONFIGS["tiny_fp32"].with_(name="small_bf16", dtype="bf16", S=33, d_model=64, Hq=4, Hkv=2, D=16)


def test_deterministic_and_shapes():
    a = make_inputs(SMALL, seed=0)
    b = make_inputs(SMALL, seed=0)
    c = make_inputs(SMALL, seed=1)
    for k in "XWQKV":
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
    assert not torch.equal(a["Q"], c["Q"])
    assert a["X"].shape == (1, 33, 64) and a["W"].shape == (64, 4 * 16)
    assert a["Q"].shape == (1, 33, 4, 16) and a["K"].shape == (1, 33, 2, 16)
    assert all(a[k].dtype == torch.bfloat16 for k in "XWQKV")


def test_bf16_cast_is_round_to_nearest_even():
    cfg = SMALL
    inp = make_inputs(cfg, seed=0)
    g = torch.Generator().manual_seed(0)
    X32 = torch.randn(1 * 33 * 64, generator=g).numpy()
    W32 = (torch.randn(64 * 64, generator=g) * (1.0 / math.sqrt(64))).numpy()
    got_x = inp["X"].reshape(-1).view(torch.int16).numpy().view(np.uint16)
    got_w = inp["W"].reshape(-1).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_x, rne_bf16_bits(X32))
    assert np.array_equal(got_w, rne_bf16_bits(W32))


def test_rne_helper_on_ties():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32)
    bits = rne_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0 + 2 ** -6, -1.0]


def test_token0_keys_scaled_exactly():
    cfg = SMALL.with_(sink_scale=8.0)
    a = make_inputs(cfg, seed=0)
    b = make_inputs(SMALL, seed=0)
    assert torch.equal(a["K"][:, 0].float(), 8.0 * b["K"][:, 0].float())
    assert torch.equal(a["K"][:, 1:], b["K"][:, 1:]) and torch.equal(a["V"], b["V"])


def test_widening_is_exact():
    t = torch.tensor([1.5, -3.0e38, 1e-40, 0.1], dtype=torch.bfloat16)
    assert np.array_equal(to_float64_numpy(t), t.double().numpy())


def test_config_work_counts():
    c2 = CONFIGS["dense_prefill"]
    assert c2.attention_flops() == 137_472_507_904
    assert c2.gate_flops() == 68_719_476_736
    c3 = CONFIGS["gqa_prefill"]
    assert c3.total_flops() == 551_970_406_400
    c4 = CONFIGS["long_prefill"]
    assert c4.total_flops() == 4_673_058_635_776
    c5 = CONFIGS["decode"]
    assert c5.decode_bytes()["total"] == 4_330_094_592
    assert c5.causal_pairs() == 16384
