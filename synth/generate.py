"""Seeded input generation.

Recipe (one torch.Generator on the target device, seeded once): draw float32
standard normals in the order X, W_theta, Q, K, V; scale W_theta by
1/sqrt(d_model); cast to the config's dtype (bf16 by round-to-nearest-even);
then multiply the keys of token 0 by ``sink_scale`` (a power of two, so exact in
bf16).  For decode the query tensors have one token per batch and K, V are the
cache of length L, which already holds the current token.

Draws made on a CUDA generator differ from CPU draws with the same seed; each is
deterministic for its device.  Callers that compare against the oracle copy the
device tensors back to the host, so both sides always see identical values.
"""
import math

import numpy as np
import torch

from .configs import Config

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _randn(shape, gen, device, dtype, scale=1.0, chunk=1 << 26):
    """Standard normals drawn in float32 chunk by chunk (bounded host memory), scaled, cast."""
    n = math.prod(shape)
    out = torch.empty(n, dtype=dtype, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        t = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        out[s:e] = t.to(dtype)
    return out.view(shape)


def make_inputs(cfg: Config, seed: int = 0, device="cpu"):
    """Return dict X [B,S,dm], W [dm,N], Q [B,S,Hq,D], K,V [B,Skv,Hkv,D] on ``device``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = _DT[cfg.dtype]
    S, Skv = cfg.S, cfg.Skv
    X = _randn((cfg.B, S, cfg.d_model), gen, device, dt)
    N = cfg.N if cfg.N > 0 else cfg.Hq * cfg.D
    W = _randn((cfg.d_model, N), gen, device, dt, scale=1.0 / math.sqrt(cfg.d_model))
    Q = _randn((cfg.B, S, cfg.Hq, cfg.D), gen, device, dt)
    K = _randn((cfg.B, Skv, cfg.Hkv, cfg.D), gen, device, dt)
    V = _randn((cfg.B, Skv, cfg.Hkv, cfg.D), gen, device, dt)
    if cfg.sink_scale != 1.0:
        K[:, 0, :, :] *= cfg.sink_scale
    return {"X": X, "W": W, "Q": Q, "K": K, "V": V}


def make_grad(cfg: Config, seed: int = 0, device="cpu"):
    """Upstream gradient dY' [B,S,Hq,D] ~ N(0,1) in the config's dtype, from its own
    generator seeded with ``seed + 1_000_003`` (independent of make_inputs' draws)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1_000_003)
    return _randn((cfg.B, cfg.S, cfg.Hq, cfg.D), gen, device, _DT[cfg.dtype])


def make_projection(cfg: Config, W, seed: int = 0, device="cpu"):
    """Projection weights W_Q [dm, Hq·D], W_K and W_V [dm, Hkv·D] ~ N(0, 1/dm) (variance,
    as W_θ) in the config's dtype, from their own generator seeded with
    ``seed + 2_000_003`` (drawn in that order), and the concatenation
    [W_Q | W_K | W_V | W] the fused projection reads (W is the gate weight from
    make_inputs; None for no gate)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 2_000_003)
    dt = _DT[cfg.dtype]
    sc = 1.0 / math.sqrt(cfg.d_model)
    Wq = _randn((cfg.d_model, cfg.Hq * cfg.D), gen, device, dt, scale=sc)
    Wk = _randn((cfg.d_model, cfg.Hkv * cfg.D), gen, device, dt, scale=sc)
    Wv = _randn((cfg.d_model, cfg.Hkv * cfg.D), gen, device, dt, scale=sc)
    parts = [Wq, Wk, Wv] + ([] if W is None else [W])
    return {"Wq": Wq, "Wk": Wk, "Wv": Wv, "Wcat": torch.cat(parts, dim=1).contiguous()}


def make_decode_inputs(cfg: Config, seed: int = 0, device="cpu"):
    """Decode inputs: X [B,1,dm], W, Q [B,1,Hq,D], K,V cache [B,L,Hkv,D]."""
    assert cfg.decode
    return make_inputs(cfg, seed, device)


def to_float64_numpy(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a float32 or bfloat16 tensor to a float64 numpy array."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.numpy().astype(np.float64)
