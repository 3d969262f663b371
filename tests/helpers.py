"""Shared helpers for the GPU parity tests: move seeded inputs, run the oracle
on chosen rows, compare with a stated tolerance and report the worst element."""
import numpy as np
import torch

import oracle
from synth import to_float64_numpy

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def f64(t):
    return to_float64_numpy(t)


def report(got, want, tol, what="", rel=0.0):
    """Assert |got - want| <= tol + rel·|want| elementwise (NaN in got fails);
    print max / mean / worst index.  rel covers a final rounding of the result
    itself, whose error grows with the element's magnitude."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want)
    if np.isnan(err).any():
        idx = np.unravel_index(np.argmax(np.isnan(err)), err.shape)
        raise AssertionError(f"{what}: NaN at {idx}")
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    over = err - rel * np.abs(want)
    idx = np.unravel_index(int(np.argmax(over)), err.shape) if err.size else ()
    worst = float(over[idx]) if err.size else 0.0
    print(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} worst={idx}", flush=True)
    assert worst <= tol, (f"{what}: |err| {err[idx]:.3e} > {tol:.1e} + {rel:.2e}*|ref| at {idx} "
                          f"(got {got[idx]}, want {want[idx]})")
    return mx


def guarded_empty(shape, dtype, device, guard=64):
    """Output buffer pre-filled with NaN, followed by a guard band filled with a sentinel."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), float("nan"), dtype=dtype, device=device)
    buf[n:] = 12345.0
    return buf[:n].view(shape), buf[n:]


def guard_ok(guard):
    return bool((guard == 12345.0).all().item())


def oracle_rows(Xr, W, Qr, K, V, mode, rows):
    """Oracle output of prefill query rows `rows` for every batch, via the per-row
    form: row i is one query at the end of the key prefix [0, i].

    Xr [B, R, dm] and Qr [B, R, Hq, D] hold only the sampled rows (R = len(rows));
    W, K, V are full.  Returns [B, R, Hq, D] float64.
    """
    B = Qr.shape[0]
    out = np.empty(Qr.shape)
    for b in range(B):
        for ri, i in enumerate(rows):
            y = oracle.gated_sdpa(Xr[b:b + 1, ri:ri + 1], W, Qr[b:b + 1, ri:ri + 1],
                                  K[b:b + 1, :i + 1], V[b:b + 1, :i + 1], mode)
            out[b, ri] = y[0, 0]
    return out


def sample_rows(S, extra_random=4, seed=0):
    base = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, S // 2 + 7, S - 129, S - 65, S - 64,
            S - 2, S - 1]
    rng = np.random.default_rng(seed)
    base += [int(x) for x in rng.integers(0, S, size=extra_random)]
    return sorted({r for r in base if 0 <= r < S})


def oracle_decode_by_batch(inp, mode, batches=None):
    """Oracle decode output [B', 1, Hq, D] for every batch (or the listed ones),
    one batch at a time so the fp64 copy of the cache stays one batch's size."""
    X, W, Q, K, V = (inp[k] for k in "XWQKV")
    bl = range(Q.shape[0]) if batches is None else batches
    Wf = f64(W) if W is not None else None
    out = []
    for b in bl:
        out.append(oracle.gated_decode(f64(X[b:b + 1]), Wf, f64(Q[b:b + 1]), f64(K[b:b + 1]),
                                       f64(V[b:b + 1]), mode)[0])
    return np.stack(out)
