"""Pins of the fused-projection oracle (oracle.project_qkvg): brute-force loops,
head layout, and the gate part equal to the gate oracle."""
import math

import numpy as np
import pytest

import oracle


def draw(rng, B, S, dm, Hq, Hkv, D, N):
    sc = 1 / math.sqrt(dm)
    return (rng.standard_normal((B, S, dm)), rng.standard_normal((dm, Hq * D)) * sc,
            rng.standard_normal((dm, Hkv * D)) * sc, rng.standard_normal((dm, Hkv * D)) * sc,
            rng.standard_normal((dm, N)) * sc)


@pytest.mark.parametrize("shape", [(1, 3, 5, 2, 1, 3, 6), (2, 4, 7, 4, 2, 2, 4)])
def test_matches_brute_force_loops(shape):
    B, S, dm, Hq, Hkv, D, N = shape
    X, Wq, Wk, Wv, W = draw(np.random.default_rng(sum(shape)), *shape)
    Q, K, V, G = oracle.project_qkvg(X, Wq, Wk, Wv, W, Hq, Hkv, D)
    for b in range(B):
        for i in range(S):
            for h in range(Hq):
                for d in range(D):
                    want = math.fsum(X[b, i, k] * Wq[k, h * D + d] for k in range(dm))
                    assert abs(Q[b, i, h, d] - want) <= 1e-13
            for c in range(Hkv):
                for d in range(D):
                    wk = math.fsum(X[b, i, k] * Wk[k, c * D + d] for k in range(dm))
                    wv = math.fsum(X[b, i, k] * Wv[k, c * D + d] for k in range(dm))
                    assert abs(K[b, i, c, d] - wk) <= 1e-13 and abs(V[b, i, c, d] - wv) <= 1e-13
            for n in range(N):
                z = math.fsum(X[b, i, k] * W[k, n] for k in range(dm))
                assert abs(G[b, i, n] - 1 / (1 + math.exp(-z))) <= 1e-15


def test_gate_part_is_the_gate_oracle_and_none_without_gate():
    X, Wq, Wk, Wv, W = draw(np.random.default_rng(1), 2, 6, 8, 4, 2, 4, 16)
    _, _, _, G = oracle.project_qkvg(X, Wq, Wk, Wv, W, 4, 2, 4)
    assert np.array_equal(G, oracle.sigmoid(oracle.gate_scores(X, W)))
    assert oracle.project_qkvg(X, Wq, Wk, Wv, None, 4, 2, 4)[3] is None


def test_unit_columns_select_input_dims():
    """W_Q = the first Hq·D columns of the identity: head h, dim d is input dim h·D + d."""
    rng = np.random.default_rng(2)
    X = rng.standard_normal((1, 3, 8))
    Wq = np.eye(8)
    Wk = np.eye(8)[:, :4]
    Q, K, V, _ = oracle.project_qkvg(X, Wq, Wk, Wk, None, 4, 2, 2)
    assert np.array_equal(Q[0, :, 1, 0], X[0, :, 2]) and np.array_equal(Q[0, :, 3, 1], X[0, :, 7])
    assert np.array_equal(K[0, :, 1, 1], X[0, :, 3])
