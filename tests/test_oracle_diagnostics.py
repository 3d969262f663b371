"""Pins of the first-token attention oracle (oracle.first_token_attention)
against brute force, closed forms, a library softmax and GQA invariants."""
import math

import numpy as np
import pytest
import torch

import oracle


def draw(rng, B, S, Hq, Hkv, D):
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)))


def brute_first_share(Q, K):
    """P_{i,0} by loops: exp(s_i0 - max) / fsum_j exp(s_ij - max) over j <= i."""
    B, S, Hq, D = Q.shape
    G = Hq // K.shape[2]
    out = np.empty((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                s = [math.fsum(Q[b, i, h, d] * K[b, j, h // G, d] for d in range(D)) / math.sqrt(D)
                     for j in range(i + 1)]
                mx = max(s)
                out[b, h, i] = math.exp(s[0] - mx) / math.fsum(math.exp(x - mx) for x in s)
    return out


@pytest.mark.parametrize("shape", [(1, 5, 2, 1, 3), (2, 9, 4, 2, 4), (1, 12, 6, 3, 2)])
def test_matches_brute_force(shape):
    Q, K, V = draw(np.random.default_rng(sum(shape)), *shape)
    F, head_mean, mean = oracle.first_token_attention(Q, K, V)
    want = brute_first_share(Q, K)
    assert np.max(np.abs(F - want)) <= 1e-12
    assert np.max(np.abs(head_mean - want.mean(axis=(0, 2)))) <= 1e-12
    assert abs(mean - want.mean()) <= 1e-12


def test_row_zero_is_one_and_rows_are_probabilities():
    Q, K, V = draw(np.random.default_rng(2), 2, 40, 4, 2, 8)
    F, _, _ = oracle.first_token_attention(Q, K, V)
    # s_00 and the log-sum-exp are rounded on different paths: equal up to an ulp or two
    assert np.max(np.abs(F[:, :, 0] - 1.0)) <= 1e-15
    assert np.all((F > 0) & (F <= 1.0 + 1e-15))


def test_equal_keys_or_zero_queries_share_evenly():
    """All scores of a row equal ⇒ every visible key gets 1/(i+1)."""
    Q, K, V = draw(np.random.default_rng(3), 1, 30, 2, 1, 4)
    want = 1.0 / (np.arange(30) + 1.0)
    Keq = np.repeat(K[:, :1], 30, axis=1)
    F, _, _ = oracle.first_token_attention(Q, Keq, V)
    assert np.max(np.abs(F - want)) <= 1e-14
    F, _, _ = oracle.first_token_attention(np.zeros_like(Q), K, V)
    assert np.max(np.abs(F - want)) <= 1e-14


def test_matches_torch_softmax_column_zero():
    Q, K, V = draw(np.random.default_rng(4), 2, 33, 4, 4, 16)
    F, _, _ = oracle.first_token_attention(Q, K, V)
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)
    k = torch.from_numpy(K).permute(0, 2, 1, 3)
    s = q @ k.transpose(-1, -2) / math.sqrt(16)
    s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
    P = torch.softmax(s, dim=-1)
    assert np.max(np.abs(F - P[..., 0].numpy())) <= 1e-14


def test_gqa_equals_mha_with_repeated_keys():
    Q, K, V = draw(np.random.default_rng(5), 1, 20, 6, 2, 4)
    F, _, _ = oracle.first_token_attention(Q, K, V)
    Fm, _, _ = oracle.first_token_attention(Q, np.repeat(K, 3, axis=2), np.repeat(V, 3, axis=2))
    assert np.max(np.abs(F - Fm)) <= 1e-15


def test_sink_key_takes_the_mass():
    """A first key aligned with every query and scaled up draws almost all attention."""
    rng = np.random.default_rng(6)
    Q, K, V = draw(rng, 1, 16, 1, 1, 8)
    Q[:] = np.abs(Q)
    K[:, 0] = 50.0
    F, _, _ = oracle.first_token_attention(Q, K, V)
    assert np.all(F[:, :, 1:] > 1 - 1e-9)


def test_row_subset_equals_full():
    Q, K, V = draw(np.random.default_rng(7), 2, 50, 4, 2, 8)
    F, _, _ = oracle.first_token_attention(Q, K, V)
    rows = [0, 3, 17, 49]
    Fr, hm, m = oracle.first_token_attention(Q, K, V, rows=rows)
    assert hm is None and m is None
    assert np.array_equal(Fr[:, :, rows], F[:, :, rows])
    assert np.isnan(np.delete(Fr, rows, axis=2)).all()
