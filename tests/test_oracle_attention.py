"""Pins of the oracle's attention forward (oracle.attention).

Each pin fixes the result from something other than the oracle's own
formula: inputs built so the scores are known exactly (one-hot queries and
keys), closed forms (a single visible key, uniform weights, two keys), the
BSHD layout through token- and head-dependent values, invariants of the
softmax (joint key permutation, a common shift of every score, scale folding),
and overflow safety.  The mutation tests plant slips these must catch.
"""
import math

import numpy as np
import pytest

import oracle
from tiled_dense_gemm_tg_amd import inputs as I

F16, BF16 = I.F16, I.BF16


def _bits(values, dtype):
    return I.values_bits(np.asarray(values, dtype=np.float64), dtype)


def _onehot_scores(Sk, D, coeffs, dtype, q_scale=1.0):
    """Q = q_scale * e_0 (one query row), K_j = coeffs[j] * e_0: the score of
    key j is exactly scale * q_scale * coeffs[j]."""
    Q = np.zeros((1, 1, 1, D))
    Q[0, 0, 0, 0] = q_scale
    K = np.zeros((1, Sk, 1, D))
    K[0, :, 0, 0] = coeffs
    return _bits(Q, dtype), _bits(K, dtype)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_causal_first_query_sees_only_the_first_key(dtype):
    B, S, H, D = 2, 9, 3, 32
    Q = I.random_bits((B, S, H, D), ("normal", 0.0, 1.0), dtype, 1)
    K = I.random_bits((B, S, H, D), ("normal", 0.0, 1.0), dtype, 2)
    V = I.random_bits((B, S, H, D), ("normal", 0.0, 1.0), dtype, 3)
    qs = [(b, 0, h) for b in range(B) for h in range(H)]
    ref64, refq = oracle.attention(B, S, S, H, D, dtype, Q, K, V, causal=True, queries=qs)
    v = V.reshape(B, S, H, D)
    for r, (b, _, h) in enumerate(qs):
        assert np.array_equal(refq[r], v[b, 0, h])
        assert np.array_equal(ref64[r], oracle.decode(dtype, v[b, 0, h]))


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_average_the_visible_values(dtype, causal):
    """K = 0: every score is 0, so O is the plain mean of V over the visible keys;
    V[b, j, h, :] = 100 b + 10 h + j pins the BSHD indexing of V."""
    B, S, H, D = 2, 12, 3, 8
    Q = I.random_bits((B, S, H, D), ("normal", 0.0, 1.0), dtype, 4)
    K = _bits(np.zeros((B, S, H, D)), dtype)
    b, j, h = np.meshgrid(np.arange(B), np.arange(S), np.arange(H), indexing="ij")
    vals = (100 * b + 10 * h + j).astype(np.float64)
    V = _bits(np.repeat(vals[..., None], D, axis=3), dtype)
    assert np.array_equal(oracle.decode(dtype, V).reshape(B, S, H, D)[..., 0], vals)   # exact in both formats
    ref64, _ = oracle.attention(B, S, S, H, D, dtype, Q, K, V, causal=causal)
    ref = ref64.reshape(B, S, H, D)
    for bb in range(B):
        for i in range(S):
            for hh in range(H):
                nk = i + 1 if causal else S
                expect = 100 * bb + 10 * hh + (nk - 1) / 2.0
                assert np.allclose(ref[bb, i, hh], expect, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_two_keys_closed_form(dtype):
    """Scores a and b exactly; O = V0 + (V1 - V0) / (1 + exp(a - b))."""
    D = 16
    a, b = 0.75, -1.5
    Q, K = _onehot_scores(2, D, [a, b], dtype)
    V = I.random_bits((1, 2, 1, D), ("normal", 0.0, 1.0), dtype, 5)
    v = oracle.decode(dtype, V).reshape(2, D)
    ref64, _ = oracle.attention(1, 1, 2, 1, D, dtype, Q, K, V, scale=1.0)
    w1 = 1.0 / (1.0 + math.exp(a - b))
    assert np.allclose(ref64[0], v[0] + (v[1] - v[0]) * w1, rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_value():
    dtype = F16
    D, Sk = 16, 20
    coeffs = np.zeros(Sk)
    coeffs[13] = 64.0                  # score 64 against 0 everywhere else: weights e^-64
    Q, K = _onehot_scores(Sk, D, coeffs, dtype)
    V = I.random_bits((1, Sk, 1, D), ("normal", 0.0, 1.0), dtype, 6)
    ref64, refq = oracle.attention(1, 1, Sk, 1, D, dtype, Q, K, V, scale=1.0)
    assert np.array_equal(refq[0], V.reshape(Sk, D)[13])


def test_scale_multiplies_every_score():
    """scale 0.5 with key coefficients 2c equals scale 1 with c; scale 0 is uniform."""
    dtype = F16
    D, Sk = 8, 6
    c = np.array([0.5, -1.0, 2.0, 0.25, -0.75, 1.5])
    V = I.random_bits((1, Sk, 1, D), ("normal", 0.0, 1.0), dtype, 7)
    Q1, K1 = _onehot_scores(Sk, D, c, dtype)
    Q2, K2 = _onehot_scores(Sk, D, 2 * c, dtype)
    r1, _ = oracle.attention(1, 1, Sk, 1, D, dtype, Q1, K1, V, scale=1.0)
    r2, _ = oracle.attention(1, 1, Sk, 1, D, dtype, Q2, K2, V, scale=0.5)
    assert np.array_equal(r1, r2)
    r0, _ = oracle.attention(1, 1, Sk, 1, D, dtype, Q1, K1, V, scale=0.0)
    assert np.allclose(r0[0], oracle.decode(dtype, V).reshape(Sk, D).mean(axis=0), rtol=1e-14, atol=1e-16)


def test_default_scale_is_one_over_sqrt_d():
    dtype = F16
    D, Sk = 64, 5
    Q, K = _onehot_scores(Sk, D, [1.0, 2.0, -1.0, 0.5, 3.0], dtype)
    V = I.random_bits((1, Sk, 1, D), ("normal", 0.0, 1.0), dtype, 8)
    a, _ = oracle.attention(1, 1, Sk, 1, D, dtype, Q, K, V)
    b, _ = oracle.attention(1, 1, Sk, 1, D, dtype, Q, K, V, scale=0.125)
    assert np.array_equal(a, b)


def test_common_shift_and_huge_scores():
    """Adding the same amount to every score changes nothing, even when the
    scores are far beyond exp's range (the maximum is subtracted first)."""
    dtype = F16
    D = 8
    c = np.array([1.0, -2.0, 0.0, 3.0])
    V = I.random_bits((1, 4, 1, D), ("normal", 0.0, 1.0), dtype, 9)
    Q1, K1 = _onehot_scores(4, D, c, dtype)
    Q2, K2 = _onehot_scores(4, D, c + 1024.0, dtype)       # integers near 1024: exact in fp16
    assert np.array_equal(oracle.decode(dtype, K2).reshape(4, D)[:, 0], c + 1024.0)
    r1, _ = oracle.attention(1, 1, 4, 1, D, dtype, Q1, K1, V, scale=1.0)
    r2, _ = oracle.attention(1, 1, 4, 1, D, dtype, Q2, K2, V, scale=1.0)
    assert np.isfinite(r2).all()
    assert np.allclose(r1, r2, rtol=1e-12, atol=1e-15)
    big = _onehot_scores(4, D, [1000.0, 1000.0, 1000.0, 1000.0], dtype)
    rb, _ = oracle.attention(1, 1, 4, 1, D, dtype, big[0], big[1], V, scale=1.0)
    assert np.allclose(rb[0], oracle.decode(dtype, V).reshape(4, D).mean(axis=0), rtol=1e-14, atol=1e-16)


def test_joint_key_permutation_changes_nothing():
    dtype = BF16
    B, Sq, Sk, H, D = 1, 5, 17, 2, 16
    Q = I.random_bits((B, Sq, H, D), ("normal", 0.0, 1.0), dtype, 10)
    K = I.random_bits((B, Sk, H, D), ("normal", 0.0, 1.0), dtype, 11).reshape(B, Sk, H, D)
    V = I.random_bits((B, Sk, H, D), ("normal", 0.0, 1.0), dtype, 12).reshape(B, Sk, H, D)
    perm = np.random.Generator(np.random.PCG64(13)).permutation(Sk)
    r1, _ = oracle.attention(B, Sq, Sk, H, D, dtype, Q, K, V)
    r2, _ = oracle.attention(B, Sq, Sk, H, D, dtype, Q, np.ascontiguousarray(K[:, perm]),
                             np.ascontiguousarray(V[:, perm]))
    assert np.allclose(r1, r2, rtol=1e-12, atol=1e-14)


def test_argument_checks():
    Q = np.zeros(16, np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(1, 2, 3, 1, 8, F16, Q, np.zeros(24, np.uint16), np.zeros(24, np.uint16), causal=True)
