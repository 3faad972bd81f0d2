"""Pins of the oracle's logits -> probabilities step (temperature, top-k,
top-p), each against something other than the oracle itself:
  * the exact 2^x it is built on against numpy's fp64 exp2 (relative error
    below 2e-7 wherever the result is a normal float) and at integers;
  * scipy's softmax of logits / T;
  * with top-k: the kept set equals numpy's stable argsort of the negated
    logits (first k), and the kept probabilities are scipy's softmax of those
    logits alone;
  * with top-p: the kept set is the shortest prefix of that stable order
    whose fp64 cumulative softmax probability (numpy) reaches top_p, after
    top-k when both are given;
  * closed forms: a constant row is uniform, and top_p = 1/2 on it keeps the
    lower half of the token ids; two logits a, b give the ratio
    exp((a - b) / T); adding a constant to a row changes nothing; a tiny
    top_p keeps only the argmax."""
import numpy as np
import pytest
import scipy.special

import oracle


def test_exp2_against_numpy():
    rng = np.random.default_rng(3)
    t = np.concatenate([-rng.random(20000) * 130.0, -rng.random(2000), [0.0, -0.5, -1.5]])
    t = t.astype(np.float32)
    got = oracle.exp2_taylor(t).astype(np.float64)
    ref = np.exp2(t.astype(np.float64))
    normal = ref >= 2.0 ** -125
    np.testing.assert_allclose(got[normal], ref[normal], rtol=2e-7)
    assert np.all(got[~normal] <= ref[~normal] * 1.0000002)
    ints = -np.arange(0, 126, dtype=np.float32)
    assert np.array_equal(oracle.exp2_taylor(ints), np.exp2(ints.astype(np.float64)).astype(np.float32))


@pytest.mark.parametrize("T", [0.8, 1.0, 2.5])
def test_matches_scipy_softmax(T):
    rng = np.random.default_rng(int(T * 10))
    z = rng.normal(0.0, 2.0, (5, 300)).astype(np.float32)
    p = oracle.probs_from_logits(z, T)
    ref = scipy.special.softmax(z.astype(np.float64) / T, axis=-1)
    np.testing.assert_allclose(p, ref, rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("k", [1, 5, 50])
def test_topk_keeps_the_stable_argsort_prefix(k):
    rng = np.random.default_rng(k)
    z = rng.choice(np.linspace(-2, 2, 9).astype(np.float32), size=(4, 200))   # many ties
    p = oracle.probs_from_logits(z, 1.0, k)
    for r in range(4):
        keep = np.argsort(-z[r], kind="stable")[:k]
        assert set(np.nonzero(p[r])[0].tolist()) == set(keep.tolist())
        np.testing.assert_allclose(p[r, keep], scipy.special.softmax(z[r, keep].astype(np.float64)),
                                   rtol=1e-6)


def topp_reference(z, T, k, top_p):
    """numpy: stable order, top-k, then the shortest prefix whose fp64
    cumulative softmax probability reaches top_p."""
    order = np.argsort(-z, kind="stable")
    if 0 < k < len(z):
        order = order[:k]
    w = scipy.special.softmax(z[order].astype(np.float64) / T)
    n = int(np.searchsorted(np.cumsum(w), top_p, side="left")) + 1
    return set(order[:min(n, len(order))].tolist())


@pytest.mark.parametrize("T,k,top_p", [(0.8, 0, 0.9), (1.0, 0, 0.5), (0.8, 50, 0.95),
                                       (2.0, 0, 0.99), (0.8, 0, 0.1), (1.0, 500, 0.7)])
def test_topp_keeps_the_shortest_prefix_reaching_p(T, k, top_p):
    rng = np.random.default_rng(int(T * 100) + k)
    z = rng.normal(0.0, 2.0, (6, 3000)).astype(np.float32)
    p = oracle.probs_from_logits(z, T, k, top_p)
    for r in range(6):
        kept = set(np.nonzero(p[r])[0].tolist())
        assert kept == topp_reference(z[r], T, k, top_p)
        idx = sorted(kept)
        np.testing.assert_allclose(p[r, idx], scipy.special.softmax(z[r, idx].astype(np.float64) / T),
                                   rtol=1e-6)


def test_closed_forms():
    p = oracle.probs_from_logits(np.full((1, 64), 3.0, np.float32), 0.7)
    np.testing.assert_allclose(p, 1.0 / 64, rtol=1e-7)
    p = oracle.probs_from_logits(np.full((1, 65), 3.0, np.float32), 0.7, 0, 0.5)
    assert np.nonzero(p[0])[0].tolist() == list(range(33))     # ties: lower ids first
    p = oracle.probs_from_logits(np.array([[1.5, -0.5]], np.float32), 0.8)
    np.testing.assert_allclose(p[0, 0] / p[0, 1], np.exp(2.0 / 0.8), rtol=1e-6)
    z = np.random.default_rng(0).normal(0, 1, (2, 50)).astype(np.float32)
    np.testing.assert_allclose(oracle.probs_from_logits(z + 64.0, 1.3, 7),
                               oracle.probs_from_logits(z, 1.3, 7), rtol=1e-5, atol=1e-9)
    p = oracle.probs_from_logits(z, 1.0, 0, 1e-6)
    assert np.array_equal(np.nonzero(p)[1], np.argmax(z, axis=1)) and np.all(p.max(1) == 1.0)
