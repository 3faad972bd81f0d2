"""Pins of the oracle's logits -> probabilities step (temperature, optional
top-k), each against something other than the oracle itself:
  * scipy's softmax of logits / T;
  * with top-k: the kept set equals numpy's stable argsort of the negated
    logits (first k), and the kept probabilities are scipy's softmax of those
    logits alone;
  * closed forms: a constant row is uniform; two logits a, b give the ratio
    exp((a - b) / T); adding a constant to a row changes nothing."""
import numpy as np
import pytest
import scipy.special

import oracle


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


def test_closed_forms():
    p = oracle.probs_from_logits(np.full((1, 64), 3.0, np.float32), 0.7)
    np.testing.assert_allclose(p, 1.0 / 64, rtol=1e-7)
    p = oracle.probs_from_logits(np.array([[1.5, -0.5]], np.float32), 0.8)
    np.testing.assert_allclose(p[0, 0] / p[0, 1], np.exp(2.0 / 0.8), rtol=1e-6)
    z = np.random.default_rng(0).normal(0, 1, (2, 50)).astype(np.float32)
    np.testing.assert_allclose(oracle.probs_from_logits(z + 64.0, 1.3, 7),
                               oracle.probs_from_logits(z, 1.3, 7), rtol=1e-5, atol=1e-9)
