"""GPU logits -> probabilities (temperature, top-k, top-p) vs the oracle on
the same seeded inputs, bit for bit: both compute 2^x with the same
range reduction and Taylor polynomial in fp32 and the masses as exact
integers, so every probability and every kept set must be identical.  Rows
of many equal logits take the tie paths (top-k: the whole-row selection;
top-p: a crossing inside a run of equal logits, settled by token id); V = 37
takes the scalar path, 32000 the register path, 40000 the streamed 16-byte
path; flat rows (T = 5) make top-p refine its histogram several times."""
import numpy as np
import pytest
import torch

import oracle
import token_tree_verification_attn_amd as ttv
from gpu_case import announce

pytestmark = pytest.mark.gpu


def check(z, T, k, top_p=1.0):
    got = ttv.probs_from_logits(torch.from_numpy(z).to("cuda"), T, k, top_p=top_p).cpu().numpy()
    ref = oracle.probs_from_logits(z, T, k, top_p)
    bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
    assert len(bad) == 0, "%d differ, first %s: gpu %r ref %r" % (
        len(bad), bad[0], got[tuple(bad[0])], ref[tuple(bad[0])])
    np.testing.assert_allclose(got.sum(-1), 1.0, rtol=1e-5)
    return got


@pytest.mark.parametrize("V", [37, 1000, 32000, 40000])
@pytest.mark.parametrize("T,k,p", [(0.8, 0, 1.0), (1.0, 50, 1.0), (0.8, 1, 1.0), (1.0, 512, 1.0),
                                   (0.8, 0, 0.9), (1.0, 50, 0.95), (2.0, 0, 0.5),
                                   (0.8, 0, 0.999), (5.0, 0, 0.9)])
def test_gaussian_logits(V, T, k, p):
    announce("probs V=%d T=%g topk=%d top_p=%g" % (V, T, k, p))
    rng = np.random.default_rng(V + k + int(100 * p))
    z = rng.normal(0.0, 2.0, (6, V)).astype(np.float32)
    check(z, T, min(k, V), p)


@pytest.mark.parametrize("V,k,p", [(37, 5, 1.0), (32000, 50, 1.0), (40000, 7, 1.0),
                                   (37, 0, 0.5), (32000, 0, 0.3), (32000, 300, 0.6),
                                   (40000, 0, 0.77)])
def test_many_equal_logits(V, k, p):
    announce("probs ties V=%d topk=%d top_p=%g" % (V, k, p))
    rng = np.random.default_rng(7 * V + k)
    z = rng.choice(np.linspace(-2, 2, 9).astype(np.float32), size=(4, V))
    check(z, 1.0, k, p)


def test_constant_rows_and_extremes():
    announce("probs constant rows / tiny top_p")
    z = np.full((2, 1000), 0.25, np.float32)
    got = check(z, 0.7, 0, 0.5)
    assert np.nonzero(got[0])[0].tolist() == list(range(500))
    rng = np.random.default_rng(5)
    z = rng.normal(0.0, 3.0, (4, 4096)).astype(np.float32)
    got = check(z, 1.0, 0, 1e-7)                        # only the argmax survives
    assert np.array_equal(np.nonzero(got)[1], np.argmax(z, axis=1))
    z[:, ::2] = 0.0
    z[:, 1::4] = -0.0                                   # signed zeros are equal logits
    check(z, 1.3, 0, 0.4)


def test_stochastic_workload_rows():
    """The stochastic workload's rows: softmax(N(0,2) / 0.8) over 32000 tokens
    for 64 nodes of 2 requests."""
    announce("probs 2 x 64 x 32000, T = 0.8")
    rng = np.random.default_rng(1005)
    z = rng.normal(0.0, 2.0, (2, 64, 32000)).astype(np.float32)
    check(z, 0.8, 0)
    check(z, 0.8, 50, 0.9)


@pytest.mark.parametrize("k,p", [(0, 1.0), (50, 1.0), (0, 0.9)])
def test_benchmark_configuration(k, p):
    """The configuration bench_expand.py --op probs times: 1024 rows of 32000
    N(0,2) logits at T = 0.8 (its own input recipe)."""
    announce("probs benchmark configuration 1024 x 32000, T=0.8, topk=%d top_p=%g" % (k, p))
    rng = np.random.default_rng(np.random.SeedSequence([1005, 13]))
    z = rng.normal(0.0, 2.0, (1024, 32000)).astype(np.float32)
    check(z, 0.8, k, p)
