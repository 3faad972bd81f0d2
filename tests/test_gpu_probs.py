"""GPU logits -> probabilities (temperature, optional top-k) vs the fp64
oracle on the same seeded inputs.  Tolerance (derived): the exponent
(z - m) log2(e) / T is rounded once in fp32, so for |x| <= 150 (below that
fp32 underflows) the relative error of 2^x is below |x| 2^-23 ln 2 < 2e-5;
v_exp_f32 and the fp32 row sum add about 1e-6: rtol 3e-5.  The kept set of a
top-k row must match exactly (integer decision), including rows of many
equal logits (which take the whole-row selection path).  V = 37 takes the
scalar path, 32000 the register path, 40000 the streamed 16-byte path."""
import numpy as np
import pytest
import torch

import oracle
import token_tree_verification_attn_amd as ttv
from gpu_case import announce

pytestmark = pytest.mark.gpu


def check(z, T, k):
    got = ttv.probs_from_logits(torch.from_numpy(z).to("cuda"), T, k).cpu().numpy()
    ref = oracle.probs_from_logits(z, T, k)
    assert np.array_equal(got > 0, ref > 0)
    np.testing.assert_allclose(got, ref, rtol=3e-5, atol=1e-30)
    np.testing.assert_allclose(got.sum(-1), 1.0, rtol=1e-5)
    return got


@pytest.mark.parametrize("V", [37, 1000, 32000, 40000])
@pytest.mark.parametrize("T,k", [(0.8, 0), (1.0, 50), (0.8, 1), (1.0, 512)])
def test_gaussian_logits(V, T, k):
    announce("probs V=%d T=%g topk=%d" % (V, T, k))
    rng = np.random.default_rng(V + k)
    z = rng.normal(0.0, 2.0, (6, V)).astype(np.float32)
    check(z, T, min(k, V))


@pytest.mark.parametrize("V,k", [(37, 5), (32000, 50), (40000, 7)])
def test_many_equal_logits(V, k):
    announce("probs ties V=%d topk=%d" % (V, k))
    rng = np.random.default_rng(7 * V + k)
    z = rng.choice(np.linspace(-2, 2, 9).astype(np.float32), size=(4, V))
    check(z, 1.0, k)


def test_stochastic_workload_rows():
    """The stochastic workload's rows: softmax(N(0,2) / 0.8) over 32000 tokens
    for 64 nodes of 2 requests."""
    announce("probs 2 x 64 x 32000, T = 0.8")
    rng = np.random.default_rng(1005)
    z = rng.normal(0.0, 2.0, (2, 64, 32000)).astype(np.float32)
    check(z, 0.8, 0)


@pytest.mark.parametrize("k", [0, 50])
def test_benchmark_configuration(k):
    """The configuration bench_expand.py --op probs times: 1024 rows of 32000
    N(0,2) logits at T = 0.8 (its own input recipe), all tokens and top-50."""
    announce("probs benchmark configuration 1024 x 32000, T=0.8, topk=%d" % k)
    rng = np.random.default_rng(np.random.SeedSequence([1005, 13]))
    z = rng.normal(0.0, 2.0, (1024, 32000)).astype(np.float32)
    check(z, 0.8, k)
