"""Stochastic verification fed with logits (tree_verify_logits) vs the oracle,
bit for bit: the oracle turns both logits tensors into probabilities (the
same fixed arithmetic as the GPU) and runs its seeded multi-step speculative
sampling on them; the GPU never writes those probabilities but computes each
one it reads from the logits and its row's statistics.  Also equal to the
GPU's own two-step pipeline (probs_from_logits, then tree_verify)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import announce
from test_oracle_varlen import varlen_batch

pytestmark = pytest.mark.gpu


def logits_case(B, N, V, seed, sigma=2.0, tree="random"):
    s = synth.Spec("vl", B, N, 1, 1, 64, 0, "f32", V, "stochastic", tree, seed, dmax=8,
                   max_children=4, prob_sigma=0.7)
    d = synth.make(s, with_kv=False)
    rng = np.random.default_rng(seed)
    d["zl"] = rng.normal(0.0, sigma, (B, N, V)).astype(np.float32)
    d["zs"] = rng.normal(0.0, sigma, (B, N, V)).astype(np.float32)
    # plant the drafted token near the top of the LLM row so that some are accepted
    for b in range(B):
        for i in range(1, N):
            d["zl"][b, d["parents"][b, i], d["tokens"][b, i]] += 3.0
            d["zs"][b, i, d["tokens"][b, i]] += 3.0
    return d


def run(d, T, k, p, step=2, n_nodes=None):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    nn = None if n_nodes is None else dev(np.asarray(n_nodes, np.int32))
    got = ttv.tree_verify_logits(dev(d["parents"]), dev(d["tokens"]), dev(d["zl"]), dev(d["zs"]),
                                 T, k, p, seed=d["seed"], step=step, n_nodes=nn)
    torch.cuda.synchronize()
    ref = oracle.verify_mss_logits(d["parents"], d["tokens"], d["zl"], d["zs"], T, k, p,
                                   d["seed"], step, n_nodes)
    for name, g, r in zip(("path", "path_len", "out_tokens", "status"), got, ref):
        assert np.array_equal(g.cpu().numpy(), r), name
    # the two-step pipeline on the GPU gives the same
    pl = ttv.probs_from_logits(dev(d["zl"]), T, k, top_p=p)
    ps = ttv.probs_from_logits(dev(d["zs"]), T, k, top_p=p)
    if n_nodes is None:
        two = ttv.tree_verify(ttv.STOCHASTIC, dev(d["parents"]), dev(d["tokens"]), pl, ps,
                              seed=d["seed"], step=step)
    else:
        two = ttv.tree_verify(ttv.STOCHASTIC, dev(d["parents"]), dev(d["tokens"]), pl, ps,
                              seed=d["seed"], step=step, n_nodes=nn)
    for g, t in zip(got, two):
        assert torch.equal(g, t)
    return ref


@pytest.mark.parametrize("V", [64, 1000, 32000])
@pytest.mark.parametrize("T,k,p", [(0.8, 0, 1.0), (1.0, 50, 1.0), (0.8, 0, 0.9), (1.0, 20, 0.8)])
def test_against_oracle(V, T, k, p):
    announce("verify logits V=%d T=%g topk=%d top_p=%g" % (V, T, k, p))
    d = logits_case(6, 40, V, seed=V + k)
    run(d, T, min(k, V), p)


# Past 32768 entries the rows no longer fit the walk's registers and its
# residual goes to the workspace (B*V floats): the first size past that, a
# common vocabulary with top-k and with top-p, a large one, and a ragged batch.
@pytest.mark.parametrize("V,T,k,p", [(32772, 0.8, 0, 1.0), (50272, 1.0, 50, 1.0),
                                     (50272, 0.8, 0, 0.9), (131072, 0.8, 20, 0.95)])
def test_large_vocabulary(V, T, k, p):
    announce("verify logits large vocabulary V=%d T=%g topk=%d top_p=%g" % (V, T, k, p))
    d = logits_case(3, 24, V, seed=V + 7)
    run(d, T, k, p)


def test_large_vocabulary_node_counts():
    announce("verify logits V=40000 with node counts")
    d = logits_case(4, 20, 40000, seed=77)
    run(d, 0.8, 0, 1.0, n_nodes=[20, 1, 13, 2])


def test_stochastic_workload_shape():
    """16 requests x 64 nodes x 32000 tokens, T = 0.8 (the stochastic
    workload's shape, its LLM and speculator rows given as logits)."""
    announce("verify logits 16 x 64 x 32000")
    d = logits_case(16, 64, 32000, seed=1005)
    run(d, 0.8, 0, 1.0)
    run(d, 0.8, 50, 0.95, step=7)


def test_batch_of_different_tree_sizes():
    announce("verify logits with node counts")
    d = varlen_batch(61, mode="stochastic", B=7, N=30, V=48)
    rng = np.random.default_rng(0)
    d["zl"] = rng.normal(0.0, 1.0, d["llm"].shape).astype(np.float32)
    d["zs"] = rng.normal(0.0, 1.0, d["ssm"].shape).astype(np.float32)
    ref = run(d, 1.0, 0, 0.9, n_nodes=d["n_nodes"])
    assert (ref[3] == 0).all()
