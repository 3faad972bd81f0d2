"""GPU tree masks (ancestor bitsets) and depths vs the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import announce

pytestmark = pytest.mark.gpu


def run(par):
    announce("topology B=%d N=%d" % par.shape)
    anc, depth, st = ttv.tree_topology(torch.from_numpy(par).cuda())
    torch.cuda.synchronize()
    r_depth, r_anc, r_st = oracle.topology(par)
    assert np.array_equal(st.cpu().numpy(), r_st)
    assert np.array_equal(depth.cpu().numpy(), r_depth)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), r_anc)


@pytest.mark.parametrize("N", [1, 2, 8, 63, 64, 65, 100, 127, 128])
def test_random_trees(N):
    rng = np.random.default_rng(N)
    par = np.stack([synth.random_tree(rng, N, dmax=N, max_children=3) for _ in range(6)])
    run(par)


@pytest.mark.parametrize("N", [1, 64, 65, 128])
def test_chains_and_stars(N):
    run(np.stack([synth.chain_tree(N), synth.star_tree(N)]))


def test_workload_trees():
    for name in ("c1", "c2", "c3", "c4", "c5"):
        run(synth.make(name, with_kv=False, with_verify=False)["parents"])


def test_malformed_trees_flagged():
    par = np.stack([synth.chain_tree(70) for _ in range(4)])
    par[1, 0] = 0
    par[2, 66] = 66
    par[3, 65] = 69
    run(par)
