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


@pytest.mark.parametrize("name,bad", [("c3", False), ("c4", False), ("c2", True)])
def test_tree_attn_writes_the_mask(name, bad):
    """tree_attn's nullable anc_out / depth_out hold the mask and the depths,
    bit for bit; a malformed tree gets zero words and depth -1 there and
    TTV_E_TREE from the attention itself."""
    announce("tree_attn anc_out/depth_out %s malformed=%s" % (name, bad))
    s = synth.spec(name, B=2, L=300)
    d = synth.make(s, with_verify=False)
    if bad:
        d["parents"] = d["parents"].copy()
        d["parents"][1, 5] = 7
    B, N = d["parents"].shape
    dt = torch.bfloat16
    dev = "cuda"
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev).to(dt)
         for k in ("q", "k_cache", "v_cache", "k_tree", "v_tree")}
    par = torch.from_numpy(d["parents"]).to(dev)
    anc = torch.full((B, N, (N + 63) // 64), -7, dtype=torch.int64, device=dev)
    depth = torch.full((B, N), -7, dtype=torch.int32, device=dev)
    _, _, st = ttv.tree_attn(t["q"], t["k_cache"], t["v_cache"],
                             torch.from_numpy(d["cache_len"]).to(dev), t["k_tree"], t["v_tree"],
                             par, d["Lmax"], anc_out=anc, depth_out=depth)
    torch.cuda.synchronize()
    r_depth, r_anc, r_st = oracle.topology(d["parents"])
    assert np.array_equal(depth.cpu().numpy(), r_depth)
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), r_anc)
    assert np.array_equal(st.cpu().numpy(), r_st)
