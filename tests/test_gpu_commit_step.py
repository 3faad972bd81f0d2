"""GPU kv_commit vs the oracle's byte copy, and the whole step (tree_attn ->
tree_verify -> kv_commit on one stream, no host synchronisation between the
calls) on every workload, each stage checked against the oracle."""
import numpy as np
import pytest
import torch

import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import (announce, check_attn, check_commit, check_verify, sample_rows, to_dev)

pytestmark = pytest.mark.gpu


def commit_case(**kw):
    base = dict(name="k", B=4, N=16, Hq=4, Hkv=2, D=128, L=(0, 90), dtype="bf16", V=32,
                mode="greedy", tree="random", seed=31)
    base.update(kw)
    return synth.make(synth.Spec(**base), with_verify=False)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("kw", [dict(), dict(dtype="f32", D=64), dict(N=128, tree="chain"),
                                dict(B=9, N=1), dict(Hkv=8, Hq=8, N=40, B=3), dict(Hkv=1, Hq=4)])
def test_commit_paths(kw, in_place):
    announce("commit %s in_place=%s" % (kw, in_place))
    d = commit_case(**kw)
    t = to_dev(d)
    rng = np.random.default_rng(5)
    B, N = d["B"], d["N"]
    # accepted paths: root then a random descending chain of the tree
    path = np.full((B, N), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        u, p = 0, [0]
        while True:
            kids = np.nonzero(d["parents"][b] == u)[0]
            if len(kids) == 0 or rng.random() < 0.3:
                break
            u = int(kids[rng.integers(len(kids))])
            p.append(u)
        path[b, :len(p)] = p
        plen[b] = len(p)
    check_commit(d, t, torch.from_numpy(path).cuda(), torch.from_numpy(plen).cuda(), in_place)


@pytest.mark.parametrize("in_place", [False, True])
def test_commit_rejects_bad_requests(in_place):
    announce("commit bad requests in_place=%s" % in_place)
    d = commit_case(B=4)
    t = to_dev(d)
    path = torch.zeros((4, 16), dtype=torch.int32, device="cuda") - 1
    path[:, 0] = 0
    path[2, 1] = 16                                    # node id out of range
    plen = torch.tensor([1, 17, 2, 0], dtype=torch.int32, device="cuda")  # 17 > N
    check_commit(d, t, path, plen, in_place)


def test_commit_in_place_lengths():
    announce("commit aliasing lengths")
    d = commit_case()
    t = to_dev(d)
    path = torch.zeros((4, 16), dtype=torch.int32, device="cuda") - 1
    path[:, 0] = 0
    plen = torch.ones(4, dtype=torch.int32, device="cuda")
    lens = t["cache_len"].clone()
    ttv.kv_commit(t["k_tree"], t["v_tree"], t["k_cache"], t["v_cache"], lens, path, plen,
                  d["Lmax"], cache_len_out=lens)
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), d["cache_len"] + 1)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_full_step(name):
    announce("full step %s" % name)
    d = synth.make(name)
    t = to_dev(d)
    rows = None if name in ("c1", "c2") else sample_rows(d, 256, seed=1)
    # the three calls are enqueued back to back; checks read results afterwards
    out, lse, st_a = ttv.tree_attn(t["q"], t["k_cache"], t["v_cache"], t["cache_len"],
                                   t["k_tree"], t["v_tree"], t["parents"], d["Lmax"],
                                   scale=d["scale"])
    mode = ttv.GREEDY if d["mode"] == "greedy" else ttv.STOCHASTIC
    path, plen, outt, st_v = ttv.tree_verify(mode, t["parents"], t["tokens"], t["llm"],
                                             t.get("ssm"), seed=d.get("seed", 0),
                                             step=d.get("step", 0))
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    clo, src, st_c = ttv.kv_commit(t["k_tree"], t["v_tree"], kc, vc, t["cache_len"], path,
                                   plen, d["Lmax"])
    torch.cuda.synchronize()
    assert torch.all(st_a == 0) and torch.all(st_v == 0) and torch.all(st_c == 0)
    # each stage against the oracle
    check_attn(d, t=t, rows=rows, repeat=False)
    check_verify(d, t=t)
    assert np.array_equal(clo.cpu().numpy(), d["cache_len"] + plen.cpu().numpy())
    assert torch.equal(src, path)
    for b in range(d["B"]):
        L, n = int(d["cache_len"][b]), int(plen[b])
        idx = path[b, :n].long()
        assert torch.equal(kc[b, :, L:L + n], t["k_tree"][b][:, idx])
        assert torch.equal(vc[b, :, L:L + n], t["v_tree"][b][:, idx])
        assert torch.equal(kc[b, :, :L], t["k_cache"][b, :, :L])
        assert torch.equal(kc[b, :, L + n:], t["k_cache"][b, :, L + n:])
