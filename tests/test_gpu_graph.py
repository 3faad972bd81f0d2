"""The whole step captured in a HIP graph: every replay, with eager work and
synchronisations between replays, reproduces the eager result bit for bit --
with verification and commit as two calls, and as one pass
(tree_verify_commit), in both verification modes."""
import numpy as np
import pytest
import torch

import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import announce, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("one_pass", [False, True])
@pytest.mark.parametrize("name", ["c2", "c5"])
def test_graph_replays_match_eager(name, one_pass):
    announce("graph replay %s one_pass=%s" % (name, one_pass))
    d = synth.make(name)
    t = to_dev(d)
    mode = ttv.GREEDY if d["mode"] == "greedy" else ttv.STOCHASTIC
    B, N, Hq, D = t["q"].shape
    ws = torch.zeros(max(1, ttv.tree_attn_workspace_size(t["q"].dtype, B, N, Hq, d["Hkv"], D,
                                                         d["Lmax"])), dtype=torch.uint8,
                     device="cuda")
    wsv = torch.zeros(max(1, ttv.tree_verify_workspace_size(mode, B, N, d["V"])),
                      dtype=torch.uint8, device="cuda")
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    out = torch.empty_like(t["q"])
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device="cuda")
    path = torch.empty((B, N), dtype=torch.int32, device="cuda")
    plen = torch.empty(B, dtype=torch.int32, device="cuda")
    outt = torch.empty((B, N), dtype=torch.int32, device="cuda")
    clo = torch.empty(B, dtype=torch.int32, device="cuda")

    def step():
        ttv.tree_attn(t["q"], kc, vc, t["cache_len"], t["k_tree"], t["v_tree"], t["parents"],
                      d["Lmax"], scale=d["scale"], out=out, lse=lse, workspace=ws)
        if one_pass:
            ttv.tree_verify_commit(mode, t["parents"], t["tokens"], t["llm"], t["k_tree"],
                                   t["v_tree"], kc, vc, t["cache_len"], d["Lmax"],
                                   ssm=t.get("ssm"), seed=d.get("seed", 0),
                                   step=d.get("step", 0), cache_len_out=clo, path=path,
                                   path_len=plen, out_tokens=outt, workspace=wsv)
            return
        ttv.tree_verify(mode, t["parents"], t["tokens"], t["llm"], t.get("ssm"),
                        seed=d.get("seed", 0), step=d.get("step", 0), path=path, path_len=plen,
                        out_tokens=outt, workspace=wsv)
        ttv.kv_commit(t["k_tree"], t["v_tree"], kc, vc, t["cache_len"], path, plen, d["Lmax"],
                      cache_len_out=clo)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, path, plen, outt, clo, kc, vc)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for x in (out, lse, path, plen, outt, clo):   # eager work between replays
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, path, plen, outt, clo, kc, vc), ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep
