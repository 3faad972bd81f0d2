"""The tree kept inside the KV cache: node i's K/V at cache row L_b + i.

Tree attention with NULL tree pointers vs the oracle on the same values in
the separate-tree form (the test places the tree rows in the cache and fills
every row past L_b + N with NaN, so a read beyond the tree shows); every
launch shape, the FMA path, the device-planned split and a rejected length.
The in-place commit (the accepted rows compacted to L_b, L_b+1, ..) vs its
oracle bit for bit, with separate and shared length arrays; and one whole
step in that layout (attention, greedy verification, in-place commit)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import ATTN_TOL, announce, to_dev

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="incache", B=2, N=16, Hq=8, Hkv=2, D=128, L=200, dtype="bf16", V=64,
                mode="greedy", tree="random", seed=777, dmax=8, max_children=4)
    base.update(kw)
    return synth.Spec(**base)


def in_cache(d):
    """Cache arrays with the tree rows at L_b + i and NaN after them."""
    kc, vc = d["k_cache"].copy(), d["v_cache"].copy()
    N = d["N"]
    for b, L in enumerate(d["cache_len"]):
        L = int(min(max(L, 0), d["Lmax"]))
        kc[b, :, L:L + N] = d["k_tree"][b]
        vc[b, :, L:L + N] = d["v_tree"][b]
        kc[b, :, L + N:] = np.nan
        vc[b, :, L + N:] = np.nan
    return kc, vc


def run_in_cache(d, **hints):
    t = to_dev(d)
    kc, vc = in_cache(d)
    dt = t["q"].dtype
    t["k_cache"] = torch.from_numpy(kc).to("cuda").to(dt)
    t["v_cache"] = torch.from_numpy(vc).to("cuda").to(dt)
    out, lse, st = ttv.tree_attn(t["q"], t["k_cache"], t["v_cache"], t["cache_len"], None, None,
                                 t["parents"], d["Lmax"], scale=d["scale"], **hints)
    torch.cuda.synchronize()
    return out, lse, st


CASES = {
    "rows64": (dict(B=2, N=64, Hq=4, Hkv=4, L=300), dict(rows_per_block=64)),
    "rows128": (dict(B=2, N=32, Hq=16, Hkv=4, L=333), dict(rows_per_block=128)),
    "rows256": (dict(B=1, N=128, Hq=16, Hkv=2, L=150, dmax=16), dict(rows_per_block=256)),
    "balanced_split": (dict(B=6, N=24, Hq=8, Hkv=2, L=(1, 900)), {}),
    "fixed_split": (dict(B=3, N=48, Hq=16, Hkv=4, L=(100, 900)), dict(chunk_keys=128)),
    "fma_bf16": (dict(B=3, N=3, Hq=8, Hkv=2, L=(5, 90)), {}),
    "fma_f32": (dict(B=2, N=20, Hq=4, Hkv=2, L=150, dtype="f32"), {}),
    "empty_prefix": (dict(B=2, N=40, Hq=8, Hkv=2, L=0), {}),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_tree_attn_in_cache(case):
    announce("attn tree in cache: %s" % case)
    kw, hints = CASES[case]
    d = synth.make(spec(**kw))
    out, lse, st = run_in_cache(d, **hints)
    assert int(st.abs().sum()) == 0
    rows = oracle.all_rows(d["B"], d["N"], d["Hq"])
    ref, ref_lse, _ = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                            d["k_tree"], d["v_tree"], d["parents"], d["scale"], rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    atol, rtol = ATTN_TOL[d["dtype"]]
    np.testing.assert_allclose(got, ref, atol=atol, rtol=rtol)


def test_tree_attn_in_cache_rejected_length():
    announce("attn tree in cache: length past the promise")
    d = synth.make(spec(B=3, N=16, L=(50, 300)))
    d["cache_len"] = d["cache_len"].copy()
    d["cache_len"][1] = d["Lmax"] + 5          # rejected: tree read at Lmax .. Lmax+N
    out, lse, st = run_in_cache(d)
    assert st.cpu().tolist() == [0, ttv.E_SHAPE, 0]
    assert torch.all(out[1] == 0)
    rows = np.array([r for r in oracle.all_rows(3, 16, 8) if r[0] != 1], np.int32)
    ref, _, _ = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                      d["k_tree"], d["v_tree"], d["parents"], d["scale"], rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    np.testing.assert_allclose(got, ref, atol=2e-2, rtol=1e-2)


def random_paths(rng, parents, n_max):
    B, N = parents.shape
    path = np.full((B, N), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        leaf = int(rng.integers(0, N))
        p = []
        while leaf != -1:
            p.append(leaf)
            leaf = int(parents[b, leaf])
        p = p[::-1][:n_max]
        path[b, :len(p)] = p
        plen[b] = len(p)
    return path, plen


@pytest.mark.parametrize("dtype,shared_len", [("bf16", False), ("bf16", True), ("f32", False)])
def test_kv_commit_inplace(dtype, shared_len):
    announce("kv_commit_inplace %s shared_len=%s" % (dtype, shared_len))
    rng = np.random.default_rng(5)
    d = synth.make(spec(B=5, N=40, Hkv=4, L=(10, 400), dtype=dtype, dmax=12))
    kc, vc = in_cache(d)
    kc = np.nan_to_num(kc, nan=3.0)            # NaN payloads would not compare equal
    vc = np.nan_to_num(vc, nan=-3.0)
    path, plen = random_paths(rng, d["parents"], 40)
    L = d["cache_len"].copy()
    L[3] = d["Lmax"] + 1                       # rejected
    path[4, 1] = 40                            # rejected: not a node
    plen[4] = max(plen[4], 2)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    t_kc = torch.from_numpy(kc).to("cuda").to(tdt)
    t_vc = torch.from_numpy(vc).to("cuda").to(tdt)
    host_k = t_kc.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    host_v = t_vc.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    t_len = torch.from_numpy(L).to("cuda")
    out_len = t_len if shared_len else torch.empty_like(t_len)
    clo, src, st = ttv.kv_commit_inplace(t_kc, t_vc, t_len, torch.from_numpy(path).to("cuda"),
                                         torch.from_numpy(plen).to("cuda"), d["Lmax"], 40,
                                         cache_len_out=out_len)
    torch.cuda.synchronize()
    rk, rv, rclo, rsrc, rst = oracle.kv_commit_inplace(host_k, host_v, L, path, plen, d["Lmax"], 40)
    gk = t_kc.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    gv = t_vc.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert np.array_equal(clo.cpu().numpy(), rclo) and np.array_equal(src.cpu().numpy(), rsrc)
    assert np.array_equal(st.cpu().numpy(), rst) and rst.tolist()[3:] == [2, 2]


def test_whole_step_in_cache():
    """Attention over the in-cache tree, greedy verification, in-place commit:
    the cache ends as prefix ++ accepted path, as the separate-tree oracle
    step gives."""
    announce("step with the tree in the cache")
    d = synth.make(spec(B=4, N=32, Hq=16, Hkv=4, L=(100, 700), V=512, dmax=10))
    kc, vc = in_cache(d)
    t = to_dev(d)
    t["k_cache"] = torch.from_numpy(kc).to("cuda").to(torch.bfloat16)
    t["v_cache"] = torch.from_numpy(vc).to("cuda").to(torch.bfloat16)
    out, lse, st_a = ttv.tree_attn(t["q"], t["k_cache"], t["v_cache"], t["cache_len"], None, None,
                                   t["parents"], d["Lmax"], scale=d["scale"])
    path, plen, outt, st_v = ttv.tree_verify(ttv.GREEDY, t["parents"], t["tokens"], t["llm"])
    clo, src, st_c = ttv.kv_commit_inplace(t["k_cache"], t["v_cache"], t["cache_len"], path, plen,
                                           d["Lmax"], d["N"])
    torch.cuda.synchronize()
    assert int(st_a.abs().sum() + st_v.abs().sum() + st_c.abs().sum()) == 0
    r_path, r_plen, _, _ = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
    assert np.array_equal(path.cpu().numpy(), r_path) and np.array_equal(plen.cpu().numpy(), r_plen)
    kt16 = torch.from_numpy(d["k_tree"]).to(torch.bfloat16).view(torch.int16).numpy()
    vt16 = torch.from_numpy(d["v_tree"]).to(torch.bfloat16).view(torch.int16).numpy()
    k0 = torch.from_numpy(kc).to(torch.bfloat16).view(torch.int16).numpy()
    v0 = torch.from_numpy(vc).to(torch.bfloat16).view(torch.int16).numpy()
    rk, rv, rclo, _, _ = oracle.kv_commit(kt16, vt16, k0, v0, d["cache_len"], r_path, r_plen, d["Lmax"])
    gk = t["k_cache"].cpu().view(torch.int16).numpy()
    gv = t["v_cache"].cpu().view(torch.int16).numpy()
    for b in range(d["B"]):
        end = int(rclo[b])
        assert np.array_equal(gk[b, :, :end], rk[b, :, :end])
        assert np.array_equal(gv[b, :, :end], rv[b, :, :end])
    assert np.array_equal(clo.cpu().numpy(), rclo)
