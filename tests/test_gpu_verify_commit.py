"""Verification + KV commit in one pass (tree_verify_commit, greedy and
stochastic) vs the two calls it replaces (tree_verify, then kv_commit on its
path) and vs the oracle, bit for bit: path, path_len, out_tokens, cache rows,
lengths, sources and statuses.  Shapes cover both element types and head sizes, 128 nodes,
one node, one to 32 kv heads, ragged prefixes, the greedy workloads at full
size, malformed trees, rejected lengths, and a shared length array (one
workgroup per request instead of one per request and kv head)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import announce, to_dev

pytestmark = pytest.mark.gpu


def case(**kw):
    base = dict(name="vc", B=4, N=16, Hq=4, Hkv=2, D=128, L=(0, 90), dtype="bf16", V=64,
                mode="greedy", tree="random", seed=41)
    base.update(kw)
    return synth.make(synth.Spec(**base))


def bits(x):
    return x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def run_and_check(d, want_src=True, shared_len=False):
    t = to_dev(d)
    lens = t["cache_len"]
    greedy = d["mode"] == "greedy"
    mode = ttv.GREEDY if greedy else ttv.STOCHASTIC
    extra = {} if greedy else dict(ssm=t["ssm"], seed=d["seed"], step=d["step"])
    # the fused pass
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    lens1 = lens.clone()
    path, plen, outt, clo, src, st = ttv.tree_verify_commit(
        mode, t["parents"], t["tokens"], t["llm"], t["k_tree"], t["v_tree"], kc, vc, lens1,
        d["Lmax"], cache_len_out=lens1 if shared_len else None, want_src=want_src, **extra)
    # the two calls
    kc2, vc2 = t["k_cache"].clone(), t["v_cache"].clone()
    lens2 = lens.clone()
    path2, plen2, outt2, st_v = ttv.tree_verify(mode, t["parents"], t["tokens"], t["llm"],
                                                **extra)
    clo2, src2, st_c = ttv.kv_commit(t["k_tree"], t["v_tree"], kc2, vc2, lens2, path2, plen2,
                                     d["Lmax"], cache_len_out=lens2 if shared_len else None,
                                     want_src=want_src)
    torch.cuda.synchronize()
    st_seq = torch.where(st_v != 0, st_v, st_c)
    pairs = [("path", path, path2), ("path_len", plen, plen2), ("out_tokens", outt, outt2),
             ("cache_len_out", clo, clo2), ("status", st, st_seq)]
    if want_src:
        pairs.append(("committed_src", src, src2))
    else:
        assert src is None
    for name, a, b in pairs:
        assert torch.equal(a, b), name
    assert np.array_equal(bits(kc), bits(kc2)) and np.array_equal(bits(vc), bits(vc2))
    # and the oracle
    if greedy:
        r_path, r_plen, r_outt, r_st = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
    else:
        r_path, r_plen, r_outt, r_st = oracle.verify_mss_seeded(
            d["parents"], d["tokens"], d["llm"], d["ssm"], d["seed"], d["step"])
    assert np.array_equal(path.cpu().numpy(), r_path)
    assert np.array_equal(plen.cpu().numpy(), r_plen)
    assert np.array_equal(outt.cpu().numpy(), r_outt)
    rk, rv, rclo, rsrc, rst = oracle.kv_commit(bits(t["k_tree"]), bits(t["v_tree"]),
                                               bits(t["k_cache"]), bits(t["v_cache"]),
                                               d["cache_len"], r_path, r_plen, d["Lmax"])
    assert np.array_equal(bits(kc), rk) and np.array_equal(bits(vc), rv)
    assert np.array_equal(clo.cpu().numpy(), rclo)
    if want_src:
        assert np.array_equal(src.cpu().numpy(), rsrc)
    want = np.where(r_st != 0, r_st, np.where(rst == 0, 0, ttv.E_SHAPE))
    assert np.array_equal(st.cpu().numpy(), want)
    return st.cpu().numpy(), plen.cpu().numpy()


SHAPES = {
    "default": dict(),
    "f32_d64": dict(dtype="f32", D=64),
    "bf16_128x128_chain": dict(N=128, tree="chain", L=(0, 40)),
    "f32_128x128_star": dict(dtype="f32", N=128, tree="star", L=(3, 70), V=300),
    "one_node": dict(B=9, N=1),
    "one_head": dict(Hkv=1, Hq=4, N=33),
    "eight_heads": dict(Hkv=8, Hq=8, N=40, B=3, V=4100),
    "wide_vocab": dict(B=2, N=24, Hkv=4, Hq=8, V=32000, tree="expansion", L=300),
    # stochastic: the walk's own workgroup commits (every head of the request)
    "mss_default": dict(mode="stochastic", V=64),
    "mss_f32_d64_v50": dict(mode="stochastic", dtype="f32", D=64, V=50),
    "mss_32000_8heads": dict(mode="stochastic", B=3, N=40, Hkv=8, Hq=16, V=32000, L=(5, 300)),
    "mss_chain128": dict(mode="stochastic", N=128, tree="chain", V=40, L=(0, 40)),
    # empty prefixes (L = Lmax = 0): the path lands at cache rows 0..
    "empty_prefix": dict(L=0, N=20, Hkv=4, Hq=8),
    "mss_empty_prefix": dict(mode="stochastic", L=0, N=20, Hkv=4, Hq=8, V=64),
    # the residual in the workspace (V past 36864)
    "mss_large_vocab": dict(mode="stochastic", B=3, N=24, Hkv=2, Hq=8, V=50272, L=(0, 200)),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_fused_equals_two_calls(name):
    announce("verify_commit %s" % name)
    st, plen = run_and_check(case(**SHAPES[name]))
    assert (st == 0).all()


def test_without_sources():
    announce("verify_commit no committed_src")
    run_and_check(case(B=3), want_src=False)


def test_malformed_trees_and_rejected_lengths():
    """Request 1: a cycle (TTV_E_TREE, nothing committed); request 2: L past
    the promised Lmax; request 3: L < 0 (both TTV_E_SHAPE with the path still
    reported)."""
    announce("verify_commit malformed / rejected")
    d = case(B=5, N=20, Hkv=3, Hq=6)
    d["parents"] = d["parents"].copy()
    d["parents"][1, 7] = 9
    d["parents"][1, 9] = 7
    d["cache_len"] = d["cache_len"].copy()
    d["cache_len"][2] = d["Lmax"] + 1
    d["cache_len"][3] = -1
    st, plen = run_and_check(d)
    assert st.tolist() == [0, ttv.E_TREE, ttv.E_SHAPE, ttv.E_SHAPE, 0]
    assert plen[1] == 0 and plen[2] >= 1


def test_stochastic_bad_token_and_rejected_lengths():
    """Stochastic: request 1 has a token outside the vocabulary (the
    verifier's TTV_E_SHAPE, path_len 0, nothing committed), request 2 a cycle
    (TTV_E_TREE), request 3 a prefix length past Lmax (the commit's
    TTV_E_SHAPE with the path still reported)."""
    announce("verify_commit stochastic malformed / rejected")
    d = case(B=5, N=20, Hkv=3, Hq=6, mode="stochastic", V=64)
    d["tokens"] = d["tokens"].copy()
    d["tokens"][1, 4] = 64
    d["parents"] = d["parents"].copy()
    d["parents"][2, 7] = 9
    d["parents"][2, 9] = 7
    d["cache_len"] = d["cache_len"].copy()
    d["cache_len"][3] = d["Lmax"] + 1
    st, plen = run_and_check(d)
    assert st.tolist() == [0, ttv.E_SHAPE, ttv.E_TREE, ttv.E_SHAPE, 0]
    assert plen[1] == 0 and plen[2] == 0 and plen[3] >= 1


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workloads(name):
    """Every workload at full size (c2 is the benchmark's default, c5 the
    stochastic one)."""
    announce("verify_commit workload %s" % name)
    st, _ = run_and_check(synth.make(name))
    assert (st == 0).all()


@pytest.mark.parametrize("kw", [dict(), dict(Hkv=1, Hq=2), dict(B=3, N=128, Hkv=8, Hq=8,
                                                             tree="chain"),
                                dict(mode="stochastic", Hkv=4, Hq=4, N=30)])
def test_shared_length_array(kw):
    """cache_len_out = cache_len_in: the new lengths overwrite the old."""
    announce("verify_commit shared lengths %s" % kw)
    d = case(**kw)
    d["cache_len"] = d["cache_len"].copy()
    d["cache_len"][-1] = d["Lmax"] + 2                    # rejected: keeps its length
    st, plen = run_and_check(d, shared_len=True)
    assert (st[:-1] == 0).all() and st[-1] == ttv.E_SHAPE


@pytest.mark.parametrize("shared_len", [False, True])
def test_stochastic_whole_chain_accepted(shared_len):
    """A 128-node chain whose speculator rows equal the LLM rows of the parent
    (every test accepts): 128 rows of every kv head are committed."""
    announce("verify_commit stochastic chain accepted shared_len=%s" % shared_len)
    d = case(B=3, N=128, Hkv=4, Hq=8, tree="chain", mode="stochastic", V=40, L=(0, 60))
    d["ssm"] = d["ssm"].copy()
    d["ssm"][:, 1:] = d["llm"][:, :-1]
    st, plen = run_and_check(d, shared_len=shared_len)
    assert (st == 0).all() and (plen == 128).all()
