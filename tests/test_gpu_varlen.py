"""Batches of trees of different sizes on the GPU (the _varlen entry points)
vs the oracle, which is pinned to treat each request as if it were alone
with its rows cut to its node count.  The padding past each request's nodes
is NaN in the queries and the tree K/V, and in the parents and tokens either
a valid, acceptable tree extension or entries that would make the tree
malformed -- none of it may change a result.  Covered: the matrix-core path
with the split planned on the device, the FMA path (fp32 and small bf16),
two-word trees (N = 128 with counts on both sides of 64), the tree stored in
the cache, the host split (more than 64 requests), the tree mask outputs,
greedy and stochastic verification, verification + commit in one pass, and
node counts outside [1, N]."""
import numpy as np
import pytest
import torch

import oracle
import token_tree_verification_attn_amd as ttv
from gpu_case import ATTN_TOL, announce, to_dev
from test_oracle_varlen import varlen_batch

pytestmark = pytest.mark.gpu


def dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def check_attn_varlen(d, in_cache=False):
    t = to_dev(d)
    n = dev_i32(d["n_nodes"])
    B, N, Hq, D = t["q"].shape
    if in_cache:  # node i's K/V at cache row L_b + i; rows past the request's nodes are NaN
        kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
        for b in range(B):
            L, nb = int(d["cache_len"][b]), int(d["n_nodes"][b])
            kc[b, :, L:L + N] = t["k_tree"][b]
            vc[b, :, L:L + N] = t["v_tree"][b]
            kc[b, :, L + max(nb, 0):] = float("nan")
            vc[b, :, L + max(nb, 0):] = float("nan")
        kt = vt = None
    else:
        kc, vc, kt, vt = t["k_cache"], t["v_cache"], t["k_tree"], t["v_tree"]
    W = (N + 63) // 64
    anc = torch.full((B, N, W), -7, dtype=torch.int64, device="cuda")
    depth = torch.full((B, N), -7, dtype=torch.int32, device="cuda")
    out, lse, st = ttv.tree_attn(t["q"], kc, vc, t["cache_len"], kt, vt, t["parents"],
                                 d["Lmax"], scale=d["scale"], n_nodes=n, anc_out=anc,
                                 depth_out=depth)
    torch.cuda.synchronize()
    ref, ref_lse, ref_st = oracle.tree_attn(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                            d["k_tree"], d["v_tree"], d["parents"], d["scale"],
                                            d["n_nodes"])
    atol, rtol = ATTN_TOL[d["dtype"]]
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, ref, atol=atol, rtol=rtol)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, atol=1e-3, rtol=1e-4)
    assert np.array_equal(st.cpu().numpy(), ref_st[:, 0, 0])
    r_dep, r_anc, _ = oracle.topology(d["parents"], d["n_nodes"])
    ok = ref_st[:, 0, 0] != ttv.E_SHAPE  # a rejected count: the mask outputs are empty too
    assert np.array_equal(depth.cpu().numpy()[ok], r_dep[ok])
    assert np.array_equal(anc.cpu().numpy().view(np.uint64)[ok], r_anc[ok])
    return st.cpu().numpy()


ATTN = {
    "mfma_balanced": dict(B=6, N=64, Hq=16, Hkv=4, D=128, L=(100, 2000), dtype="bf16"),
    "mfma_two_words": dict(B=5, N=128, Hq=8, Hkv=2, D=128, L=(10, 700), dtype="bf16",
                           n=[128, 65, 64, 1, 100], dmax=20),
    "mfma_d64_g8": dict(B=4, N=40, Hq=16, Hkv=2, D=64, L=(0, 300), dtype="bf16"),
    "fma_fp32": dict(B=5, N=24, Hq=4, Hkv=2, D=128, L=(3, 200), dtype="f32"),
    "fma_bf16_small_groups": dict(B=4, N=7, Hq=4, Hkv=2, D=128, L=(3, 400), dtype="bf16"),
    "host_split_70_requests": dict(B=70, N=16, Hq=8, Hkv=2, D=64, L=(0, 900), dtype="bf16"),
}


@pytest.mark.parametrize("case", sorted(ATTN))
def test_attention(case):
    announce("attn varlen %s" % case)
    kw = dict(ATTN[case])
    st = check_attn_varlen(varlen_batch(11, **kw))
    assert (st == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_tree_in_cache(dtype):
    announce("attn varlen tree in cache %s" % dtype)
    d = varlen_batch(12, B=5, N=48, Hq=8, Hkv=2, D=128, L=(20, 600), dtype=dtype)
    st = check_attn_varlen(d, in_cache=True)
    assert (st == 0).all()


@pytest.mark.parametrize("bad", [0, -3, 65])
def test_attention_rejected_counts(bad):
    announce("attn varlen node count %d" % bad)
    d = varlen_batch(13, B=4, N=64, Hq=8, Hkv=2, D=128, L=(50, 500), dtype="bf16",
                     n=[64, bad, 30, 1])
    st = check_attn_varlen(d)
    assert st.tolist() == [0, ttv.E_SHAPE, 0, 0]


def verify_both(d, mode):
    t = to_dev(d)
    n = dev_i32(d["n_nodes"])
    if mode == ttv.GREEDY:
        got = ttv.tree_verify(mode, t["parents"], t["tokens"], t["llm"], n_nodes=n)
        ref = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"], d["n_nodes"])
    else:
        got = ttv.tree_verify(mode, t["parents"], t["tokens"], t["llm"], t["ssm"], seed=d["seed"],
                              step=3, n_nodes=n)
        ref = oracle.verify_mss_seeded(d["parents"], d["tokens"], d["llm"], d["ssm"], d["seed"],
                                       3, d["n_nodes"])
    torch.cuda.synchronize()
    for name, g, r in zip(("path", "path_len", "out_tokens", "status"), got, ref):
        assert np.array_equal(g.cpu().numpy(), r), name
    return ref


@pytest.mark.parametrize("seed", range(3))
def test_greedy(seed):
    announce("verify varlen greedy seed %d" % seed)
    ref = verify_both(varlen_batch(20 + seed, B=9, N=70, V=300, dmax=12), ttv.GREEDY)
    assert ref[1].max() >= 2


@pytest.mark.parametrize("seed", range(3))
def test_stochastic(seed):
    announce("verify varlen stochastic seed %d" % seed)
    d = varlen_batch(30 + seed, mode="stochastic", B=9, N=70, V=40, dmax=12)
    ref = verify_both(d, ttv.STOCHASTIC)
    assert ref[1].max() >= 2


def test_stochastic_large_vocabulary():
    announce("verify varlen stochastic V=40000")
    d = varlen_batch(33, mode="stochastic", B=6, N=30, V=40000, dmax=12, n=[30, 1, 0, 17, 2, 29])
    ref = verify_both(d, ttv.STOCHASTIC)
    assert ref[3].tolist() == [0, 0, ttv.E_SHAPE, 0, 0, 0]


def test_verify_rejected_counts():
    announce("verify varlen bad counts")
    for mode, kw in ((ttv.GREEDY, {}), (ttv.STOCHASTIC, dict(mode="stochastic"))):
        d = varlen_batch(40, B=4, N=30, V=50, n=[30, 0, 31, 2], **kw)
        ref = verify_both(d, mode)
        assert ref[3].tolist() == [0, ttv.E_SHAPE, ttv.E_SHAPE, 0]


@pytest.mark.parametrize("mode", ["greedy", "stochastic"])
@pytest.mark.parametrize("shared_len", [False, True])
def test_verify_commit(mode, shared_len):
    """One pass of verification and commit for a batch of different tree
    sizes: path, tokens, committed rows, lengths and statuses as the oracle's
    verification followed by its commit."""
    announce("verify_commit varlen %s shared_len=%s" % (mode, shared_len))
    d = varlen_batch(50, mode=mode, B=7, N=40, V=64, Hq=8, Hkv=4, D=128, L=(0, 90),
                     dtype="bf16", n=[40, 1, 17, 33, 2, 40, 0])
    t = to_dev(d)
    n = dev_i32(d["n_nodes"])
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    # the tree K/V of padding nodes is NaN: bits of the rows compared exactly
    lens = t["cache_len"].clone()
    extra = dict(ssm=t["ssm"], seed=d["seed"], step=5) if mode == "stochastic" else {}
    m = ttv.STOCHASTIC if mode == "stochastic" else ttv.GREEDY
    path, plen, outt, clo, src, st = ttv.tree_verify_commit(
        m, t["parents"], t["tokens"], t["llm"], t["k_tree"], t["v_tree"], kc, vc, lens, d["Lmax"],
        cache_len_out=lens if shared_len else None, n_nodes=n, **extra)
    torch.cuda.synchronize()
    if m == ttv.GREEDY:
        r = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"], d["n_nodes"])
    else:
        r = oracle.verify_mss_seeded(d["parents"], d["tokens"], d["llm"], d["ssm"], d["seed"], 5,
                                     d["n_nodes"])
    for name, g, x in zip(("path", "path_len", "out_tokens"), (path, plen, outt), r):
        assert np.array_equal(g.cpu().numpy(), x), name
    bits = lambda x: x.view(torch.int16).cpu().numpy()
    rk, rv, rclo, rsrc, rst = oracle.kv_commit(bits(t["k_tree"]), bits(t["v_tree"]),
                                               bits(t["k_cache"]), bits(t["v_cache"]),
                                               d["cache_len"], r[0], r[1], d["Lmax"])
    assert np.array_equal(bits(kc), rk) and np.array_equal(bits(vc), rv)
    assert np.array_equal(clo.cpu().numpy(), rclo)
    assert np.array_equal(src.cpu().numpy(), rsrc)
    want = np.where(r[3] != 0, r[3], np.where(rst == 0, 0, ttv.E_SHAPE))
    assert np.array_equal(st.cpu().numpy(), want)
    assert st.cpu().numpy()[-1] == ttv.E_SHAPE and st.cpu().numpy()[0] == 0
