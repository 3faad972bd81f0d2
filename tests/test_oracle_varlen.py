"""Pins of the oracle's batches of trees of different sizes (n_nodes[b]
nodes in the first entries of each request's rows; the rest is padding):
every request's results equal the oracle's run on that request alone with
its rows cut to n_nodes[b] -- the pinned single-request definitions -- and
padding never matters.  The padding is made as tempting as possible: half
the requests carry padding nodes that form a valid extension of the tree
whose tokens the verifier would accept (greedy: the parent's argmax) and
whose K/V and queries are NaN; the other half carry parents that would make
the tree malformed.  [SI] §5 "Scheduling" (a continuous batch verifies
requests of different tree sizes together)."""
import numpy as np
import pytest

import oracle
import synth

INVALID_N = 2  # status of a request whose node count is outside [1, N]


def varlen_batch(seed, mode="greedy", B=6, N=24, V=40, Hq=4, Hkv=2, D=64, L=(3, 60),
                 dtype="f32", n=None, dmax=8):
    """A batch of B trees of N-entry rows with node counts n (random in
    [1, N] with the first request full and the last a lone root, unless
    given), padded as the module docstring says."""
    rng = np.random.default_rng(seed)
    s = synth.Spec("vl", B, N, Hq, Hkv, D, L, dtype, V, mode, "random", 900 + seed, dmax=dmax,
                   max_children=4, plant=0.8, prob_sigma=0.5)
    d = synth.make(s)
    if n is None:
        n = rng.integers(1, N + 1, size=B).astype(np.int32)
        n[0], n[-1] = N, 1
    n = np.asarray(n, np.int32)
    par = d["parents"].copy()
    tok = d["tokens"].copy()
    llm = d["llm"].copy()
    for b in range(B):
        for i in range(n[b], N):
            if b % 2 == 0:   # a valid, acceptable extension
                par[b, i] = rng.integers(0, i) if i > 0 else -1
                if mode == "greedy":
                    tok[b, i] = int(np.argmax(llm[b, par[b, i]]))
                else:
                    tok[b, i] = int(np.argmax(d["ssm"][b, i]))
            else:            # would make the tree malformed
                par[b, i] = i if i % 3 else -7
                tok[b, i] = V + 3 if i % 2 else -2
        for k in ("q",):
            d[k][b, n[b]:] = np.nan
        for k in ("k_tree", "v_tree"):
            d[k][b, :, n[b]:] = np.nan
    d.update(parents=par, tokens=tok, llm=llm, n_nodes=n)
    return d


def alone(d, b):
    """Request b alone, its rows cut to its node count."""
    n = int(d["n_nodes"][b])
    out = dict(d)
    for k in ("parents", "tokens", "u_accept"):
        if k in d:
            out[k] = d[k][b:b + 1, :n]
    for k in ("llm", "ssm", "q"):
        if k in d:
            out[k] = d[k][b:b + 1, :n]
    for k in ("k_tree", "v_tree"):
        out[k] = d[k][b:b + 1, :, :n]
    for k in ("k_cache", "v_cache", "cache_len", "u_bonus"):
        if k in d:
            out[k] = d[k][b:b + 1]
    return out, n


@pytest.mark.parametrize("seed", range(4))
def test_topology_per_request(seed):
    d = varlen_batch(seed)
    dep, anc, st = oracle.topology(d["parents"], d["n_nodes"])
    for b in range(d["B"]):
        a, n = alone(d, b)
        rd, ra, rs = oracle.topology(a["parents"])
        assert st[b] == rs[0]
        assert np.array_equal(dep[b, :n], rd[0]) and np.all(dep[b, n:] == -1)
        assert np.array_equal(anc[b, :n, :ra.shape[2]], ra[0]) and not anc[b, n:].any()


@pytest.mark.parametrize("seed", range(3))
def test_attention_per_request(seed):
    d = varlen_batch(seed)
    B, N, Hq = d["B"], d["N"], d["Hq"]
    out, lse, st = oracle.tree_attn(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                    d["k_tree"], d["v_tree"], d["parents"], d["scale"],
                                    d["n_nodes"])
    for b in range(B):
        a, n = alone(d, b)
        ro, rl, rs = oracle.tree_attn(a["q"], a["k_cache"], a["v_cache"], a["cache_len"],
                                      a["k_tree"], a["v_tree"], a["parents"], d["scale"])
        assert np.array_equal(out[b, :n], ro[0]) and np.array_equal(lse[b, :n], rl[0])
        assert np.all(out[b, n:] == 0) and np.all(lse[b, n:] == 0)
        assert np.all(st[b] == rs[0, 0])
    assert np.isfinite(out).all()


@pytest.mark.parametrize("seed", range(6))
def test_greedy_per_request(seed):
    d = varlen_batch(seed)
    path, plen, outt, st = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"], d["n_nodes"])
    for b in range(d["B"]):
        a, n = alone(d, b)
        rp, rl, ro, rs = oracle.verify_greedy(a["parents"], a["tokens"], a["llm"])
        assert plen[b] == rl[0] and st[b] == rs[0]
        assert np.array_equal(path[b, :n], rp[0]) and np.all(path[b, n:] == -1)
        assert np.array_equal(outt[b, :n], ro[0]) and np.all(outt[b, n:] == -1)
    assert plen.max() >= 2


@pytest.mark.parametrize("seed", range(6))
def test_stochastic_per_request(seed):
    d = varlen_batch(seed, mode="stochastic", V=12)
    res = oracle.verify_mss(d["parents"], d["tokens"], d["llm"], d["ssm"], d["u_accept"],
                            d["u_bonus"], d["n_nodes"])
    for b in range(d["B"]):
        a, n = alone(d, b)
        ref = oracle.verify_mss(a["parents"], a["tokens"], a["llm"], a["ssm"], a["u_accept"],
                                a["u_bonus"])
        for g, r in zip(res, ref):
            g = g[b] if g.ndim == 1 else g[b]
            r = r[0]
            if np.ndim(g) == 0:
                assert g == r
            else:
                assert np.array_equal(g[:n], r) and np.all(g[n:] == -1)
    assert res[1].max() >= 2


def test_seeded_stochastic_equals_its_uniforms():
    """The seeded walk on a batch of different sizes draws exactly the
    uniforms of its counters (j, u, b, step): the explicit-uniform walk given
    them (computed here by numpy's Philox) agrees on every request."""
    import test_oracle_philox as PH
    d = varlen_batch(7, mode="stochastic", V=12, B=8)
    n = d["n_nodes"]
    par = d["parents"].copy()
    for b in range(d["B"]):        # the counters of valid nodes only
        par[b, n[b]:] = 0
    ua = PH.numpy_uniforms(par, 31, 4)
    path, plen, _, st = oracle.verify_mss(d["parents"], d["tokens"], d["llm"], d["ssm"], ua,
                                          np.zeros(d["B"], np.float32), n)
    ub = np.zeros(d["B"], np.float32)
    for b in range(d["B"]):
        if st[b] == 0:
            end = int(path[b, plen[b] - 1])
            r24 = int(PH.np_block((PH.BONUS, end, b, 4), (31, 0))[0]) >> 40
            ub[b] = np.float32(r24) * np.float32(2.0 ** -24)
    ref = oracle.verify_mss(d["parents"], d["tokens"], d["llm"], d["ssm"], ua, ub, n)
    got = oracle.verify_mss_seeded(d["parents"], d["tokens"], d["llm"], d["ssm"], 31, 4, n)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("bad", [0, -1, 25])
def test_node_count_outside_the_rows_is_rejected(bad):
    d = varlen_batch(1)
    n = d["n_nodes"].copy()
    n[2] = bad
    dep, anc, st = oracle.topology(d["parents"], n)
    assert st[2] == INVALID_N and np.all(dep[2] == -1) and not anc[2].any()
    out, lse, st = oracle.tree_attn(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                    d["k_tree"], d["v_tree"], d["parents"], d["scale"], n)
    assert np.all(st[2] == INVALID_N) and np.all(out[2] == 0)
    path, plen, outt, st = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"], n)
    assert st[2] == INVALID_N and plen[2] == 0 and np.all(path[2] == -1)
    assert st[0] == 0
