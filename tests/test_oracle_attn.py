"""Pins of the oracle's tree attention.

[SI] §4 "Tree Attention": a node's output is the output for the token sequence
that node represents; "Tree-Based Parallel Decoding": with causal masking,
shared-prefix tokens get identical outputs.  The pins:

* brute force (T1): for every node i, materialise X_i = prefix ++ tree rows on
  root -> i, run ordinary causal attention over X_i with the library routine
  torch.nn.functional.scaled_dot_product_attention (CPU, fp64) and take the
  row of node i;
* a chain tree is plain causal attention over prefix ++ tree for all rows at
  once (the tree-width-1 case of [SI] §6 "Token-tree analysis");
* closed forms: one key gives that key's value exactly; equal keys give the
  mean of the values;
* a topological relabelling of the nodes permutes the outputs;
* GQA: query head hq reads kv head hq // (Hq/Hkv).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth


def ancestors_by_inverse(par):
    """Nodes on root -> i, via (I - P)^-1 (independent of the oracle's walk)."""
    N = len(par)
    P = np.zeros((N, N))
    for i in range(1, N):
        P[i, par[i]] = 1.0
    M = np.rint(np.linalg.inv(np.eye(N) - P)).astype(np.int64)
    return [np.nonzero(M[i])[0] for i in range(N)]   # ascending = root first


def sdpa_last_row(qrow, K, V, scale):
    """Causal attention over a sequence whose last query is qrow; returns the
    output of the last position (it sees the whole sequence)."""
    T, D = K.shape
    Q = torch.zeros((1, 1, T, D), dtype=torch.float64)
    Q[0, 0, -1] = torch.from_numpy(qrow.astype(np.float64))
    k = torch.from_numpy(K.astype(np.float64))[None, None]
    v = torch.from_numpy(V.astype(np.float64))[None, None]
    o = F.scaled_dot_product_attention(Q, k, v, is_causal=True, scale=scale)
    return o[0, 0, -1].numpy()


def brute_force(d):
    B, N, Hq, Hkv, D = d["B"], d["N"], d["Hq"], d["Hkv"], d["D"]
    G = Hq // Hkv
    out = np.zeros((B, N, Hq, D))
    for b in range(B):
        paths = ancestors_by_inverse(d["parents"][b])
        L = d["cache_len"][b]
        for hq in range(Hq):
            h = hq // G
            for i in range(N):
                K = np.concatenate([d["k_cache"][b, h, :L], d["k_tree"][b, h, paths[i]]])
                V = np.concatenate([d["v_cache"][b, h, :L], d["v_tree"][b, h, paths[i]]])
                out[b, i, hq] = sdpa_last_row(d["q"][b, i, hq], K, V, d["scale"])
    return out


def small(**kw):
    base = dict(name="t", B=2, N=9, Hq=4, Hkv=2, D=8, L=(0, 5), dtype="f32", V=16,
                mode="greedy", tree="random", seed=77, dmax=4, max_children=3)
    base.update(kw)
    return synth.make(synth.Spec(**base), with_verify=False)


def run_oracle(d):
    return oracle.tree_attn(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                            d["k_tree"], d["v_tree"], d["parents"], d["scale"])


@pytest.mark.parametrize("kw", [
    {},
    dict(B=3, N=16, Hq=8, Hkv=2, D=16, L=(3, 20), seed=5),
    dict(B=1, N=12, Hq=3, Hkv=3, D=8, L=7, tree="star", seed=6),
    dict(B=2, N=7, Hq=2, Hkv=1, D=4, L=0, seed=8),
    dict(B=1, N=1, Hq=2, Hkv=1, D=8, L=6, seed=9),
    dict(B=2, N=10, Hq=4, Hkv=4, D=8, L=(1, 9), dtype="bf16", seed=10),
])
def test_brute_force_sdpa(kw):
    d = small(**kw)
    out, lse, st = run_oracle(d)
    assert np.all(st == 0)
    np.testing.assert_allclose(out, brute_force(d), rtol=0, atol=1e-12)


def test_chain_is_causal_attention():
    d = small(B=1, N=12, Hq=2, Hkv=1, D=8, L=9, tree="chain", seed=11)
    out, _, _ = run_oracle(d)
    L = 9
    for hq in range(2):
        K = np.concatenate([d["k_cache"][0, 0, :L], d["k_tree"][0, 0]])
        V = np.concatenate([d["v_cache"][0, 0, :L], d["v_tree"][0, 0]])
        Q = np.concatenate([np.zeros((L, 8)), d["q"][0, :, hq]])
        t = lambda a: torch.from_numpy(a.astype(np.float64))[None, None]
        o = F.scaled_dot_product_attention(t(Q), t(K), t(V), is_causal=True,
                                           scale=d["scale"])[0, 0, L:].numpy()
        np.testing.assert_allclose(out[0, :, hq], o, rtol=0, atol=1e-12)


def test_single_key_returns_value_exactly():
    d = small(B=1, N=1, Hq=1, Hkv=1, D=8, L=0, seed=12)
    out, lse, st = run_oracle(d)
    assert np.array_equal(out[0, 0, 0], d["v_tree"][0, 0, 0].astype(np.float64))
    s = d["scale"] * float(np.dot(d["q"][0, 0, 0].astype(np.float64),
                                  d["k_tree"][0, 0, 0].astype(np.float64)))
    assert abs(lse[0, 0, 0] - s) < 1e-12


def test_equal_keys_give_mean_of_values():
    d = small(B=1, N=6, Hq=1, Hkv=1, D=8, L=5, tree="chain", seed=13)
    d["k_cache"][:] = 0.5
    d["k_tree"][:] = 0.5
    out, lse, _ = run_oracle(d)
    for i in range(6):
        V = np.concatenate([d["v_cache"][0, 0, :5], d["v_tree"][0, 0, : i + 1]])
        np.testing.assert_allclose(out[0, i, 0], V.astype(np.float64).mean(0), atol=1e-12)
        s = d["scale"] * 0.5 * d["q"][0, i, 0].astype(np.float64).sum()
        assert abs(lse[0, i, 0] - (s + np.log(5 + i + 1))) < 1e-12


def test_topological_relabelling_permutes_outputs():
    d = small(B=1, N=12, Hq=2, Hkv=1, D=8, L=4, seed=14, dmax=6)
    out, _, _ = run_oracle(d)
    par = d["parents"][0]
    # a different topological order: repeatedly pick a random ready node
    rng = np.random.default_rng(3)
    order, ready, done = [0], [c for c in range(12) if par[c] == 0], {0}
    while ready:
        c = ready.pop(rng.integers(len(ready)))
        order.append(c)
        done.add(c)
        ready += [k for k in range(12) if par[k] == c]
    new_of = {old: new for new, old in enumerate(order)}
    par2 = np.array([-1] + [new_of[par[o]] for o in order[1:]], np.int32)
    e = dict(d)
    e["parents"] = par2[None]
    for key in ("q",):
        e[key] = d[key][:, order]
    for key in ("k_tree", "v_tree"):
        e[key] = d[key][:, :, order]
    out2, _, _ = run_oracle(e)
    np.testing.assert_allclose(out2[0], out[0][order], rtol=0, atol=1e-12)


def test_gqa_head_mapping():
    """Query heads of one group share their kv head: moving kv head h's data
    changes only query heads h*G .. h*G+G-1."""
    d = small(B=1, N=5, Hq=6, Hkv=3, D=8, L=4, seed=15)
    out, _, _ = run_oracle(d)
    e = dict(d)
    e["k_cache"] = d["k_cache"].copy()
    e["k_cache"][:, 1] = -e["k_cache"][:, 1]
    out2, _, _ = run_oracle(e)
    changed = np.abs(out2 - out).max(axis=(0, 1, 3)) > 1e-9
    assert list(changed) == [False, False, True, True, False, False]


def test_rows_beyond_prefix_are_not_read():
    d = small(B=2, N=6, L=(2, 4), seed=16)
    out, _, _ = run_oracle(d)
    e = dict(d)
    e["v_cache"] = d["v_cache"].copy()
    e["k_cache"] = d["k_cache"].copy()
    for b in range(2):
        e["v_cache"][b, :, d["cache_len"][b]:] = -7.0
        e["k_cache"][b, :, d["cache_len"][b]:] = 3.0
    out2, _, _ = run_oracle(e)
    assert np.array_equal(out, out2)


def test_malformed_tree_and_bad_length():
    d = small(B=3, N=5, seed=17)
    d["parents"] = d["parents"].copy()
    d["parents"][1, 3] = 4
    d["cache_len"] = d["cache_len"].copy()
    d["cache_len"][2] = d["k_cache"].shape[2] + 1
    out, lse, st = run_oracle(d)
    assert np.all(st[0] == 0)
    assert np.all(st[1] == oracle.E_TREE) and np.all(out[1] == 0) and np.all(lse[1] == 0)
    assert np.all(st[2] == oracle.E_SHAPE) and np.all(out[2] == 0)


def test_sampled_rows_equal_full_rows():
    d = small(B=2, N=9, seed=18)
    out, lse, _ = run_oracle(d)
    rows = np.array([[1, 8, 3], [0, 0, 0], [1, 4, 1]], np.int32)
    o, l, st = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                     d["k_tree"], d["v_tree"], d["parents"], d["scale"],
                                     rows)
    for r, (b, i, h) in enumerate(rows):
        assert np.array_equal(o[r], out[b, i, h]) and l[r] == lse[b, i, h]
