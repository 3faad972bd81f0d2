"""Pins of the oracle's tree topology ([SI] §4 "Tree Attention": node i stands
for the sequence root -> i, so its mask row is the set of nodes on that path).

Independent routes used here:
* closed forms for chains and stars;
* the ancestor matrix as (I - P)^-1 for the parent matrix P (P is nilpotent,
  so the inverse is sum_k P^k, whose (i, j) entry counts the paths i -> j
  along parent edges: 1 for the ancestors-or-self of i, 0 otherwise), computed
  with numpy.linalg.inv;
* invariants (popcount = depth + 1, the parent's row is a subset).
"""
import numpy as np
import pytest

import oracle
import synth


def bits_to_matrix(anc, N):
    W = anc.shape[-1]
    M = np.zeros((N, N), np.int64)
    for i in range(N):
        for j in range(N):
            M[i, j] = (int(anc[i, j // 64]) >> (j % 64)) & 1
    assert W == (N + 63) // 64
    return M


def test_chain_closed_form():
    N = 70
    depth, anc, st = oracle.topology(synth.chain_tree(N)[None])
    assert st[0] == 0
    assert np.array_equal(depth[0], np.arange(N))
    M = bits_to_matrix(anc[0], N)
    assert np.array_equal(M, np.tril(np.ones((N, N), np.int64)))


def test_star_closed_form():
    N = 65
    depth, anc, st = oracle.topology(synth.star_tree(N)[None])
    assert st[0] == 0
    assert depth[0, 0] == 0 and np.all(depth[0, 1:] == 1)
    M = bits_to_matrix(anc[0], N)
    expect = np.eye(N, dtype=np.int64)
    expect[:, 0] = 1
    assert np.array_equal(M, expect)


@pytest.mark.parametrize("N,seed", [(1, 0), (2, 1), (8, 2), (33, 3), (64, 4), (65, 5),
                                    (128, 6)])
def test_matches_inverse_of_parent_matrix(N, seed):
    rng = np.random.default_rng(seed)
    trees = [synth.random_tree(rng, N, dmax=N, max_children=4) for _ in range(3)]
    par = np.stack(trees)
    depth, anc, st = oracle.topology(par)
    assert np.all(st == 0)
    for b in range(len(trees)):
        P = np.zeros((N, N))
        for i in range(1, N):
            P[i, par[b, i]] = 1.0
        closure = np.rint(np.linalg.inv(np.eye(N) - P)).astype(np.int64)
        M = bits_to_matrix(anc[b], N)
        assert np.array_equal(M, closure)
        assert np.array_equal(depth[b], closure.sum(axis=1) - 1)


def test_invariants_on_workload_trees():
    for name in ("c1", "c2", "c3", "c4", "c5"):
        d = synth.make(name, with_kv=False, with_verify=False)
        par = d["parents"]
        depth, anc, st = oracle.topology(par)
        assert np.all(st == 0)
        B, N = par.shape
        for b in range(B):
            for i in range(N):
                row = [int(w) for w in anc[b, i]]
                pop = sum(bin(w).count("1") for w in row)
                assert pop == depth[b, i] + 1
                assert (row[i // 64] >> (i % 64)) & 1
                if i:
                    prow = [int(w) for w in anc[b, par[b, i]]]
                    assert all((p & ~r) == 0 for p, r in zip(prow, row))


def test_workload_tree_shapes():
    """The generators produce the shapes the workloads describe."""
    c1 = synth.make("c1", with_kv=False, with_verify=False)
    assert oracle.topology(c1["parents"])[0].max() <= 4
    c2 = synth.make("c2", with_kv=False, with_verify=False)
    d2 = oracle.topology(c2["parents"])[0][0]
    assert list(np.bincount(d2)) == [1, 1, 1, 3, 3, 3, 3, 3, 3, 3, 3, 9, 9, 9, 9, 1]
    c3 = synth.make("c3", with_kv=False, with_verify=False)
    assert oracle.topology(c3["parents"])[0].max() <= 8
    for b in range(c3["B"]):
        assert np.bincount(c3["parents"][b, 1:], minlength=32).max() <= 4
    c4 = synth.make("c4", with_kv=False, with_verify=False)
    d4 = oracle.topology(c4["parents"])[0]
    assert d4.max() == 16 and c4["parents"].shape == (4, 128)


@pytest.mark.parametrize("bad", [
    [0, 0, 1],      # root has a parent
    [-1, 1, 0],     # self loop
    [-1, 0, 5],     # forward reference
    [-1, -1, 0],    # second root
    [-1, 0, 2],     # points at itself later
])
def test_malformed_trees_rejected(bad):
    par = np.array([bad, [-1, 0, 0]], np.int32)
    depth, anc, st = oracle.topology(par)
    assert st[0] == oracle.E_TREE and st[1] == 0
    assert np.all(depth[0] == -1) and np.all(anc[0] == 0)
