"""Pins of the oracle's merge step ([SI] §3 "Merge-based token tree
construction": the outputs of several speculative models combined into one
tree containing each of their token sequences), each against something other
than the oracle itself:
  * a hand-derived example;
  * brute force with Python sets: the nodes are exactly the distinct
    non-empty prefixes (one each), every node's root path spells its prefix,
    and the node's source sequence has that prefix;
  * the numbering: depth by depth, then by the lowest sequence index whose
    prefix the node is;
  * closed forms: identical sequences give one chain; sequences with distinct
    first tokens give disjoint chains of 1 + sum(len) nodes;
  * rejected requests get nothing."""
import numpy as np
import pytest

import oracle


def test_hand_example():
    seqs = np.array([[[5, 6, 7], [5, 6, 8], [5, 9, 0], [1, 1, 1]]], np.int32)
    ln = np.array([[3, 3, 2, 0]], np.int32)
    par, tok, src, n, st = oracle.tree_merge(seqs, ln, np.array([42], np.int32), 10)
    assert st.tolist() == [0] and n.tolist() == [6]
    assert par[0, :6].tolist() == [-1, 0, 1, 1, 2, 2]
    assert tok[0, :6].tolist() == [42, 5, 6, 9, 7, 8]
    assert src[0, :6].tolist() == [-1, 0, 1, 7, 2, 5]     # s*Ls + d of the leader
    assert (par[0, 6:] == -1).all()


def brute_check(seqs, ln, par, tok, src, n):
    S, Ls = seqs.shape
    prefixes = {tuple(seqs[s, :d]) for s in range(S) for d in range(1, ln[s] + 1)}
    assert n == 1 + len(prefixes)
    paths, depth = {}, [0] * n
    for i in range(1, n):
        assert 0 <= par[i] < i
        depth[i] = depth[par[i]] + 1
        p, path = i, []
        while p != 0:
            path.append(int(tok[p]))
            p = par[p]
        paths[i] = tuple(reversed(path))
    assert set(paths.values()) == prefixes and len(paths) == len(prefixes)
    leader = {}
    for i in range(1, n):
        s, d = divmod(int(src[i]), Ls)
        assert d == depth[i] - 1 and tuple(seqs[s, :d + 1]) == paths[i]
        assert s == min(t for t in range(S) if ln[t] > d and tuple(seqs[t, :d + 1]) == paths[i])
        leader[i] = s
    order = [(depth[i], leader[i]) for i in range(1, n)]
    assert order == sorted(order)


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_prefix_sets(seed):
    rng = np.random.default_rng(seed)
    B, S, Ls = 3, int(rng.integers(1, 12)), int(rng.integers(1, 9))
    seqs = rng.integers(0, 3, (B, S, Ls)).astype(np.int32)     # small vocabulary: many shared prefixes
    ln = rng.integers(0, Ls + 1, (B, S)).astype(np.int32)
    par, tok, src, n, st = oracle.tree_merge(seqs, ln, np.arange(B, dtype=np.int32), 128)
    assert (st == 0).all()
    for b in range(B):
        brute_check(seqs[b], ln[b], par[b], tok[b], src[b], int(n[b]))
        assert tok[b, 0] == b and src[b, 0] == -1


def test_closed_forms():
    seqs = np.tile(np.arange(7, dtype=np.int32), (1, 5, 1))    # five identical sequences
    par, tok, src, n, st = oracle.tree_merge(seqs, np.full((1, 5), 7, np.int32),
                                             np.zeros(1, np.int32), 16)
    assert n[0] == 8 and par[0, :8].tolist() == [-1] + list(range(7))
    assert (src[0, 1:8] == np.arange(7)).all()                 # all led by sequence 0
    seqs = np.arange(24, dtype=np.int32).reshape(1, 4, 6)       # distinct first tokens
    ln = np.array([[6, 2, 0, 5]], np.int32)
    par, tok, src, n, st = oracle.tree_merge(seqs, ln, np.zeros(1, np.int32), 32)
    assert n[0] == 1 + 13
    assert par[0, 1:4].tolist() == [0, 0, 0]                   # depth 1: sequences 0, 1, 3


def test_rejected_requests_get_nothing():
    seqs = np.zeros((3, 2, 4), np.int32)
    seqs[2] = np.arange(8).reshape(2, 4)
    ln = np.array([[4, 5], [-1, 0], [4, 4]], np.int32)          # 5 > Ls; -1 < 0; 9 nodes > 8
    par, tok, src, n, st = oracle.tree_merge(seqs, ln, np.zeros(3, np.int32), 8)
    assert st.tolist() == [2, 2, 2] and n.tolist() == [0, 0, 0]
    assert (par == -1).all() and (tok == -1).all() and (src == -1).all()
