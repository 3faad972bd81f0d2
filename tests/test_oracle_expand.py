"""Pins of the oracle's expansion step ([SI] §3 "Expansion-based token tree
construction": a speculative model's top-k tokens at a node become its
children), each against something other than the oracle itself:
  * a hand-derived example;
  * numpy's stable argsort of the negated row (its first k entries are the k
    most probable tokens, equal probabilities in increasing token order) on
    rows full of ties;
  * level-by-level expansion under a width schedule numbers the nodes as the
    independent breadth-first generator of the workload trees does;
  * structural invariants (parents before children, distinct sibling tokens,
    non-increasing probabilities, the frontier's -1 entries skipped);
  * the error cases leave a request untouched."""
import numpy as np
import pytest

import oracle
import synth


def empty_tree(B, Ncap, n_in=1):
    par = np.full((B, Ncap), -1, np.int32)
    tok = np.zeros((B, Ncap), np.int32)
    return par, tok, np.full(B, n_in, np.int32)


def test_hand_example():
    # row 0.1 0.3 0.3 0.2, k = 3: ids 1 and 2 tie at 0.3 (lower id first), then 3
    probs = np.array([[[0.1, 0.3, 0.3, 0.2]]], np.float32)
    par, tok, n_in = empty_tree(1, 8)
    par2, tok2, src, n_out, st = oracle.tree_expand(probs, np.array([[0]], np.int32), n_in, 3,
                                                    par, tok)
    assert st.tolist() == [0] and n_out.tolist() == [4]
    assert par2[0, :4].tolist() == [-1, 0, 0, 0]
    assert tok2[0, 1:4].tolist() == [1, 2, 3]
    assert src[0, 1:4].tolist() == [0, 0, 0]


@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_stable_argsort_with_ties(seed):
    rng = np.random.default_rng(seed)
    B, F, V = 3, 5, 37
    probs = rng.choice(np.array([0.0, 0.125, 0.25, 0.5, 1.0], np.float32), size=(B, F, V))
    k = int(rng.integers(1, 9))
    frontier = np.tile(np.arange(F, dtype=np.int32), (B, 1))
    par, tok, _ = empty_tree(B, 64)
    n_in = np.full(B, F, np.int32)
    par2, tok2, src, n_out, st = oracle.tree_expand(probs, frontier, n_in, k, par, tok)
    assert (st == 0).all() and (n_out == F + F * k).all()
    for b in range(B):
        for f in range(F):
            want = np.argsort(-probs[b, f], kind="stable")[:k]
            got = tok2[b, F + f * k: F + (f + 1) * k]
            assert got.tolist() == want.tolist()
            assert (par2[b, F + f * k: F + (f + 1) * k] == f).all()
            assert (src[b, F + f * k: F + (f + 1) * k] == f).all()


@pytest.mark.parametrize("widths", [(1, 1, 3, 1, 1, 1, 1, 1), (2, 3), (4, 1, 2)])
def test_levels_number_nodes_breadth_first(widths):
    """Expanding the nodes of each depth in index order with k = the schedule's
    width for that depth gives the breadth-first numbering of the workload
    generator (compared at level boundaries, where it does not truncate)."""
    rng = np.random.default_rng(7)
    V, Ncap = 50, 128
    par, tok, n_in = empty_tree(1, Ncap)
    depth = [0]
    level = [0]
    d = 0
    while True:
        k = widths[d % len(widths)]
        if n_in[0] + len(level) * k > Ncap:
            break
        probs = rng.random((1, len(level), V), dtype=np.float32)
        par, tok, src, n_out, st = oracle.tree_expand(
            probs, np.array([level], np.int32), n_in, k, par, tok)
        assert st[0] == 0
        new = list(range(n_in[0], n_out[0]))
        depth += [d + 1] * len(new)
        n_in = n_out
        level = new
        d += 1
        ref = synth.expansion_tree(int(n_in[0]), widths)
        assert par[0, :n_in[0]].tolist() == ref.tolist()
    assert n_in[0] > 10


def test_invariants_and_skipped_frontier_entries():
    rng = np.random.default_rng(3)
    B, F, V, k = 2, 6, 40, 3
    probs = rng.random((B, F, V), dtype=np.float32)
    frontier = np.array([[0, -1, 2, -1, 1, 3], [-1, -1, -1, 0, -1, -1]], np.int32)
    par = np.full((B, 40), -1, np.int32)
    par[0, :4] = [-1, 0, 0, 1]
    tok = np.zeros((B, 40), np.int32)
    n_in = np.array([4, 1], np.int32)
    par2, tok2, src, n_out, st = oracle.tree_expand(probs, frontier, n_in, k, par, tok)
    assert st.tolist() == [0, 0] and n_out.tolist() == [4 + 4 * k, 1 + k]
    assert par2[0, :4].tolist() == par[0, :4].tolist()      # existing nodes untouched
    for b in range(B):
        valid = [f for f in range(F) if frontier[b, f] >= 0]
        for r, f in enumerate(valid):
            sl = slice(n_in[b] + r * k, n_in[b] + (r + 1) * k)
            assert (par2[b, sl] == frontier[b, f]).all() and (src[b, sl] == f).all()
            t = tok2[b, sl]
            assert len(set(t.tolist())) == k
            p = probs[b, f, t]
            assert (np.diff(p) <= 0).all()
            rest = np.delete(probs[b, f], t)
            assert p.min() >= rest.max()
        for i in range(1, n_out[b]):
            assert 0 <= par2[b, i] < i


def test_errors_leave_the_request_untouched():
    probs = np.ones((3, 2, 10), np.float32)
    frontier = np.array([[0, 5], [0, -1], [0, 0]], np.int32)   # 5 >= n_in: not a node
    par, tok, _ = empty_tree(3, 4)
    n_in = np.array([2, 2, 0], np.int32)
    par2, tok2, src, n_out, st = oracle.tree_expand(probs, frontier, n_in, 3, par, tok)
    # request 0: bad frontier id; request 1: 2 + 3 > 4 nodes; request 2: no root
    assert st.tolist() == [7, 2, 7]
    assert n_out.tolist() == [2, 2, 0]
    assert (par2 == par).all() and (tok2 == tok).all() and (src == -1).all()
