"""Pins of the oracle's greedy verification.

[SI] §6 "Distributed LLM inference": tree verification generates exactly the
token sequences incremental decoding generates.  The pin simulates incremental
greedy decoding with the per-node logits as the model: start at the root, take
t = numpy.argmax (first index on ties) of the current node's logits, emit t,
move to the child whose token is t if there is one, else stop.  Plus closed
forms (all edges planted along a branch; no edge planted) and a hand-derived
example in tests/golden/.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def incremental_greedy(par, tok, llm):
    u, path, emitted = 0, [0], []
    while True:
        t = int(np.argmax(llm[u]))
        emitted.append(t)
        kids = [c for c in range(len(par)) if par[c] == u and tok[c] == t]
        if not kids:
            return path, emitted
        assert len(kids) == 1, "sibling tokens are distinct in these inputs"
        u = kids[0]
        path.append(u)


def check_against_incremental(d):
    path, plen, outt, st = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
    assert np.all(st == 0)
    for b in range(d["B"]):
        p, e = incremental_greedy(d["parents"][b], d["tokens"][b], d["llm"][b])
        assert plen[b] == len(p)
        assert list(path[b, : len(p)]) == p and np.all(path[b, len(p):] == -1)
        assert list(outt[b, : len(e)]) == e and np.all(outt[b, len(e):] == -1)
    return plen


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workloads_match_incremental_decoding(name):
    d = synth.make(name, with_kv=False)
    plen = check_against_incremental(d)
    if name != "c1":
        assert plen.max() >= 2  # planted edges give multi-token acceptance


@pytest.mark.parametrize("seed", range(6))
def test_random_small_trees(seed):
    s = synth.Spec("t", 5, 24, 1, 1, 8, 0, "f32", 6, "greedy", "random", 500 + seed,
                   dmax=6, max_children=4, logit_sigma=1.0, plant=0.5)
    check_against_incremental(synth.make(s, with_kv=False))


def test_hand_derived_example():
    g = json.load(open(os.path.join(GOLDEN, "greedy_hand_example.json")))
    par = np.array([g["parents"]], np.int32)
    tok = np.array([g["tokens"]], np.int32)
    llm = np.array([g["logits"]], np.float32)
    path, plen, outt, st = oracle.verify_greedy(par, tok, llm)
    assert st[0] == 0 and plen[0] == g["path_len"]
    assert list(path[0]) == g["path"] and list(outt[0]) == g["out_tokens"]


def test_fully_planted_branch_is_accepted():
    N, V = 10, 50
    par = synth.chain_tree(N)[None]
    tok = np.arange(N, dtype=np.int32)[None] + 7
    llm = np.zeros((1, N, V), np.float32)
    for u in range(N - 1):
        llm[0, u, tok[0, u + 1]] = 1.0
    llm[0, N - 1, 3] = 2.0
    path, plen, outt, _ = oracle.verify_greedy(par, tok, llm)
    assert plen[0] == N and list(path[0]) == list(range(N))
    assert list(outt[0]) == list(tok[0, 1:]) + [3]


def test_nothing_planted_accepts_only_the_root():
    s = synth.spec("c2", plant=0.0)
    d = synth.make(s, with_kv=False)
    path, plen, outt, _ = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
    # with V = 32000 an accidental match on the root's 1 child is unlikely
    # (and this seed has none): the step emits just the root's argmax
    assert plen[0] == 1 and path[0, 0] == 0 and np.all(path[0, 1:] == -1)
    assert outt[0, 0] == int(np.argmax(d["llm"][0, 0])) and np.all(outt[0, 1:] == -1)


def test_ties_go_to_lowest_index():
    par = np.array([[-1, 0, 0]], np.int32)
    tok = np.array([[0, 4, 2]], np.int32)
    llm = np.zeros((1, 3, 6), np.float32)
    llm[0, 0, [2, 4]] = 1.0      # tie between tokens 2 and 4 -> 2 (node 2)
    llm[0, 2, :] = -0.0          # all (signed) zeros -> token 0
    llm[0, 2, 0] = 0.0
    path, plen, outt, _ = oracle.verify_greedy(par, tok, llm)
    assert list(path[0]) == [0, 2, -1] and list(outt[0]) == [2, 0, -1]


def test_deepest_accepted_node_wins_over_lower_index():
    # two accepted branches when sibling tokens repeat: the deeper one ends the
    # path; at equal depth the lower index does
    par = np.array([[-1, 0, 0, 2, 1]], np.int32)
    tok = np.array([[0, 1, 1, 1, 2]], np.int32)
    llm = np.zeros((1, 5, 4), np.float32)
    llm[0, 0, 1] = 1.0   # root -> token 1: nodes 1 and 2 both accepted
    llm[0, 2, 1] = 1.0   # node 2 -> token 1: node 3 accepted (depth 2)
    llm[0, 1, 3] = 1.0   # node 1 -> token 3: node 4 (token 2) rejected
    path, plen, outt, _ = oracle.verify_greedy(par, tok, llm)
    assert list(path[0, :3]) == [0, 2, 3] and plen[0] == 3
    llm[0, 2, 1] = 0.0   # now nodes 1 and 2 are the deepest accepted: node 1
    path, plen, outt, _ = oracle.verify_greedy(par, tok, llm)
    assert list(path[0, :2]) == [0, 1] and plen[0] == 2


def test_malformed_tree():
    par = np.array([[-1, 0, 3, 1], [-1, 0, 0, 1]], np.int32)
    tok = np.zeros((2, 4), np.int32)
    llm = np.zeros((2, 4, 3), np.float32)
    path, plen, outt, st = oracle.verify_greedy(par, tok, llm)
    assert st[0] == oracle.E_TREE and plen[0] == 0
    assert np.all(path[0] == -1) and np.all(outt[0] == -1)
    assert st[1] == 0 and plen[1] >= 1
