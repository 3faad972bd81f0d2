"""GPU tree expansion (one level of expansion-based token-tree construction)
vs the oracle on the same seeded inputs, bit for bit: parents, tokens,
source rows, node counts and statuses.  Rows full of equal probabilities
check the lower-token-id rule; V = 37 and 100 take the scalar and 16-byte
load paths; k = 1..16 covers every list size; frontier holes, untouched
entries, rejected requests, the largest sizes, and a level-by-level build of
the 64-node expansion schedule over 32000-token rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import announce

pytestmark = pytest.mark.gpu


def run_both(probs, frontier, n_in, k, parents, tokens, src_row):
    """The GPU call and the oracle on the same host arrays; returns both
    results as (parents, tokens, src_row, n_out, status) numpy arrays."""
    dev = "cuda"
    t = [torch.from_numpy(np.ascontiguousarray(a)).to(dev)
         for a in (probs, frontier, n_in, parents, tokens, src_row)]
    n_out, st = ttv.tree_expand(t[0], t[1], t[2], k, t[3], t[4], src_row=t[5])
    torch.cuda.synchronize()
    got = (t[3].cpu().numpy(), t[4].cpu().numpy(), t[5].cpu().numpy(), n_out.cpu().numpy(),
           st.cpu().numpy())
    ref = oracle.tree_expand(probs, frontier, n_in, k, parents, tokens, src_row)
    return got, ref


def check(probs, frontier, n_in, k, Ncap, fill=-7):
    B = probs.shape[0]
    parents = np.full((B, Ncap), fill, np.int32)
    tokens = np.full((B, Ncap), fill, np.int32)
    src = np.full((B, Ncap), fill, np.int32)
    parents[:, 0] = -1
    got, ref = run_both(probs, frontier, n_in, k, parents, tokens, src)
    for g, r, name in zip(got, ref, ("parents", "tokens", "src_row", "n_out", "status")):
        assert np.array_equal(g, r), name
    return got


def tie_rows(rng, B, F, V):
    return rng.choice(np.array([0.0, 0.125, 0.25, 0.5, 1.0], np.float32), size=(B, F, V))


@pytest.mark.parametrize("V", [37, 100, 32000])
@pytest.mark.parametrize("k", [1, 3, 4, 5, 8, 9, 16])
def test_ties_and_list_sizes(V, k):
    announce("expand V=%d k=%d" % (V, k))
    rng = np.random.default_rng(100 * k + V)
    B, F = 3, 5
    probs = tie_rows(rng, B, F, V)
    frontier = np.tile(np.arange(F, dtype=np.int32), (B, 1))
    check(probs, frontier, np.full(B, F, np.int32), k, 128)


def test_frontier_holes_and_untouched_entries():
    announce("expand frontier holes")
    rng = np.random.default_rng(5)
    B, F, V, k = 4, 9, 1000, 4
    probs = rng.random((B, F, V), dtype=np.float32)
    frontier = np.full((B, F), -1, np.int32)
    frontier[0, [0, 3, 8]] = [0, 2, 1]
    frontier[1, 4] = 0
    frontier[3, :] = np.arange(F) % 3
    got = check(probs, frontier, np.array([3, 1, 1, 3], np.int32), k, 64)
    assert got[4].tolist() == [0, 0, 0, 0]
    assert got[3].tolist() == [3 + 3 * k, 1 + k, 1, 3 + F * k]
    assert (got[0][2, 1:] == -7).all()      # request 2: empty frontier, nothing written


def test_rejected_requests():
    announce("expand rejected requests")
    rng = np.random.default_rng(6)
    B, F, V, k = 4, 3, 64, 2
    probs = rng.random((B, F, V), dtype=np.float32)
    frontier = np.array([[0, 1, 2], [0, 5, -1], [0, -2, -1], [0, 1, 2]], np.int32)
    n_in = np.array([3, 3, 3, 0], np.int32)
    got = check(probs, frontier, n_in, k, 8)   # request 0: 3 + 6 > 8 nodes
    assert got[4].tolist() == [ttv.E_SHAPE, ttv.E_TREE, ttv.E_TREE, ttv.E_TREE]
    assert got[3].tolist() == [3, 3, 3, 0]


def test_largest_sizes():
    announce("expand F=128 Ncap=128, B=64 V=32000")
    rng = np.random.default_rng(8)
    probs = rng.random((2, 127, 256), dtype=np.float32)
    frontier = np.tile(np.arange(127, dtype=np.int32) % 1, (2, 1))
    frontier[:, 1:] = -1
    frontier[1, :] = -1
    frontier[1, 126] = 0
    check(probs, frontier, np.ones(2, np.int32), 16, 128)
    probs = rng.random((2, 128, 64), dtype=np.float32)
    frontier = np.zeros((2, 128), np.int32)
    check(probs, frontier, np.ones(2, np.int32), 1, 128)        # 1 + 128 > 128: rejected
    probs = rng.random((64, 8, 32000), dtype=np.float32)
    check(probs, np.tile(np.arange(8, dtype=np.int32), (64, 1)), np.full(64, 8, np.int32), 4, 64)


def test_expansion_schedule_builds_the_workload_tree():
    """Level by level with the 64-node expansion schedule (widths cycling
    1,1,3,1,1,1,1,1), rows of 32000 speculator probabilities: the GPU tree
    equals the oracle's at every level, and its shape is the breadth-first
    tree of the workload generator."""
    announce("expand level by level, widths 1,1,3,1,1,1,1,1, V=32000")
    widths = (1, 1, 3, 1, 1, 1, 1, 1)
    rng = np.random.default_rng(9)
    B, V, Ncap = 4, 32000, 128
    par = np.full((B, Ncap), -1, np.int32)
    tok = np.zeros((B, Ncap), np.int32)
    src = np.full((B, Ncap), -1, np.int32)
    tok[:, 0] = rng.integers(0, V, B)
    n_in = np.ones(B, np.int32)
    level = [[0]] * B
    d = 0
    while True:
        k = widths[d % len(widths)]
        F = len(level[0])
        if n_in[0] + F * k > 64:
            break
        z = rng.normal(0.0, 2.0, (B, F, V))
        e = np.exp((z - z.max(-1, keepdims=True)) / 0.8)
        probs = (e / e.sum(-1, keepdims=True)).astype(np.float32)
        frontier = np.array(level, np.int32)
        got, ref = run_both(probs, frontier, n_in, k, par, tok, src)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)
        par, tok, src, n_out, st = got
        assert (st == 0).all()
        level = [list(range(n_in[b], n_out[b])) for b in range(B)]
        n_in = n_out
        d += 1
    ref_tree = synth.expansion_tree(int(n_in[0]), widths)
    for b in range(B):
        assert par[b, :n_in[b]].tolist() == ref_tree.tolist()


def test_benchmark_configuration():
    """The configuration bench_expand.py times: 16 requests x 16 frontier rows
    of 32000 probabilities (its own input recipe), k = 4."""
    announce("expand benchmark configuration 16 x 16 x 32000, k=4")
    import bench_expand
    probs = bench_expand.make_probs(16, 16, 32000)
    frontier = np.tile(np.arange(16, dtype=np.int32), (16, 1))
    check(probs, frontier, np.full(16, 16, np.int32), 4, 128)
