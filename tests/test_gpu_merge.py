"""GPU merge-based tree construction vs the oracle on the same seeded
inputs, bit for bit: parents, tokens, sources, node counts and statuses.
Sequences over a 3-token vocabulary share many prefixes; S = 1..64 with
ragged lengths (0 included); a raw bound above the capacity whose merged tree
still fits (the counting pass), one that does not, bad lengths, the 128-node
limit, and merged trees shaped like the long-context workload's (4 sequences
of 16 tokens, each repeating the first 0..3 tokens of the one before, from a
vocabulary of 32000)."""
import numpy as np
import pytest
import torch

import oracle
import token_tree_verification_attn_amd as ttv
from gpu_case import announce

pytestmark = pytest.mark.gpu


def check(seqs, ln, root, Ncap):
    t = [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in (seqs, ln, root)]
    par, tok, src, n, st = ttv.tree_merge(t[0], t[1], t[2], Ncap)
    torch.cuda.synchronize()
    got = [x.cpu().numpy() for x in (par, tok, src, n, st)]
    ref = oracle.tree_merge(seqs, ln, root, Ncap)
    for g, r, name in zip(got, ref, ("parents", "tokens", "src", "n_out", "status")):
        assert np.array_equal(g, r), name
    return got


@pytest.mark.parametrize("S,Ls", [(1, 1), (1, 16), (4, 8), (17, 5), (64, 3), (64, 16)])
def test_shared_prefixes(S, Ls):
    announce("merge S=%d Ls=%d" % (S, Ls))
    rng = np.random.default_rng(S * 131 + Ls)
    B = 5
    seqs = rng.integers(0, 3, (B, S, Ls)).astype(np.int32)
    ln = rng.integers(0, Ls + 1, (B, S)).astype(np.int32)
    ln[0] = Ls
    got = check(seqs, ln, rng.integers(0, 100, B).astype(np.int32), 128)
    assert (got[4] == 0).all() or (1 + ln.sum(1) > 128).any()


def test_counting_pass_and_overflow():
    announce("merge capacity: counting pass, overflow, bad lengths")
    rng = np.random.default_rng(11)
    S, Ls = 32, 8
    seqs = np.tile(rng.integers(0, 50, (1, 1, Ls)).astype(np.int32), (4, S, 1))
    seqs[1, :, 4:] = rng.integers(0, 50, (S, 4))      # request 1: 32 different tails
    ln = np.full((4, S), Ls, np.int32)
    ln[3, 5] = Ls + 1                                   # request 3: bad length
    ln[2, 0] = -1                                       # request 2: bad length
    got = check(seqs, ln, np.zeros(4, np.int32), 40)
    # request 0: 1 + 256 > 40 raw, but one chain of 8 fits; request 1: 1 + 4 + 128 > 40
    assert got[4].tolist() == [0, ttv.E_SHAPE, ttv.E_SHAPE, ttv.E_SHAPE]
    assert got[3].tolist() == [9, 0, 0, 0]


def test_node_limit():
    announce("merge 127 and 128 deep chains")
    seqs = np.tile(np.arange(128, dtype=np.int32), (2, 64, 1))
    ln = np.full((2, 64), 128, np.int32)
    ln[0] = 127                                          # 128 nodes: fits
    got = check(seqs, ln, np.array([7, 7], np.int32), 128)
    assert got[3].tolist() == [128, 0] and got[4].tolist() == [0, ttv.E_SHAPE]


def test_long_context_shaped_merges():
    announce("merge 4 x 16 speculator sequences, vocab 32000")
    rng = np.random.default_rng(1004)
    B, S, Ls = 4, 4, 16
    seqs = rng.integers(0, 32000, (B, S, Ls)).astype(np.int32)
    for b in range(B):
        for s in range(1, S):
            d = int(rng.integers(0, 4))
            seqs[b, s, :d] = seqs[b, s - 1, :d]
    got = check(seqs, np.full((B, S), Ls, np.int32), rng.integers(0, 32000, B).astype(np.int32),
                128)
    assert (got[4] == 0).all() and (got[3] <= 1 + S * Ls).all()
