"""Pins of the oracle's counter-based random numbers and of how the seeded
stochastic verifier uses them.

The generator is Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11, "Parallel
random numbers: as easy as 1, 2, 3").  numpy ships the same generator as
``numpy.random.Philox``; numpy increments the 256-bit counter before it
computes a block, so the block of counter c is
``Philox(counter=c - 1, key=k).random_raw(4)`` (the decrement borrowing from
word 0 upward).  The oracle must match that library routine bit for bit.

The seeded verifier draws the uniform of the ratio test of the j-th child
(ascending node index) of node u in request b from counter (j, u, b, step)
and the final draw at u from counter (2^63, u, b, step), key (seed, 0), using
the 24 high bits of output word 0.  With those uniforms computed here by
numpy and handed to the explicit-uniform verifier, both must give identical
paths, lengths and tokens.
"""
import numpy as np
import pytest

import oracle
import synth

BONUS = 1 << 63


def np_block(counter_words, key_words):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter_words))
    k = int(key_words[0]) + (int(key_words[1]) << 64)
    bg = np.random.Philox(counter=(c - 1) % (1 << 256), key=k)
    return bg.random_raw(4)


def test_matches_numpy_philox():
    rng = np.random.default_rng(7)
    cases = [((0, 0, 0, 0), (0, 0)), ((0, 1, 0, 0), (1, 0)), ((0, 0, 0, 1), (2**64 - 1, 3)),
             ((2**64 - 1,) * 4, (2**64 - 1, 2**64 - 1)), ((BONUS, 5, 2, 0), (1005, 0))]
    for _ in range(200):
        cases.append((tuple(int(x) for x in rng.integers(0, 2**64, 4, dtype=np.uint64)),
                      tuple(int(x) for x in rng.integers(0, 2**64, 2, dtype=np.uint64))))
    for ctr, key in cases:
        got = oracle.philox4x64_10(np.array(ctr, np.uint64), np.array(key, np.uint64))
        assert np.array_equal(got, np_block(ctr, key)), (ctr, key)


def numpy_uniforms(parents, seed, step):
    """u_accept[b,c] of every non-root node from numpy's Philox under the
    counter layout above."""
    B, N = parents.shape
    ua = np.zeros((B, N), np.float32)
    for b in range(B):
        for c in range(1, N):
            u = int(parents[b, c])
            j = int(np.sum(parents[b, u + 1:c] == u))  # earlier siblings of c
            r24 = int(np_block((j, u, b, step), (seed, 0))[0]) >> 40
            ua[b, c] = np.float32(r24) * np.float32(2.0 ** -24)
    return ua


@pytest.mark.parametrize("seed,step,kw", [
    (1005, 0, dict()),
    (2**63 + 11, 2**40 + 3, dict(V=7)),
    (42, 1, dict(N=64, dmax=12, max_children=4, V=33, prob_sigma=4.0)),
    (9, 5, dict(N=30, tree="star", V=40)),
    (3, 2, dict(B=64, N=9, tree="star", V=8, prob_sigma=3.0)),  # many later attempts
])
def test_seeded_walk_uses_documented_counters(seed, step, kw):
    base = dict(name="s", B=16, N=24, Hq=1, Hkv=1, D=64, L=0, dtype="f32", V=50,
                mode="stochastic", tree="random", seed=321, dmax=6, max_children=4,
                temperature=0.8, prob_sigma=1.0)
    base.update(kw)
    d = synth.make(synth.Spec(**base), with_kv=False)
    par, tok, llm, ssm = d["parents"], d["tokens"], d["llm"], d["ssm"]
    B = par.shape[0]
    ua = numpy_uniforms(par, seed, step)
    # the path does not depend on the final uniform; its end names the bonus counter
    path, plen, _, _ = oracle.verify_mss(par, tok, llm, ssm, ua, np.zeros(B, np.float32))
    ub = np.zeros(B, np.float32)
    for b in range(B):
        end = int(path[b, plen[b] - 1])
        r24 = int(np_block((BONUS, end, b, step), (seed, 0))[0]) >> 40
        ub[b] = np.float32(r24) * np.float32(2.0 ** -24)
    ref = oracle.verify_mss(par, tok, llm, ssm, ua, ub)
    got = oracle.verify_mss_seeded(par, tok, llm, ssm, seed, step)
    for name, g, r in zip(("path", "path_len", "out_tokens", "status"), got, ref):
        assert np.array_equal(g, r), name
    assert plen.max() >= 2  # some child was accepted


def test_different_steps_draw_different_samples():
    """The step word of the counter changes the draws: over many steps the
    bonus token of a one-node tree takes many values."""
    V = 16
    par = np.full((4, 1), -1, np.int32)
    tok = np.zeros((4, 1), np.int32)
    llm = np.full((4, 1, V), 1.0 / V, np.float32)
    ssm = np.zeros_like(llm)
    seen = set()
    for step in range(40):
        _, _, outt, _ = oracle.verify_mss_seeded(par, tok, llm, ssm, 77, step)
        seen.update(outt[:, 0].tolist())
    assert len(seen) >= 12
