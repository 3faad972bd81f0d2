"""Pins of the oracle's multi-step speculative sampling (stochastic verify).

[SI] §4 "Token Verification": multi-step speculative sampling verifies a
stochastic token tree across branches and provably keeps the LLM's output
distribution (the same as incremental sampling).  The pages give the
guarantee, not the steps, so the pins check the guarantee and the textbook
pieces it is made of:

* acceptance of one drafted token x ~ q has probability min(1, p(x)/q(x))
  (the standard speculative-sampling rule; tree width 1 is sequence-based
  speculation, [SI] §6 "Token-tree analysis"): checked by sweeping the
  caller's uniform over a fine grid;
* after a rejection the next draw comes from norm(max(0, p - q)): checked by
  sweeping the final uniform over a grid;
* closed forms: p == q always accepts; P(accept) = sum_x min(p(x), q(x)) for
  x ~ q (Monte Carlo); p = 0.5 q empties the residual and falls back to p;
* the whole procedure keeps the distribution: the first three tokens of
  repeated verify steps over depth-2 trees drafted from q follow the
  incremental distribution p(t1) p(t2|t1) p(t3|t1,t2) (chi-square, scipy).
"""
import numpy as np
import pytest
from scipy import stats

import oracle

ONE_MINUS = np.float32(1.0) - np.float32(2.0 ** -24)


def grid(K):
    return ((np.arange(K) + 0.5) / K).astype(np.float32)


def norm32(x):
    x = np.asarray(x, np.float64)
    return (x / x.sum(-1, keepdims=True)).astype(np.float32)


def one_child_batch(p_root, q_child, x, r, ub, p_child=None):
    """B requests of the 2-node tree root -> child (token x)."""
    B = len(r)
    V = len(p_root)
    par = np.tile(np.array([-1, 0], np.int32), (B, 1))
    tok = np.tile(np.array([0, x], np.int32), (B, 1))
    llm = np.zeros((B, 2, V), np.float32)
    ssm = np.zeros((B, 2, V), np.float32)
    llm[:, 0] = p_root
    llm[:, 1] = p_root if p_child is None else p_child
    ssm[:, 1] = q_child
    ua = np.zeros((B, 2), np.float32)
    ua[:, 1] = r
    return oracle.verify_mss(par, tok, llm, ssm, ua, np.asarray(ub, np.float32))


def test_p_equals_q_always_accepts():
    rng = np.random.default_rng(1)
    B, N, V = 64, 9, 11
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))    # chains
    llm = norm32(rng.random((B, N, V)) + 0.05)
    ssm = np.zeros_like(llm)
    ssm[:, 1:] = llm[:, :-1]                                         # q_c = p_parent
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    ua = rng.random((B, N), dtype=np.float32)
    ua[0, :] = ONE_MINUS                                             # largest uniform
    ub = rng.random(B, dtype=np.float32)
    path, plen, outt, st = oracle.verify_mss(par, tok, llm, ssm, ua, ub)
    assert np.all(st == 0) and np.all(plen == N)
    assert np.array_equal(path, np.tile(np.arange(N), (B, 1)))
    assert np.array_equal(outt[:, : N - 1], tok[:, 1:])


@pytest.mark.parametrize("seed", range(4))
def test_accept_probability_is_min_ratio(seed):
    rng = np.random.default_rng(10 + seed)
    V, K = 7, 4096
    p = norm32(rng.random(V) + 0.02)
    q = norm32(rng.random(V) + 0.02)
    for x in range(V):
        _, plen, _, _ = one_child_batch(p, q, x, grid(K), np.zeros(K))
        frac = np.mean(plen == 2)
        assert abs(frac - min(1.0, p[x] / q[x])) <= 1.0 / K + 1e-6


@pytest.mark.parametrize("seed", range(3))
def test_sample_after_rejection_is_normalised_residual(seed):
    rng = np.random.default_rng(20 + seed)
    V, K = 9, 1 << 14
    p = norm32(rng.random(V) + 0.01)
    q = norm32(rng.random(V) + 0.01)
    x = int(np.argmax(q / p))                 # p(x) < q(x): rejectable
    assert p[x] < 0.99 * q[x]
    r = np.full(K, ONE_MINUS, np.float32)     # rejects
    _, plen, outt, _ = one_child_batch(p, q, x, r, grid(K))
    assert np.all(plen == 1)
    hist = np.bincount(outt[:, 0], minlength=V) / K
    res = np.maximum(p.astype(np.float64) - q, 0.0)
    np.testing.assert_allclose(hist, res / res.sum(), atol=2.0 / K + 1e-6)


def test_second_child_tested_against_residual():
    rng = np.random.default_rng(30)
    V, K = 6, 4096
    p = norm32(rng.random(V) + 0.05)
    q1 = norm32(rng.random(V) + 0.05)
    q2 = norm32(rng.random(V) + 0.05)
    x1 = int(np.argmax(q1 / p))
    res = np.maximum(p.astype(np.float64) - q1, 0.0)
    res /= res.sum()
    for x2 in range(V):
        B = K
        par = np.tile(np.array([-1, 0, 0], np.int32), (B, 1))
        tok = np.tile(np.array([0, x1, x2], np.int32), (B, 1))
        llm = np.zeros((B, 3, V), np.float32)
        ssm = np.zeros((B, 3, V), np.float32)
        llm[:] = p
        ssm[:, 1] = q1
        ssm[:, 2] = q2
        ua = np.zeros((B, 3), np.float32)
        ua[:, 1] = ONE_MINUS
        ua[:, 2] = grid(K)
        path, plen, _, _ = oracle.verify_mss(par, tok, llm, ssm, ua, np.zeros(B, np.float32))
        frac = np.mean((plen == 2) & (path[:, 1] == 2))
        assert abs(frac - min(1.0, res[x2] / q2[x2])) <= 1.0 / K + 1e-5


def test_leaf_bonus_comes_from_its_own_row():
    rng = np.random.default_rng(40)
    V, K = 10, 1 << 14
    p = norm32(rng.random(V))
    B = K
    par = np.full((B, 1), -1, np.int32)
    _, plen, outt, _ = oracle.verify_mss(par, np.zeros((B, 1), np.int32),
                                         np.tile(p, (B, 1, 1)), np.zeros((B, 1, V), np.float32),
                                         np.zeros((B, 1), np.float32), grid(K))
    assert np.all(plen == 1)
    np.testing.assert_allclose(np.bincount(outt[:, 0], minlength=V) / K, p,
                               atol=2.0 / K + 1e-6)


def test_inverse_cdf_end_points():
    p = np.array([0, 0, 0.25, 0, 0.5, 0.25, 0], np.float32)
    _, _, outt, _ = one_child_batch(p, p, 0, np.full(2, ONE_MINUS, np.float32),
                                    np.array([0.0, ONE_MINUS], np.float32),
                                    p_child=p)
    # token 0 has q = p = 0 there: r*q*s = 0 < w[0] = 0 is false -> rejected,
    # residual max(p - p, 0) = 0 is empty -> sample from p itself
    assert list(outt[:, 0]) == [2, 5]


def test_half_q_empties_residual_and_falls_back_to_p():
    rng = np.random.default_rng(50)
    V, K = 8, 1 << 13
    q = norm32(rng.random(V) + 0.05)
    p = (np.float32(0.5) * q).astype(np.float32)       # unnormalised on purpose
    x = 3
    # acceptance iff r*q[x] < 0.5*q[x]  <=> r < 0.5
    _, plen, _, _ = one_child_batch(p, q, x, grid(K), np.zeros(K))
    assert np.array_equal(plen == 2, grid(K) < 0.5)
    # on rejection the residual max(0.5q - q, 0) is empty: draw from p ~ q
    _, plen, outt, _ = one_child_batch(p, q, x, np.full(K, 0.75, np.float32), grid(K))
    assert np.all(plen == 1)
    np.testing.assert_allclose(np.bincount(outt[:, 0], minlength=V) / K, norm32(p),
                               atol=2.0 / K + 1e-6)


def test_chain_acceptance_rate_is_sum_of_min():
    rng = np.random.default_rng(60)
    V, B = 8, 200_000
    p = norm32(rng.random(V) + 0.1)
    q = norm32(rng.random(V) + 0.1)
    x = rng.choice(V, size=B, p=q.astype(np.float64) / q.sum()).astype(np.int32)
    par = np.tile(np.array([-1, 0], np.int32), (B, 1))
    tok = np.stack([np.zeros(B, np.int32), x], 1)
    llm = np.tile(p, (B, 2, 1))
    ssm = np.tile(q, (B, 2, 1))
    ua = rng.random((B, 2), dtype=np.float32)
    _, plen, _, _ = oracle.verify_mss(par, tok, llm, ssm, ua, rng.random(B, dtype=np.float32))
    a = np.minimum(p.astype(np.float64), q).sum()
    assert abs(np.mean(plen == 2) - a) < 5 * np.sqrt(a * (1 - a) / B)


class TinyModel:
    """Seeded next-token tables p(.|seq) and q(.|seq) over V tokens for all
    sequences up to length 4; sequence code = sum (t_i + 1) * (V+1)^i."""

    def __init__(self, V, seed):
        rng = np.random.default_rng(seed)
        n = (V + 1) ** 4
        self.V = V
        self.P = norm32(rng.dirichlet(np.full(V, 3.0), size=n))
        self.Q = norm32(rng.dirichlet(np.full(V, 3.0), size=n))

    def child(self, code, length, tok):
        return code + (tok + 1) * (self.V + 1) ** length


def draw(rng, rows):
    c = np.cumsum(rows.astype(np.float64), axis=-1)
    u = rng.random(rows.shape[0])[:, None] * c[:, -1:]
    return (c < u).sum(-1).clip(0, rows.shape[1] - 1).astype(np.int32)


def test_distribution_preserved_chi_square():
    V, T = 3, 200_000
    m = TinyModel(V, 7)
    rng = np.random.default_rng(70)
    seqs = np.full((T, 8), -1, np.int32)
    lens = np.zeros(T, np.int64)
    codes = np.zeros(T, np.int64)
    par = np.array([-1, 0, 0, 1, 1, 2, 2], np.int32)
    while True:
        act = np.nonzero(lens < 3)[0]
        if len(act) == 0:
            break
        B = len(act)
        c0, k = codes[act], lens[act]
        tok = np.zeros((B, 7), np.int32)
        ccode = np.zeros((B, 7), np.int64)
        ccode[:, 0] = c0
        for c in (1, 2):                       # children drafted from q(.|ctx)
            tok[:, c] = draw(rng, m.Q[c0])
            ccode[:, c] = m.child(c0, k, tok[:, c])
        for g in (3, 4, 5, 6):                 # grandchildren from q(.|ctx, x_c)
            pc = par[g]
            tok[:, g] = draw(rng, m.Q[ccode[:, pc]])
            ccode[:, g] = m.child(ccode[:, pc], k + 1, tok[:, g])
        llm = m.P[ccode]                       # p(.|sequence of the node)
        ssm = np.zeros_like(llm)
        ssm[:, 1:] = m.Q[ccode[:, par[1:]]]    # the row each token was drawn from
        path, plen, outt, st = oracle.verify_mss(
            np.tile(par, (B, 1)), tok, llm, ssm, rng.random((B, 7), dtype=np.float32),
            rng.random(B, dtype=np.float32))
        assert np.all(st == 0)
        for j in range(3):
            take = plen > j
            rows = act[take]
            seqs[rows, lens[rows]] = outt[take, j]
            codes[rows] = m.child(codes[rows], lens[rows], outt[take, j])
            lens[rows] += 1
    first3 = seqs[:, :3]
    cell = first3[:, 0] * V * V + first3[:, 1] * V + first3[:, 2]
    obs = np.bincount(cell, minlength=V ** 3)
    expect = np.zeros(V ** 3)
    P = m.P.astype(np.float64)
    P /= P.sum(-1, keepdims=True)
    for t1 in range(V):
        c1 = m.child(0, 0, t1)
        for t2 in range(V):
            c2 = m.child(c1, 1, t2)
            for t3 in range(V):
                expect[t1 * V * V + t2 * V + t3] = P[0, t1] * P[c1, t2] * P[c2, t3]
    chi = stats.chisquare(obs, expect * T / expect.sum())
    assert chi.pvalue > 1e-4, chi


def test_malformed_tree_and_determinism():
    rng = np.random.default_rng(80)
    B, N, V = 4, 6, 5
    par = np.tile(np.array([-1, 0, 0, 1, 1, 2], np.int32), (B, 1))
    par[2, 4] = 4
    llm = norm32(rng.random((B, N, V)))
    ssm = norm32(rng.random((B, N, V)))
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    ua = rng.random((B, N), dtype=np.float32)
    ub = rng.random(B, dtype=np.float32)
    a = oracle.verify_mss(par, tok, llm, ssm, ua, ub)
    b = oracle.verify_mss(par, tok, llm, ssm, ua, ub)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    path, plen, outt, st = a
    assert st[2] == oracle.E_TREE and plen[2] == 0 and np.all(path[2] == -1)
    assert np.all(st[[0, 1, 3]] == 0)
    tok[3, 5] = V          # a drafted token outside the vocabulary
    path, plen, outt, st = oracle.verify_mss(par, tok, llm, ssm, ua, ub)
    assert st[3] == oracle.E_SHAPE and plen[3] == 0 and np.all(outt[3] == -1)
