"""Pins of the oracle's in-place commit (tree node i at cache row L + i):
  * it equals the pinned separate-tree commit given the tree rows
    cache[L .. L+N) as the tree tensor, on random paths of random trees;
  * closed form: the path 0, 1, .., n-1 leaves the cache unchanged;
  * a hand example whose sources and destinations overlap;
  * rejected requests are untouched."""
import numpy as np
import pytest

import oracle


def random_case(seed, B=3, Hkv=2, N=12, D=8, Lmax=20):
    rng = np.random.default_rng(seed)
    Lcap = Lmax + N + 3
    kc = rng.normal(size=(B, Hkv, Lcap, D)).astype(np.float32)
    vc = rng.normal(size=(B, Hkv, Lcap, D)).astype(np.float32)
    L = rng.integers(0, Lmax + 1, B).astype(np.int32)
    path = np.full((B, N), -1, np.int32)
    plen = np.zeros(B, np.int32)
    for b in range(B):
        n = int(rng.integers(0, N + 1))
        nodes = np.sort(rng.choice(np.arange(1, N), size=max(n - 1, 0), replace=False)) if n else []
        p = ([0] + list(nodes))[:n]
        path[b, :n] = p
        plen[b] = n
    return kc, vc, L, path, plen, Lmax, N


@pytest.mark.parametrize("seed", range(6))
def test_equals_separate_tree_commit(seed):
    kc, vc, L, path, plen, Lmax, N = random_case(seed)
    B = kc.shape[0]
    kt = np.stack([kc[b, :, L[b]:L[b] + N] for b in range(B)])
    vt = np.stack([vc[b, :, L[b]:L[b] + N] for b in range(B)])
    ref = oracle.kv_commit(kt, vt, kc, vc, L, path, plen, Lmax)
    got = oracle.kv_commit_inplace(kc, vc, L, path, plen, Lmax, N)
    for b in range(B):   # rows L+n .. L+N keep the old tree rows in place; compare the rest
        n, l0 = plen[b], L[b]
        for g, r in zip(got[:2], ref[:2]):
            assert np.array_equal(g[b, :, :l0 + n], r[b, :, :l0 + n])
            assert np.array_equal(g[b, :, l0 + N:], r[b, :, l0 + N:])
    for g, r in zip(got[2:], ref[2:]):
        assert np.array_equal(g, r)


def test_identity_path_changes_nothing():
    kc, vc, L, path, plen, Lmax, N = random_case(9)
    for b in range(kc.shape[0]):
        path[b, :plen[b]] = np.arange(plen[b])
    k2, v2, clo, src, st = oracle.kv_commit_inplace(kc, vc, L, path, plen, Lmax, N)
    assert (st == 0).all() and np.array_equal(k2, kc) and np.array_equal(v2, vc)
    assert np.array_equal(clo, L + plen)


def test_overlapping_rows_hand_example():
    # rows 5..9 hold nodes 0..4 with values 0..4; path 0, 2, 3 -> rows 5, 6, 7 = 0, 2, 3
    kc = np.zeros((1, 1, 12, 1), np.float32)
    kc[0, 0, 5:10, 0] = np.arange(5)
    k2, v2, clo, src, st = oracle.kv_commit_inplace(
        kc, kc.copy(), np.array([5], np.int32), np.array([[0, 2, 3, -1, -1]], np.int32),
        np.array([3], np.int32), 5, 5)
    assert k2[0, 0, 5:10, 0].tolist() == [0, 2, 3, 3, 4] and clo.tolist() == [8]
    assert src.tolist() == [[0, 2, 3, -1, -1]]


def test_rejected_requests_untouched():
    kc, vc, L, path, plen, Lmax, N = random_case(4)
    L[0] = Lmax + 1                 # breaks the promise
    plen[1] = N + 1                 # longer than the tree
    path[2, 0] = N                  # not a node
    plen[2] = max(plen[2], 1)
    k2, v2, clo, src, st = oracle.kv_commit_inplace(kc, vc, L, path, plen, Lmax, N)
    assert st.tolist() == [2, 2, 2] and np.array_equal(k2, kc) and np.array_equal(v2, vc)
    assert np.array_equal(clo, L) and (src == -1).all()
