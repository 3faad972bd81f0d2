"""Pins of the oracle's KV commit ([SI] §4 "Tree-Based Parallel Decoding":
verified and speculated tokens share one KV cache, so committing a step keeps
the accepted path's rows, in path order, right after the prefix).

* a chain whose every node is accepted turns the cache into prefix ++ tree;
* rows at or after the new length and other requests are untouched (canaries);
* committed_src equals the path; bad lengths leave the request untouched.
"""
import numpy as np

import oracle


def setup(B=3, N=6, Hkv=2, D=4, Lcap=16, seed=0, dtype=np.uint16):
    rng = np.random.default_rng(seed)
    kt = rng.integers(0, 60000, (B, Hkv, N, D)).astype(dtype)
    vt = rng.integers(0, 60000, (B, Hkv, N, D)).astype(dtype)
    kc = np.full((B, Hkv, Lcap, D), 0xABCD, dtype)
    vc = np.full((B, Hkv, Lcap, D), 0x1234, dtype)
    return kt, vt, kc, vc


def test_full_chain_acceptance_appends_tree():
    kt, vt, kc, vc = setup(B=1, N=6, Lcap=16)
    L = np.array([5], np.int32)
    kc[0, :, :5] = 7
    path = np.arange(6, dtype=np.int32)[None]
    k2, v2, clo, src, st = oracle.kv_commit(kt, vt, kc, vc, L, path, np.array([6], np.int32),
                                            Lmax=5)
    assert st[0] == 0 and clo[0] == 11
    assert np.array_equal(k2[0, :, 5:11], kt[0]) and np.array_equal(v2[0, :, 5:11], vt[0])
    assert np.all(k2[0, :, :5] == 7) and np.all(k2[0, :, 11:] == 0xABCD)
    assert np.array_equal(src[0], path[0])


def test_partial_path_and_canaries():
    kt, vt, kc, vc = setup(B=3, N=6, Lcap=20)
    L = np.array([3, 0, 9], np.int32)
    path = np.array([[0, 2, 5, -1, -1, -1], [0, -1, -1, -1, -1, -1],
                     [0, 1, -1, -1, -1, -1]], np.int32)
    plen = np.array([3, 1, 2], np.int32)
    k2, v2, clo, src, st = oracle.kv_commit(kt, vt, kc, vc, L, path, plen, Lmax=9)
    assert np.all(st == 0) and list(clo) == [6, 1, 11]
    for b in range(3):
        for j in range(plen[b]):
            assert np.array_equal(k2[b, :, L[b] + j], kt[b, :, path[b, j]])
            assert np.array_equal(v2[b, :, L[b] + j], vt[b, :, path[b, j]])
        untouched = np.ones(20, bool)
        untouched[L[b]: L[b] + plen[b]] = False
        assert np.all(k2[b][:, untouched] == 0xABCD) and np.all(v2[b][:, untouched] == 0x1234)
        assert list(src[b, : plen[b]]) == list(path[b, : plen[b]])
        assert np.all(src[b, plen[b]:] == -1)


def test_float32_payload_is_bit_exact():
    kt, vt, kc, vc = setup(B=1, N=3, D=5, Lcap=8, dtype=np.float32)
    kt.view(np.uint32)[0, 0, 1, 0] = 0x7FC00001  # a NaN payload survives the copy
    path = np.array([[0, 1, 2]], np.int32)
    k2, _, _, _, st = oracle.kv_commit(kt, vt, kc, vc, np.array([2], np.int32), path,
                                       np.array([3], np.int32), Lmax=2)
    assert st[0] == 0
    assert np.array_equal(k2[0, :, 2:5].view(np.uint32), kt[0].view(np.uint32))


def test_out_of_bounds_requests_are_untouched():
    kt, vt, kc, vc = setup(B=4, N=4, Lcap=8)
    L = np.array([4, -1, 5, 2], np.int32)
    path = np.array([[0, 1, -1, -1], [0, -1, -1, -1], [0, -1, -1, -1], [0, 9, -1, -1]],
                    np.int32)
    plen = np.array([2, 1, 1, 2], np.int32)
    k2, v2, clo, src, st = oracle.kv_commit(kt, vt, kc, vc, L, path, plen, Lmax=4)
    assert st[0] == 0 and clo[0] == 6
    assert list(st[1:]) == [oracle.E_SHAPE] * 3     # L < 0; L > Lmax; bad node id
    assert list(clo[1:]) == [-1, 5, 2]
    assert np.all(k2[1:] == 0xABCD) and np.all(src[1:] == -1)


def test_aliasing_lengths_in_place():
    kt, vt, kc, vc = setup(B=2, N=4, Lcap=12)
    L = np.array([2, 3], np.int32)
    path = np.array([[0, 1, -1, -1], [0, 2, 3, -1]], np.int32)
    plen = np.array([2, 3], np.int32)
    _, _, clo, _, _ = oracle.kv_commit(kt, vt, kc, vc, L, path, plen, Lmax=3)
    assert list(clo) == [4, 6]
