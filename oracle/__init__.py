"""CPU oracle of the tree-based parallel decoding step -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never imports, links or calls it, and
this package imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64 attention); this module only
marshals numpy arrays.  Each function names the passage it follows:

* [SI]  "SpecInfer: Accelerating Generative Large Language Model Serving with
  Tree-based Speculative Inference and Verification" (paperlayer.ai summary of
  arXiv 2305.09781v4).
* [SSD] "Accelerating LLM Inference with Staged Speculative Decoding"
  (paperlayer.ai summary of arXiv 2308.04623v1).

Pinned by tests/test_oracle_*.py against closed forms, library routines
(torch SDPA in fp64, numpy matrix inverse and argmax), brute force and
statistical tests; see each function for its pins.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, E_SHAPE, E_TREE = 0, 2, 7


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fused multiply-adds)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fopenmp",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.orc_topology.argtypes = [I, I, P, P, P, P, P]
    lib.orc_tree_attn_rows.argtypes = [I, I, I, I, I, ctypes.c_double, P, P, P, I,
                                       P, P, P, P, P, I, P, P, P, P]
    lib.orc_verify_greedy.argtypes = [I, I, I, P, P, P, P, P, P, P, P]
    lib.orc_verify_mss.argtypes = [I, I, I, P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_kv_commit.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
    lib.orc_tree_expand.argtypes = [I, I, I, I, P, P, P, I, P, P, P, P, P]
    lib.orc_tree_merge.argtypes = [I, I, I, P, P, P, I, P, P, P, P, P]
    lib.orc_probs_from_logits.argtypes = [I, I, ctypes.c_float, I, ctypes.c_float, P, P]
    lib.orc_exp2_taylor.argtypes = [I, P, P]
    lib.orc_kv_commit_inplace.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P]
    U64 = ctypes.c_uint64
    lib.orc_philox4x64_10.argtypes = [P, P, P]
    lib.orc_verify_mss_seeded.argtypes = [I, I, I, P, P, P, P, P, U64, U64, P, P, P, P]
    lib.orc_set_threads.argtypes = [I]
    lib.orc_max_threads.restype = I
    for f in (lib.orc_kv_commit_inplace, lib.orc_topology, lib.orc_tree_attn_rows, lib.orc_verify_greedy,
              lib.orc_verify_mss, lib.orc_kv_commit, lib.orc_tree_expand, lib.orc_tree_merge,
              lib.orc_probs_from_logits, lib.orc_philox4x64_10, lib.orc_verify_mss_seeded,
              lib.orc_exp2_taylor,
              lib.orc_set_threads):
        f.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Run the wrappers against another build of oracle.c (the mutation tests
    compile deliberately broken copies to show that the pins catch them)."""
    global _lib
    saved = _load()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _nodes(n_nodes, B):
    """Per-request node counts int32 [B] (a batch of trees of different
    sizes, each in the first n_nodes[b] entries of its rows), or None: every
    request has N nodes."""
    if n_nodes is None:
        return None, None
    a, p = _c(n_nodes, np.int32)
    assert a.shape == (B,)
    return a, p


def topology(parents, n_nodes=None):
    """[SI] §4 "Tree Attention": depth and root->node ancestor bitsets.

    parents int32 [B,N], n_nodes int32 [B] or None -> (depth int32 [B,N],
    anc uint64 [B,N,W], status [B]); padding nodes get depth -1, no bits.
    """
    par, pp = _c(parents, np.int32)
    B, N = par.shape
    nn, nnp = _nodes(n_nodes, B)
    W = (N + 63) // 64
    depth = np.empty((B, N), np.int32)
    anc = np.empty((B, N, W), np.uint64)
    status = np.empty(B, np.int32)
    _load().orc_topology(B, N, pp, nnp, depth.ctypes.data_as(ctypes.c_void_p),
                         anc.ctypes.data_as(ctypes.c_void_p),
                         status.ctypes.data_as(ctypes.c_void_p))
    return depth, anc, status


def tree_attn_rows(q, k_cache, v_cache, cache_len, k_tree, v_tree, parents, scale,
                   rows, n_nodes=None):
    """[SI] §4 "Tree Attention"/"Tree-Based Parallel Decoding", [SSD] §3.

    Attention of the listed rows (b, i, hq) over prefix ++ path(root -> i), in
    fp64.  q [B,N,Hq,D], k/v_cache [B,Hkv,Lcap,D], k/v_tree [B,Hkv,N,D] (any
    float type; widened to float32 exactly), rows int [R,3], n_nodes int32
    [B] or None (rows of padding nodes i >= n_nodes[b] are zero).
    Returns (out float64 [R,D], lse float64 [R], status int32 [R]).
    """
    q, qp = _c(q, np.float32)
    kc, kcp = _c(k_cache, np.float32)
    vc, vcp = _c(v_cache, np.float32)
    kt, ktp = _c(k_tree, np.float32)
    vt, vtp = _c(v_tree, np.float32)
    par, pp = _c(parents, np.int32)
    cl, clp = _c(cache_len, np.int32)
    rows, rp = _c(np.asarray(rows).reshape(-1, 3), np.int32)
    B, N, Hq, D = q.shape
    Hkv, Lcap = kc.shape[1], kc.shape[2]
    assert kc.shape == (B, Hkv, Lcap, D) and vc.shape == kc.shape
    assert kt.shape == (B, Hkv, N, D) and vt.shape == kt.shape
    assert par.shape == (B, N) and cl.shape == (B,) and Hq % Hkv == 0
    assert rows.size == 0 or (rows[:, 0].min() >= 0 and rows[:, 0].max() < B
                              and rows[:, 2].min() >= 0 and rows[:, 2].max() < Hq)
    R = rows.shape[0]
    nn, nnp = _nodes(n_nodes, B)
    out = np.zeros((R, D), np.float64)
    lse = np.zeros(R, np.float64)
    status = np.zeros(R, np.int32)
    _load().orc_tree_attn_rows(B, N, Hq, Hkv, D, float(scale), qp, kcp, vcp, Lcap, clp,
                               ktp, vtp, pp, nnp, R, rp,
                               out.ctypes.data_as(ctypes.c_void_p),
                               lse.ctypes.data_as(ctypes.c_void_p),
                               status.ctypes.data_as(ctypes.c_void_p))
    return out, lse, status


def all_rows(B, N, Hq):
    """Every (b, i, hq) row in [B,N,Hq] order."""
    b, i, h = np.meshgrid(np.arange(B), np.arange(N), np.arange(Hq), indexing="ij")
    return np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1).astype(np.int32)


def tree_attn(q, k_cache, v_cache, cache_len, k_tree, v_tree, parents, scale, n_nodes=None):
    """Full output [B,N,Hq,D] (fp64), lse [B,N,Hq], per-row status."""
    B, N, Hq, D = np.shape(q)
    out, lse, st = tree_attn_rows(q, k_cache, v_cache, cache_len, k_tree, v_tree,
                                  parents, scale, all_rows(B, N, Hq), n_nodes)
    return out.reshape(B, N, Hq, D), lse.reshape(B, N, Hq), st.reshape(B, N, Hq)


def verify_greedy(parents, tokens, llm, n_nodes=None):
    """[SI] §4 "Token Tree Verification", §6: greedy acceptance of the tree.

    parents/tokens int32 [B,N], llm float32 [B,N,V] logits, n_nodes int32 [B]
    or None.  Returns (path [B,N], path_len [B], out_tokens [B,N], status [B]).
    """
    par, pp = _c(parents, np.int32)
    tok, tp = _c(tokens, np.int32)
    lg, lp = _c(llm, np.float32)
    B, N = par.shape
    V = lg.shape[2]
    assert lg.shape == (B, N, V) and tok.shape == (B, N)
    nn, nnp = _nodes(n_nodes, B)
    path = np.empty((B, N), np.int32)
    plen = np.empty(B, np.int32)
    outt = np.empty((B, N), np.int32)
    st = np.empty(B, np.int32)
    _load().orc_verify_greedy(B, N, V, pp, tp, nnp, lp, path.ctypes.data_as(ctypes.c_void_p),
                              plen.ctypes.data_as(ctypes.c_void_p),
                              outt.ctypes.data_as(ctypes.c_void_p),
                              st.ctypes.data_as(ctypes.c_void_p))
    return path, plen, outt, st


def verify_mss(parents, tokens, llm, ssm, u_accept, u_bonus, n_nodes=None):
    """[SI] §4 "Token Verification": multi-step speculative sampling.

    llm/ssm float32 [B,N,V] probabilities, u_accept float32 [B,N], u_bonus
    float32 [B] uniforms in [0,1).  Returns (path, path_len, out_tokens, status).
    """
    par, pp = _c(parents, np.int32)
    tok, tp = _c(tokens, np.int32)
    p, ppr = _c(llm, np.float32)
    q, qpr = _c(ssm, np.float32)
    ua, uap = _c(u_accept, np.float32)
    ub, ubp = _c(u_bonus, np.float32)
    B, N = par.shape
    V = p.shape[2]
    assert p.shape == (B, N, V) and q.shape == p.shape
    assert ua.shape == (B, N) and ub.shape == (B,) and tok.shape == (B, N)
    nn, nnp = _nodes(n_nodes, B)
    path = np.empty((B, N), np.int32)
    plen = np.empty(B, np.int32)
    outt = np.empty((B, N), np.int32)
    st = np.empty(B, np.int32)
    _load().orc_verify_mss(B, N, V, pp, tp, nnp, ppr, qpr, uap, ubp,
                           path.ctypes.data_as(ctypes.c_void_p),
                           plen.ctypes.data_as(ctypes.c_void_p),
                           outt.ctypes.data_as(ctypes.c_void_p),
                           st.ctypes.data_as(ctypes.c_void_p))
    return path, plen, outt, st


def philox4x64_10(counter, key):
    """Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11, "Parallel random
    numbers: as easy as 1, 2, 3"): the four 64-bit output words for a counter
    of four 64-bit words (word 0 least significant) and a key of two."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64).reshape(2))
    out = np.empty(4, np.uint64)
    P = ctypes.c_void_p
    _load().orc_philox4x64_10(c.ctypes.data_as(P), k.ctypes.data_as(P), out.ctypes.data_as(P))
    return out


def verify_mss_seeded(parents, tokens, llm, ssm, seed, step, n_nodes=None):
    """[SI] §4 "Token Verification": multi-step speculative sampling with the
    uniforms drawn from Philox4x64-10, key (seed, 0): the ratio test of the
    j-th child (ascending node index) of node u in request b takes counter
    (j, u, b, step), the final draw at u counter (2^63, u, b, step), each
    using the 24 high bits of output word 0.  Returns (path, path_len,
    out_tokens, status) as verify_mss."""
    par, pp = _c(parents, np.int32)
    tok, tp = _c(tokens, np.int32)
    p, ppr = _c(llm, np.float32)
    q, qpr = _c(ssm, np.float32)
    B, N = par.shape
    V = p.shape[2]
    assert p.shape == (B, N, V) and q.shape == p.shape and tok.shape == (B, N)
    nn, nnp = _nodes(n_nodes, B)
    path = np.empty((B, N), np.int32)
    plen = np.empty(B, np.int32)
    outt = np.empty((B, N), np.int32)
    st = np.empty(B, np.int32)
    P = ctypes.c_void_p
    _load().orc_verify_mss_seeded(B, N, V, pp, tp, nnp, ppr, qpr, int(seed) & (2**64 - 1),
                                  int(step) & (2**64 - 1), path.ctypes.data_as(P),
                                  plen.ctypes.data_as(P), outt.ctypes.data_as(P),
                                  st.ctypes.data_as(P))
    return path, plen, outt, st


def set_threads(n):
    """Threads the oracle's parallel loops use from now on."""
    _load().orc_set_threads(int(n))


def max_threads():
    """Threads the oracle's parallel loops use."""
    return int(_load().orc_max_threads())


def kv_commit(k_tree, v_tree, k_cache, v_cache, cache_len_in, path, path_len, Lmax):
    """[SI] §4 "Tree-Based Parallel Decoding": keep the accepted path's KV.

    Works on copies of k_cache/v_cache (any dtype, bytes are copied).  Returns
    (k_cache', v_cache', cache_len_out, committed_src, status).
    """
    kt = np.ascontiguousarray(k_tree)
    vt = np.ascontiguousarray(v_tree)
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    assert kt.dtype == kc.dtype == vt.dtype == vc.dtype
    B, Hkv, N, D = kt.shape
    Lcap = kc.shape[2]
    cl, clp = _c(cache_len_in, np.int32)
    pa, pap = _c(path, np.int32)
    pl, plp = _c(path_len, np.int32)
    clo = np.empty(B, np.int32)
    src = np.empty((B, N), np.int32)
    st = np.empty(B, np.int32)
    V = ctypes.c_void_p
    _load().orc_kv_commit(B, N, Hkv, D, kt.dtype.itemsize, Lcap, int(Lmax),
                          kt.ctypes.data_as(V), vt.ctypes.data_as(V),
                          kc.ctypes.data_as(V), vc.ctypes.data_as(V), clp,
                          clo.ctypes.data_as(V), pap, plp, src.ctypes.data_as(V),
                          st.ctypes.data_as(V))
    return kc, vc, clo, src, st


def tree_expand(probs, frontier, n_in, k, parents, tokens, src_row=None):
    """[SI] §3 "Expansion-based token tree construction", one level: every
    frontier node (in order) gets its row's k most probable tokens (ties: the
    lower token id) as children, appended after the n_in[b] existing nodes.

    probs float32 [B,F,V], frontier int32 [B,F] (-1 = none), n_in int32 [B],
    parents/tokens int32 [B,Ncap] (the existing tree; copies are returned),
    src_row int32 [B,Ncap] or None ->
    (parents, tokens, src_row, n_out int32 [B], status int32 [B]).
    """
    pr, pp = _c(probs, np.float32)
    B, F, V = pr.shape
    fr, fp = _c(frontier, np.int32)
    ni, nip = _c(n_in, np.int32)
    par = np.array(parents, np.int32, copy=True, order="C")
    tok = np.array(tokens, np.int32, copy=True, order="C")
    Ncap = par.shape[1]
    src = (np.full((B, Ncap), -1, np.int32) if src_row is None
           else np.array(src_row, np.int32, copy=True, order="C"))
    n_out = np.empty(B, np.int32)
    status = np.empty(B, np.int32)
    P = ctypes.c_void_p
    _load().orc_tree_expand(B, F, V, int(k), pp, fp, nip, Ncap, par.ctypes.data_as(P),
                            tok.ctypes.data_as(P), src.ctypes.data_as(P),
                            n_out.ctypes.data_as(P), status.ctypes.data_as(P))
    return par, tok, src, n_out, status


def tree_merge(seqs, seq_len, root_tok, Ncap):
    """[SI] §3 "Merge-based token tree construction": the union of S
    speculated sequences below the root, each distinct prefix one node,
    numbered depth by depth in order of the lowest sequence index reaching it.

    seqs int32 [B,S,Ls], seq_len int32 [B,S], root_tok int32 [B] ->
    (parents, tokens, src int32 [B,Ncap] (-1 past n_out), n_out [B], status [B]).
    """
    sq, sp = _c(seqs, np.int32)
    B, S, Ls = sq.shape
    ln, lp = _c(seq_len, np.int32)
    rt, rp = _c(root_tok, np.int32)
    par = np.full((B, Ncap), -1, np.int32)
    tok = np.full((B, Ncap), -1, np.int32)
    src = np.full((B, Ncap), -1, np.int32)
    n_out = np.empty(B, np.int32)
    status = np.empty(B, np.int32)
    P = ctypes.c_void_p
    _load().orc_tree_merge(B, S, Ls, sp, lp, rp, int(Ncap), par.ctypes.data_as(P),
                           tok.ctypes.data_as(P), src.ctypes.data_as(P),
                           n_out.ctypes.data_as(P), status.ctypes.data_as(P))
    return par, tok, src, n_out, status


def probs_from_logits(logits, T=1.0, topk=0, top_p=1.0):
    """[SI] §4 "Token Verification", §7 (top-k / top-p sampling); [SSD] §4:
    next-token probabilities from logits [..., V] at temperature T, over the
    topk highest logits when topk > 0 (equal logits: the lower token id
    first), then over the shortest prefix of those holding the share top_p
    of their mass when 0 < top_p < 1.  fp32 arithmetic fixed exactly (see
    oracle.c): 2^x by a degree-7 Taylor polynomial after range reduction,
    masses as integers in 2^-40 units."""
    z, zp = _c(logits, np.float32)
    V = z.shape[-1]
    R = z.size // V
    out = np.empty_like(z)
    _load().orc_probs_from_logits(R, V, float(T), int(topk), float(top_p), zp,
                                  out.ctypes.data_as(ctypes.c_void_p))
    return out


def exp2_taylor(t):
    """2^t (fp32, t <= 0) exactly as the probabilities compute it."""
    t, tp = _c(t, np.float32)
    out = np.empty_like(t)
    _load().orc_exp2_taylor(t.size, tp, out.ctypes.data_as(ctypes.c_void_p))
    return out


def verify_mss_logits(parents, tokens, llm_logits, ssm_logits, T, topk, top_p, seed, step,
                      n_nodes=None):
    """[SI] §4 "Token Verification" from raw logits: multi-step speculative
    sampling (seeded draws) over the distributions probs_from_logits gives
    for the LLM's and the speculator's logits at temperature T (top-k, top-p
    as there)."""
    p = probs_from_logits(llm_logits, T, topk, top_p)
    q = probs_from_logits(ssm_logits, T, topk, top_p)
    return verify_mss_seeded(parents, tokens, p, q, seed, step, n_nodes)


def kv_commit_inplace(k_cache, v_cache, cache_len_in, path, path_len, Lmax, N):
    """[SI] §4 "Tree-Based Parallel Decoding" with the tree inside the cache:
    node i at row L + i; row L + j takes the old row L + path[j] (j < n).

    Works on copies of k_cache/v_cache [B,Hkv,Lcap,D] (bytes are copied).
    Returns (k_cache', v_cache', cache_len_out, committed_src, status).
    """
    kc = np.array(k_cache, copy=True, order="C")
    vc = np.array(v_cache, copy=True, order="C")
    assert kc.dtype == vc.dtype
    B, Hkv, Lcap, D = kc.shape
    cl, clp = _c(cache_len_in, np.int32)
    pa, pap = _c(path, np.int32)
    pl, plp = _c(path_len, np.int32)
    clo = np.empty(B, np.int32)
    src = np.empty((B, N), np.int32)
    st = np.empty(B, np.int32)
    V = ctypes.c_void_p
    _load().orc_kv_commit_inplace(B, N, Hkv, D, kc.dtype.itemsize, Lcap, int(Lmax),
                                  kc.ctypes.data_as(V), vc.ctypes.data_as(V), clp,
                                  clo.ctypes.data_as(V), pap, plp, src.ctypes.data_as(V),
                                  st.ctypes.data_as(V))
    return kc, vc, clo, src, st
