"""token_tree_verification_attn_amd -- Python binding of libttv.

libttv is the C-ABI library (include/ttv.h) that runs the tree-based parallel
decoding step of tree speculative inference on AMD MI355X (gfx950):

* ``tree_topology``  ancestor bitsets / depths of each request's token tree
* ``tree_attn``      attention of every tree node over prefix KV + its root path
* ``tree_verify``    greedy or multi-step-speculative-sampling acceptance
* ``kv_commit``      accepted path's KV rows appended to the contiguous cache

This module only marshals arguments: it checks tensor dtypes, shapes, devices
and contiguity, allocates outputs with torch, and passes raw device pointers
plus torch's current HIP stream to the library.  Every step of the path runs in
the library's kernels; there is no fallback.  Importing works anywhere; the
first call raises ``LibraryNotBuilt`` if libttv.so is missing and ``TTVError``
for a non-OK status.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["tree_topology", "tree_attn", "tree_verify", "tree_verify_uniforms", "kv_commit",
           "tree_verify_commit", "tree_verify_logits", "tree_expand", "tree_merge",
           "probs_from_logits",
           "kv_commit_inplace", "tree_attn_noalloc", "tree_attn_workspace_size",
           "tree_verify_workspace_size",
           "status_string",
           "TTVError", "LibraryNotBuilt", "lib", "LIB_PATH", "GREEDY", "STOCHASTIC"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libttv.so")

(OK, E_NULL, E_SHAPE, E_DTYPE, E_UNSUPPORTED, E_WORKSPACE, E_LAUNCH, E_TREE, E_ALIGN,
 E_SCRATCH) = range(10)
NOALLOC_SCRATCH_BYTES = 48 << 20
F32, BF16 = 0, 1
GREEDY, STOCHASTIC = 0, 1
MAX_NODES = 128


class LibraryNotBuilt(ImportError):
    pass


class TTVError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))


_lib = None
_P, _I, _F, _SZ, _U64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t,
                         ctypes.c_uint64)


def lib():
    """The loaded libttv.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                "libttv.so is not built; run `python -m token_tree_verification_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.ttv_status_string.argtypes = [_I]
        L.ttv_status_string.restype = ctypes.c_char_p
        L.ttv_version.restype = _I
        L.ttv_tree_topology.argtypes = [_I, _I, _P, _P, _P, _P, _P]
        L.ttv_tree_attn.argtypes = [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P, _I, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.ttv_tree_attn_tuned.argtypes = [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P, _I, _P,
                                          _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _P]
        L.ttv_tree_attn_varlen.argtypes = [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P, _I, _P,
                                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.ttv_tree_verify_varlen.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _U64, _U64, _P,
                                             _P, _P, _P, _P, _SZ, _P]
        L.ttv_tree_verify_commit_varlen.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                                    _P, _P, _U64, _U64, _P, _P, _P, _P, _P, _P,
                                                    _I, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.ttv_tree_attn_noalloc.argtypes = [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P, _I,
                                            _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P]
        L.ttv_tree_attn_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I]
        L.ttv_tree_attn_workspace_size.restype = _SZ
        L.ttv_tree_attn_tuned_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I]
        L.ttv_tree_attn_tuned_workspace_size.restype = _SZ
        L.ttv_tree_verify.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _U64, _U64, _P, _P, _P, _P,
                                      _P, _SZ, _P]
        L.ttv_tree_verify_uniforms.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _P, _P]
        L.ttv_tree_verify_workspace_size.argtypes = [_I, _I, _I, _I]
        L.ttv_tree_verify_workspace_size.restype = _SZ
        L.ttv_kv_commit.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P,
                                    _P, _P, _P]
        L.ttv_tree_expand.argtypes = [_I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P]
        L.ttv_tree_merge.argtypes = [_I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P]
        L.ttv_probs_from_logits.argtypes = [_I, _I, _F, _I, _F, _P, _P, _P]
        L.ttv_tree_verify_logits.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _F, _I, _F, _U64,
                                             _U64, _P, _P, _P, _P, _P, _SZ, _P]
        L.ttv_tree_verify_logits_workspace_size.argtypes = [_I, _I, _I]
        L.ttv_tree_verify_logits_workspace_size.restype = _SZ
        L.ttv_kv_commit_inplace.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P,
                                            _P, _P, _P]
        L.ttv_tree_verify_commit.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _U64,
                                             _U64, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                             _P, _SZ, _P]
        for f in ("ttv_tree_verify_commit", "ttv_kv_commit_inplace", "ttv_tree_topology",
                  "ttv_tree_attn", "ttv_tree_attn_tuned", "ttv_tree_attn_noalloc",
                  "ttv_tree_attn_varlen", "ttv_tree_verify_varlen",
                  "ttv_tree_verify_commit_varlen", "ttv_tree_verify",
                  "ttv_tree_verify_uniforms", "ttv_kv_commit", "ttv_tree_expand",
                  "ttv_tree_merge", "ttv_probs_from_logits", "ttv_tree_verify_logits"):
            getattr(L, f).restype = _I
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().ttv_status_string(int(s)).decode()


def _check(fn, st):
    if st != OK:
        raise TTVError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _dt(dtype):
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dtype)


def tree_topology(parents: torch.Tensor, dev_status: Optional[torch.Tensor] = None):
    """Ancestor bitsets and depths; returns (anc int64 [B,N,W] holding the uint64
    words, depth int32 [B,N], dev_status int32 [B])."""
    B, N = parents.shape
    dev = parents.device
    _need(parents, "parents", torch.int32, (B, N), dev)
    W = (N + 63) // 64
    anc = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    _check("ttv_tree_topology", lib().ttv_tree_topology(B, N, _ptr(parents), _ptr(anc),
                                                        _ptr(depth), _ptr(dev_status),
                                                        _stream(dev)))
    return anc, depth, dev_status


def tree_attn_workspace_size(dtype, B, N, Hq, Hkv, D, Lmax, rows_per_block=0, chunk_keys=0):
    if rows_per_block or chunk_keys:
        n = lib().ttv_tree_attn_tuned_workspace_size(_dt(dtype), B, N, Hq, Hkv, D, Lmax,
                                                     rows_per_block, chunk_keys)
    else:
        n = lib().ttv_tree_attn_workspace_size(_dt(dtype), B, N, Hq, Hkv, D, Lmax)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported tree_attn sizes")
    return n


def tree_attn(q, k_cache, v_cache, cache_len, k_tree, v_tree, parents, Lmax: int,
              scale: Optional[float] = None, out=None, lse=None, want_lse: bool = True,
              dev_status=None, workspace=None, anc_out=None, depth_out=None,
              rows_per_block: int = 0, chunk_keys: int = 0, n_nodes=None):
    """Tree attention for every node; returns (out [B,N,Hq,D], lse [B,N,Hq] or None,
    dev_status [B]).  k_tree = v_tree = None reads node i's K/V from cache row
    L_b + i.  anc_out (int64 [B,N,W] holding the uint64 words) and depth_out
    (int32 [B,N]), when given, receive the tree mask and the node depths.
    rows_per_block / chunk_keys other than 0 fix the launch shape
    (ttv_tree_attn_tuned).  n_nodes (int32 [B]) gives each request's node
    count in a batch of trees of different sizes (ttv_tree_attn_varlen)."""
    B, N, Hq, D = q.shape
    Hkv, Lcap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    dt = q.dtype
    _need(q, "q", dt, (B, N, Hq, D), dev)
    _need(k_cache, "k_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(v_cache, "v_cache", dt, (B, Hkv, Lcap, D), dev)
    if k_tree is not None or v_tree is not None:  # both None: tree K/V at cache rows L_b + i
        _need(k_tree, "k_tree", dt, (B, Hkv, N, D), dev)
        _need(v_tree, "v_tree", dt, (B, Hkv, N, D), dev)
    _need(cache_len, "cache_len", torch.int32, (B,), dev)
    _need(parents, "parents", torch.int32, (B, N), dev)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=dt, device=dev)
    _need(out, "out", dt, (B, N, Hq, D), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, N, Hq), dev)
    if anc_out is not None:
        _need(anc_out, "anc_out", torch.int64, (B, N, (N + 63) // 64), dev)
    if depth_out is not None:
        _need(depth_out, "depth_out", torch.int32, (B, N), dev)
    if n_nodes is not None:
        _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
        if rows_per_block or chunk_keys:
            raise ValueError("n_nodes takes the automatic launch shape")
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = tree_attn_workspace_size(dt, B, N, Hq, Hkv, D, Lmax, rows_per_block, chunk_keys)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)  # needs no initialisation
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_dt(dt), B, N, Hq, Hkv, D, float(scale), _ptr(q), _ptr(k_cache), _ptr(v_cache), Lcap,
            _ptr(cache_len), int(Lmax), _ptr(k_tree), _ptr(v_tree), _ptr(parents), _ptr(out),
            _ptr(lse), _ptr(anc_out), _ptr(depth_out), _ptr(dev_status), _ptr(workspace), wsb)
    if n_nodes is not None:
        args = args[:16] + (_ptr(n_nodes),) + args[16:]
        _check("ttv_tree_attn_varlen", lib().ttv_tree_attn_varlen(*args, _stream(dev)))
    elif rows_per_block or chunk_keys:
        _check("ttv_tree_attn_tuned", lib().ttv_tree_attn_tuned(*args, rows_per_block,
                                                                chunk_keys, _stream(dev)))
    else:
        _check("ttv_tree_attn", lib().ttv_tree_attn(*args, _stream(dev)))
    return out, lse, dev_status


def tree_attn_noalloc(q, k_cache, v_cache, cache_len, k_tree, v_tree, parents, Lmax: int,
                      scale: Optional[float] = None, out=None, lse=None, dev_status=None,
                      anc_out=None, depth_out=None, rows_per_block: int = 0,
                      chunk_keys: int = 0):
    """tree_attn without a workspace: the library keeps the split partials in
    its own static device array (ttv_tree_attn_noalloc), so the call itself
    allocates nothing when out, lse and dev_status are given (None: allocated
    here by torch).  Calls on one GPU must not overlap in time."""
    B, N, Hq, D = q.shape
    Hkv, Lcap = k_cache.shape[1], k_cache.shape[2]
    dev = q.device
    dt = q.dtype
    _need(q, "q", dt, (B, N, Hq, D), dev)
    _need(k_cache, "k_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(v_cache, "v_cache", dt, (B, Hkv, Lcap, D), dev)
    if k_tree is not None or v_tree is not None:
        _need(k_tree, "k_tree", dt, (B, Hkv, N, D), dev)
        _need(v_tree, "v_tree", dt, (B, Hkv, N, D), dev)
    _need(cache_len, "cache_len", torch.int32, (B,), dev)
    _need(parents, "parents", torch.int32, (B, N), dev)
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=dt, device=dev)
    _need(out, "out", dt, (B, N, Hq, D), dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, N, Hq), dev)
    if anc_out is not None:
        _need(anc_out, "anc_out", torch.int64, (B, N, (N + 63) // 64), dev)
    if depth_out is not None:
        _need(depth_out, "depth_out", torch.int32, (B, N), dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib().ttv_tree_attn_noalloc(_dt(dt), B, N, Hq, Hkv, D, float(scale), _ptr(q),
                                     _ptr(k_cache), _ptr(v_cache), Lcap, _ptr(cache_len),
                                     int(Lmax), _ptr(k_tree), _ptr(v_tree), _ptr(parents),
                                     _ptr(out), _ptr(lse), _ptr(anc_out), _ptr(depth_out),
                                     _ptr(dev_status), rows_per_block, chunk_keys, _stream(dev))
    _check("ttv_tree_attn_noalloc", st)
    return out, lse, dev_status


def tree_verify_workspace_size(mode, B, N, V):
    n = lib().ttv_tree_verify_workspace_size(mode, B, N, V)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported tree_verify sizes")
    return n


def tree_verify(mode: int, parents, tokens, llm, ssm=None, seed: int = 0, step: int = 0,
                path=None, path_len=None, out_tokens=None, dev_status=None, workspace=None,
                n_nodes=None):
    """Greedy (mode GREEDY, llm = logits) or multi-step speculative sampling
    (mode STOCHASTIC, llm/ssm = probabilities, uniforms drawn on the device
    from Philox4x64-10 with key (seed, 0) and counter word 3 = step).
    n_nodes (int32 [B]): each request's node count (ttv_tree_verify_varlen).
    Returns (path [B,N], path_len [B], out_tokens [B,N], dev_status [B])."""
    B, N = parents.shape
    V = llm.shape[2]
    dev = parents.device
    _need(parents, "parents", torch.int32, (B, N), dev)
    _need(tokens, "tokens", torch.int32, (B, N), dev)
    _need(llm, "llm", torch.float32, (B, N, V), dev)
    if mode == STOCHASTIC:
        _need(ssm, "ssm", torch.float32, (B, N, V), dev)
    if n_nodes is not None:
        _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    path, path_len, out_tokens, dev_status = _verify_outputs(B, N, dev, path, path_len,
                                                             out_tokens, dev_status)
    nbytes = tree_verify_workspace_size(mode, B, N, V)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (_ptr(llm), _ptr(ssm), _u64(seed), _u64(step), _ptr(path), _ptr(path_len),
            _ptr(out_tokens), _ptr(dev_status), _ptr(workspace), wsb, _stream(dev))
    if n_nodes is not None:
        st = lib().ttv_tree_verify_varlen(mode, B, N, V, _ptr(parents), _ptr(tokens),
                                          _ptr(n_nodes), *tail)
    else:
        st = lib().ttv_tree_verify(mode, B, N, V, _ptr(parents), _ptr(tokens), *tail)
    _check("ttv_tree_verify", st)
    return path, path_len, out_tokens, dev_status


def tree_verify_uniforms(parents, tokens, llm, ssm, u_accept, u_bonus, path=None, path_len=None,
                         out_tokens=None, dev_status=None):
    """Multi-step speculative sampling with the caller's uniforms: u_accept
    [B,N] (the test of child c uses u_accept[b,c]) and u_bonus [B] (the final
    draw).  Returns (path, path_len, out_tokens, dev_status)."""
    B, N = parents.shape
    V = llm.shape[2]
    dev = parents.device
    _need(parents, "parents", torch.int32, (B, N), dev)
    _need(tokens, "tokens", torch.int32, (B, N), dev)
    _need(llm, "llm", torch.float32, (B, N, V), dev)
    _need(ssm, "ssm", torch.float32, (B, N, V), dev)
    _need(u_accept, "u_accept", torch.float32, (B, N), dev)
    _need(u_bonus, "u_bonus", torch.float32, (B,), dev)
    path, path_len, out_tokens, dev_status = _verify_outputs(B, N, dev, path, path_len,
                                                             out_tokens, dev_status)
    st = lib().ttv_tree_verify_uniforms(B, N, V, _ptr(parents), _ptr(tokens), _ptr(llm),
                                        _ptr(ssm), _ptr(u_accept), _ptr(u_bonus), _ptr(path),
                                        _ptr(path_len), _ptr(out_tokens), _ptr(dev_status),
                                        _stream(dev))
    _check("ttv_tree_verify_uniforms", st)
    return path, path_len, out_tokens, dev_status


def _u64(x):
    x = int(x)
    if not 0 <= x < 2 ** 64:
        raise ValueError("seed and step are unsigned 64-bit integers")
    return x


def _verify_outputs(B, N, dev, path, path_len, out_tokens, dev_status):
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    _need(path, "path", torch.int32, (B, N), dev)
    _need(path_len, "path_len", torch.int32, (B,), dev)
    _need(out_tokens, "out_tokens", torch.int32, (B, N), dev)
    _need(dev_status, "dev_status", torch.int32, (B,), dev)
    return path, path_len, out_tokens, dev_status


def kv_commit(k_tree, v_tree, k_cache, v_cache, cache_len_in, path, path_len, Lmax: int,
              cache_len_out=None, committed_src=None, want_src: bool = True, dev_status=None):
    """Append the accepted path's KV rows to the cache in place.  Returns
    (cache_len_out [B], committed_src [B,N] or None, dev_status [B])."""
    B, Hkv, N, D = k_tree.shape
    Lcap = k_cache.shape[2]
    dev = k_tree.device
    dt = k_tree.dtype
    _need(k_tree, "k_tree", dt, (B, Hkv, N, D), dev)
    _need(v_tree, "v_tree", dt, (B, Hkv, N, D), dev)
    _need(k_cache, "k_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(v_cache, "v_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(cache_len_in, "cache_len_in", torch.int32, (B,), dev)
    _need(path, "path", torch.int32, (B, N), dev)
    _need(path_len, "path_len", torch.int32, (B,), dev)
    if cache_len_out is None:
        cache_len_out = torch.empty(B, dtype=torch.int32, device=dev)
    _need(cache_len_out, "cache_len_out", torch.int32, (B,), dev)
    if committed_src is None and want_src:
        committed_src = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib().ttv_kv_commit(_dt(dt), B, N, Hkv, D, Lcap, _ptr(k_tree), _ptr(v_tree),
                             _ptr(k_cache), _ptr(v_cache), _ptr(cache_len_in),
                             _ptr(cache_len_out), int(Lmax), _ptr(path), _ptr(path_len),
                             _ptr(committed_src), _ptr(dev_status), _stream(dev))
    _check("ttv_kv_commit", st)
    return cache_len_out, committed_src, dev_status


def tree_verify_commit(mode: int, parents, tokens, llm, k_tree, v_tree, k_cache, v_cache,
                       cache_len_in, Lmax: int, ssm=None, seed: int = 0, step: int = 0,
                       cache_len_out=None, path=None, path_len=None, out_tokens=None,
                       committed_src=None, want_src: bool = True, dev_status=None,
                       workspace=None, n_nodes=None):
    """Verification (mode GREEDY or STOCHASTIC with (seed, step), as in
    tree_verify) and the KV
    commit of its path in one pass: the same results as tree_verify(...) then
    kv_commit(...); cache_len_out may be cache_len_in; n_nodes (int32 [B]) as
    in tree_verify.  Returns (path,
    path_len, out_tokens, cache_len_out, committed_src or None, dev_status)."""
    B, N = parents.shape
    V = llm.shape[2]
    _, Hkv, _, D = k_tree.shape
    Lcap = k_cache.shape[2]
    dev = parents.device
    dt = k_tree.dtype
    _need(parents, "parents", torch.int32, (B, N), dev)
    _need(tokens, "tokens", torch.int32, (B, N), dev)
    _need(llm, "llm", torch.float32, (B, N, V), dev)
    if mode == STOCHASTIC:
        _need(ssm, "ssm", torch.float32, (B, N, V), dev)
    _need(k_tree, "k_tree", dt, (B, Hkv, N, D), dev)
    _need(v_tree, "v_tree", dt, (B, Hkv, N, D), dev)
    _need(k_cache, "k_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(v_cache, "v_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(cache_len_in, "cache_len_in", torch.int32, (B,), dev)
    if cache_len_out is None:
        cache_len_out = torch.empty(B, dtype=torch.int32, device=dev)
    _need(cache_len_out, "cache_len_out", torch.int32, (B,), dev)
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    if path_len is None:
        path_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if committed_src is None and want_src:
        committed_src = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = tree_verify_workspace_size(mode, B, N, V)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    tail = (_ptr(llm), _ptr(ssm), _u64(seed), _u64(step), _ptr(k_tree), _ptr(v_tree),
            _ptr(k_cache), _ptr(v_cache), _ptr(cache_len_in), _ptr(cache_len_out), int(Lmax),
            _ptr(path), _ptr(path_len), _ptr(out_tokens), _ptr(committed_src), _ptr(dev_status),
            _ptr(workspace), wsb, _stream(dev))
    if n_nodes is not None:
        _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
        st = lib().ttv_tree_verify_commit_varlen(mode, _dt(dt), B, N, V, Hkv, D, Lcap,
                                                 _ptr(parents), _ptr(tokens), _ptr(n_nodes),
                                                 *tail)
    else:
        st = lib().ttv_tree_verify_commit(mode, _dt(dt), B, N, V, Hkv, D, Lcap, _ptr(parents),
                                          _ptr(tokens), *tail)
    _check("ttv_tree_verify_commit", st)
    return path, path_len, out_tokens, cache_len_out, committed_src, dev_status


def tree_verify_logits(parents, tokens, llm_logits, ssm_logits, temperature: float,
                       topk: int = 0, top_p: float = 1.0, seed: int = 0, step: int = 0,
                       n_nodes=None, path=None, path_len=None, out_tokens=None,
                       dev_status=None, workspace=None):
    """Multi-step speculative sampling fed with logits [B,N,V]: the
    distributions probs_from_logits(temperature, topk, top_p) gives for
    them, computed by the verifier as it reads them.  Returns (path,
    path_len, out_tokens, dev_status)."""
    B, N = parents.shape
    V = llm_logits.shape[2]
    dev = parents.device
    _need(parents, "parents", torch.int32, (B, N), dev)
    _need(tokens, "tokens", torch.int32, (B, N), dev)
    _need(llm_logits, "llm_logits", torch.float32, (B, N, V), dev)
    _need(ssm_logits, "ssm_logits", torch.float32, (B, N, V), dev)
    if n_nodes is not None:
        _need(n_nodes, "n_nodes", torch.int32, (B,), dev)
    path, path_len, out_tokens, dev_status = _verify_outputs(B, N, dev, path, path_len,
                                                             out_tokens, dev_status)
    nbytes = lib().ttv_tree_verify_logits_workspace_size(B, N, V)
    if nbytes == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported tree_verify_logits sizes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    st = lib().ttv_tree_verify_logits(B, N, V, _ptr(parents), _ptr(tokens), _ptr(n_nodes),
                                      _ptr(llm_logits), _ptr(ssm_logits), float(temperature),
                                      int(topk), float(top_p), _u64(seed), _u64(step),
                                      _ptr(path), _ptr(path_len), _ptr(out_tokens),
                                      _ptr(dev_status), _ptr(workspace), wsb, _stream(dev))
    _check("ttv_tree_verify_logits", st)
    return path, path_len, out_tokens, dev_status


def tree_expand(probs, frontier, n_in, k: int, parents, tokens, src_row=None, n_out=None,
                dev_status=None):
    """One level of expansion-based tree construction, appended in place to
    parents/tokens [B,Ncap] (and src_row [B,Ncap] if given): every frontier
    node's k most probable tokens become its children.  Returns (n_out [B],
    dev_status [B])."""
    B, F, V = probs.shape
    Ncap = parents.shape[1]
    dev = probs.device
    _need(probs, "probs", torch.float32, (B, F, V), dev)
    _need(frontier, "frontier", torch.int32, (B, F), dev)
    _need(n_in, "n_in", torch.int32, (B,), dev)
    _need(parents, "parents", torch.int32, (B, Ncap), dev)
    _need(tokens, "tokens", torch.int32, (B, Ncap), dev)
    if src_row is not None:
        _need(src_row, "src_row", torch.int32, (B, Ncap), dev)
    if n_out is None:
        n_out = torch.empty(B, dtype=torch.int32, device=dev)
    _need(n_out, "n_out", torch.int32, (B,), dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib().ttv_tree_expand(B, F, V, int(k), _ptr(probs), _ptr(frontier), _ptr(n_in), Ncap,
                               _ptr(parents), _ptr(tokens), _ptr(src_row), _ptr(n_out),
                               _ptr(dev_status), _stream(dev))
    _check("ttv_tree_expand", st)
    return n_out, dev_status


def tree_merge(seqs, seq_len, root_tok, Ncap: int = 128, parents=None, tokens=None, src=None,
               n_out=None, dev_status=None):
    """The union of S speculated sequences below each request's root as one
    token tree.  Returns (parents [B,Ncap], tokens [B,Ncap], src [B,Ncap],
    n_out [B], dev_status [B]); entries past n_out are as passed in (-1 when
    allocated here)."""
    B, S, Ls = seqs.shape
    dev = seqs.device
    _need(seqs, "seqs", torch.int32, (B, S, Ls), dev)
    _need(seq_len, "seq_len", torch.int32, (B, S), dev)
    _need(root_tok, "root_tok", torch.int32, (B,), dev)
    out = []
    for t, name in ((parents, "parents"), (tokens, "tokens"), (src, "src")):
        if t is None:
            t = torch.full((B, Ncap), -1, dtype=torch.int32, device=dev)
        _need(t, name, torch.int32, (B, Ncap), dev)
        out.append(t)
    if n_out is None:
        n_out = torch.empty(B, dtype=torch.int32, device=dev)
    _need(n_out, "n_out", torch.int32, (B,), dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib().ttv_tree_merge(B, S, Ls, _ptr(seqs), _ptr(seq_len), _ptr(root_tok), Ncap,
                              _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(n_out),
                              _ptr(dev_status), _stream(dev))
    _check("ttv_tree_merge", st)
    return out[0], out[1], out[2], n_out, dev_status


def probs_from_logits(logits, temperature: float = 1.0, topk: int = 0, out=None,
                      top_p: float = 1.0):
    """Probabilities over the last axis of fp32 logits [..., V] at a
    temperature, restricted to the topk highest logits when topk > 0 and to
    the shortest prefix holding the share top_p of their mass when
    top_p < 1."""
    V = logits.shape[-1]
    R = logits.numel() // V
    dev = logits.device
    _need(logits, "logits", torch.float32, tuple(logits.shape), dev)
    if out is None:
        out = torch.empty_like(logits)
    _need(out, "out", torch.float32, tuple(logits.shape), dev)
    st = lib().ttv_probs_from_logits(R, V, float(temperature), int(topk), float(top_p),
                                     _ptr(logits), _ptr(out), _stream(dev))
    _check("ttv_probs_from_logits", st)
    return out


def kv_commit_inplace(k_cache, v_cache, cache_len_in, path, path_len, Lmax: int, N: int,
                      cache_len_out=None, committed_src=None, want_src: bool = True,
                      dev_status=None):
    """Keep the accepted path of a tree stored in the cache (node i at row
    L + i), compacting its rows to L, L+1, .. in place.  Returns
    (cache_len_out [B], committed_src [B,N] or None, dev_status [B])."""
    B, Hkv, Lcap, D = k_cache.shape
    dev = k_cache.device
    dt = k_cache.dtype
    _need(k_cache, "k_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(v_cache, "v_cache", dt, (B, Hkv, Lcap, D), dev)
    _need(cache_len_in, "cache_len_in", torch.int32, (B,), dev)
    _need(path, "path", torch.int32, (B, N), dev)
    _need(path_len, "path_len", torch.int32, (B,), dev)
    if cache_len_out is None:
        cache_len_out = torch.empty(B, dtype=torch.int32, device=dev)
    _need(cache_len_out, "cache_len_out", torch.int32, (B,), dev)
    if committed_src is None and want_src:
        committed_src = torch.empty((B, N), dtype=torch.int32, device=dev)
    if dev_status is None:
        dev_status = torch.empty(B, dtype=torch.int32, device=dev)
    st = lib().ttv_kv_commit_inplace(_dt(dt), B, N, Hkv, D, Lcap, _ptr(k_cache), _ptr(v_cache),
                                     _ptr(cache_len_in), _ptr(cache_len_out), int(Lmax),
                                     _ptr(path), _ptr(path_len), _ptr(committed_src),
                                     _ptr(dev_status), _stream(dev))
    _check("ttv_kv_commit_inplace", st)
    return cache_len_out, committed_src, dev_status
