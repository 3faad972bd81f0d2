"""Seeded synthetic inputs for the tree-verification step.

This module only draws inputs; it holds none of the method's arithmetic and is
shared by the tests, the benchmark and the smoke check (the GPU library and
the CPU oracle each receive the same arrays from here and import neither this
module nor each other).

Five workloads are shaped after the pages' setting (LLaMA-7B-like heads, GQA
layers, token trees built by expansion from a speculator's top-k or by merging
several speculators' sequences -- [SI] §3 "Expansion-based" / "Merge-based
token tree construction"):

    c1  1 request, 8-node random tree (depth <= 4), 1 head, D 64, fp32,
        prefix 128, vocab 32, greedy, logits N(0, 2).
    c2  1 request, 64-node expansion tree (per-depth widths 1,1,3,1,1,1,1,1
        cycled), 32/32 heads, D 128, bf16, prefix 512, vocab 32000, greedy,
        logits N(0, 3), the argmax planted on ~70% of the edges.
    c3  8 requests, 32-node random trees (depth <= 8, 1-4 children),
        32/8 heads, D 128, bf16, prefix uniform in [1024, 4096], vocab 32000,
        greedy as c2.
    c4  4 requests, 128-node merged trees (4 speculator chains of depth 16
        sharing deduplicated prefixes, plus extra top-k leaves), 64/8 heads,
        D 128, bf16, prefix 32768, vocab 32000, greedy as c2.
    c5  16 requests, 64-node random trees, 32/8 heads, D 128, bf16, prefix
        2048, vocab 32000, stochastic: llm and ssm rows are softmax(z / 0.8),
        z ~ N(0, 2) per row, each node's token drawn from its ssm row; the
        verifier's uniforms come from Philox4x64-10 with seed 1005, step 0
        (explicit uniforms -- one per node and one per request, drawn from
        numpy's Philox stream -- for the explicit-uniform call).

Every array has its own seeded stream: ``SeedSequence([seed, stream_id])``
(seed = 1000 + k for workload ck).  Q/K/V are N(0, 1), rounded to bf16 (round
to nearest even, by torch) when the dtype is bf16; arrays are returned as
float32 holding the exact values.  Prefix-cache rows at or beyond a request's
length are filled with a poison value (V = 1000) so that reading past the
prefix shows in the output.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple, Union

import numpy as np

# stream ids
S_TREE, S_TOK, S_Q, S_KP, S_VP, S_KT, S_VT, S_LLM, S_SSM, S_PLANT, S_LEN, S_UNI = range(12)
POISON_V = 1000.0


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    L: Union[int, Tuple[int, int]]   # fixed prefix, or inclusive uniform range
    dtype: str                        # "f32" | "bf16"
    V: int
    mode: str                         # "greedy" | "stochastic"
    tree: str                         # "random" | "expansion" | "merged" | "chain" | "star"
    seed: int
    dmax: int = 8                     # random trees: maximum depth
    max_children: int = 4             # random trees: maximum branching
    widths: Tuple[int, ...] = (1, 1, 3, 1, 1, 1, 1, 1)   # expansion schedule
    chains: int = 4                   # merged trees: speculator chains
    chain_len: int = 16               # merged trees: depth of each chain
    logit_sigma: float = 3.0
    plant: float = 0.7                # greedy: P(argmax planted on an edge)
    temperature: float = 0.8          # stochastic: softmax(z / T)
    prob_sigma: float = 2.0           # stochastic: z ~ N(0, sigma)


WORKLOADS = {
    "c1": Spec("c1", 1, 8, 1, 1, 64, 128, "f32", 32, "greedy", "random", 1001,
               dmax=4, max_children=8, logit_sigma=2.0, plant=0.0),
    "c2": Spec("c2", 1, 64, 32, 32, 128, 512, "bf16", 32000, "greedy", "expansion", 1002),
    "c3": Spec("c3", 8, 32, 32, 8, 128, (1024, 4096), "bf16", 32000, "greedy", "random",
               1003),
    "c4": Spec("c4", 4, 128, 64, 8, 128, 32768, "bf16", 32000, "greedy", "merged", 1004),
    "c5": Spec("c5", 16, 64, 32, 8, 128, 2048, "bf16", 32000, "stochastic", "random",
               1005),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields replaced (edge cases)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


def stream(seed: int, sid: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, sid]))


def philox_stream(seed: int, sid: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, sid])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (nearest even) and widened back."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


# --------------------------------------------------------------------------
# trees (parents arrays in a topological numbering: parent < child)
# --------------------------------------------------------------------------
def random_tree(rng, N: int, dmax: int, max_children: int) -> np.ndarray:
    """Node i's parent is uniform among earlier nodes with room to grow."""
    par = np.full(N, -1, np.int32)
    depth = np.zeros(N, np.int32)
    nchild = np.zeros(N, np.int32)
    for i in range(1, N):
        ok = np.nonzero((depth[:i] < dmax) & (nchild[:i] < max_children))[0]
        p = int(ok[rng.integers(len(ok))])
        par[i], depth[i] = p, depth[p] + 1
        nchild[p] += 1
    return par


def chain_tree(N: int) -> np.ndarray:
    return np.arange(-1, N - 1, dtype=np.int32)


def star_tree(N: int) -> np.ndarray:
    par = np.zeros(N, np.int32)
    par[0] = -1
    return par


def expansion_tree(N: int, widths: Sequence[int]) -> np.ndarray:
    """Breadth-first expansion: each node at depth d gets widths[d % len]
    children, cycling the schedule, until N nodes exist."""
    par = [-1]
    depth = [0]
    head = 0
    while len(par) < N:
        u = head
        head += 1
        for _ in range(widths[depth[u] % len(widths)]):
            if len(par) == N:
                break
            par.append(u)
            depth.append(depth[u] + 1)
    return np.asarray(par, np.int32)


def merged_tree(rng, N: int, V: int, chains: int, chain_len: int):
    """Union of `chains` speculator sequences of length chain_len (sequence s
    repeats the first d_s ~ U{0..3} tokens of sequence s-1, shared nodes
    deduplicated), then extra leaves with fresh sibling tokens attached
    round-robin, breadth first, to nodes of depth < chain_len until N nodes.
    Returns (parents, tokens)."""
    par, tok, depth = [-1], [int(rng.integers(V))], [0]
    children = {0: {}}
    seqs = []
    for s in range(chains):
        share = 0 if s == 0 else int(rng.integers(0, 4))
        seq = list(seqs[-1][:share]) if s else []
        while len(seq) < chain_len:
            seq.append(int(rng.integers(V)))
        seqs.append(seq)
        u = 0
        for t in seq:
            if t in children[u]:
                u = children[u][t]
                continue
            if len(par) == N:
                break
            par.append(u), tok.append(t), depth.append(depth[u] + 1)
            children[u][t] = len(par) - 1
            children[len(par) - 1] = {}
            u = len(par) - 1
    while len(par) < N:
        grew = False
        for u in sorted(range(len(par)), key=lambda j: (depth[j], j)):
            if len(par) == N:
                break
            if depth[u] >= chain_len:
                continue
            t = int(rng.integers(V))
            while t in children[u]:
                t = int(rng.integers(V))
            par.append(u), tok.append(t), depth.append(depth[u] + 1)
            children[u][t] = len(par) - 1
            children[len(par) - 1] = {}
            grew = True
        assert grew
    return np.asarray(par, np.int32), np.asarray(tok, np.int32)


def sibling_distinct_tokens(rng, par: np.ndarray, V: int) -> np.ndarray:
    N = len(par)
    tok = np.zeros(N, np.int32)
    tok[0] = rng.integers(V)
    used = {}
    for i in range(1, N):
        s = used.setdefault(int(par[i]), set())
        assert len(s) < V, "more siblings than vocabulary entries"
        t = int(rng.integers(V))
        while t in s:
            t = int(rng.integers(V))
        s.add(t)
        tok[i] = t
    return tok


def topk_tokens(rng, par: np.ndarray, V: int) -> np.ndarray:
    """Children of each node take the top-k entries of a N(0,1) speculator
    row drawn for that node (k = its number of children)."""
    N = len(par)
    tok = np.zeros(N, np.int32)
    tok[0] = rng.integers(V)
    for u in range(N):
        kids = np.nonzero(par == u)[0]
        if len(kids) == 0:
            continue
        row = rng.standard_normal(V, dtype=np.float32)
        top = np.argsort(-row, kind="stable")[: len(kids)]
        tok[kids] = top
    return tok


# --------------------------------------------------------------------------
# full inputs
# --------------------------------------------------------------------------
def _normal(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _softmax_rows(rng, shape, sigma, temperature):
    z = rng.standard_normal(shape) * sigma / temperature
    z -= z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def make(s: Union[str, Spec], parents: Optional[np.ndarray] = None,
         with_kv: bool = True, with_verify: bool = True) -> dict:
    """Inputs of one workload.  `parents` [B,N] overrides the tree (tokens are
    then drawn sibling-distinct).  Returns a dict of numpy arrays and sizes."""
    if isinstance(s, str):
        s = WORKLOADS[s]
    B, N, V = s.B, s.N, s.V
    out = dict(spec=s, B=B, N=N, Hq=s.Hq, Hkv=s.Hkv, D=s.D, V=V, dtype=s.dtype,
               mode=s.mode, scale=float(1.0 / np.sqrt(s.D)))

    # ---- prefix lengths
    if isinstance(s.L, tuple):
        L = stream(s.seed, S_LEN).integers(s.L[0], s.L[1] + 1, size=B).astype(np.int32)
    else:
        L = np.full(B, s.L, np.int32)
    Lmax = int(L.max())
    Lcap = (Lmax + N + 63) // 64 * 64
    out.update(cache_len=L, Lmax=Lmax, Lcap=Lcap)

    # ---- trees and tokens
    rt, rk = stream(s.seed, S_TREE), stream(s.seed, S_TOK)
    par = np.zeros((B, N), np.int32)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        if parents is not None:
            par[b] = parents[b]
            if s.mode != "stochastic":
                tok[b] = sibling_distinct_tokens(rk, par[b], V)
            continue
        if s.tree == "random":
            par[b] = random_tree(rt, N, s.dmax, s.max_children)
        elif s.tree == "expansion":
            par[b] = expansion_tree(N, s.widths)
        elif s.tree == "chain":
            par[b] = chain_tree(N)
        elif s.tree == "star":
            par[b] = star_tree(N)
        elif s.tree == "merged":
            par[b], tok[b] = merged_tree(rt, N, V, s.chains, s.chain_len)
            continue
        else:
            raise ValueError(s.tree)
        if s.mode == "stochastic":
            continue  # drawn from the ssm rows below
        tok[b] = topk_tokens(rk, par[b], V) if s.tree == "expansion" else \
            sibling_distinct_tokens(rk, par[b], V)
    out.update(parents=par, tokens=tok)

    # ---- attention inputs
    if with_kv:
        dt = s.dtype
        out["q"] = _normal(stream(s.seed, S_Q), (B, N, s.Hq, s.D), dt)
        kc = _normal(stream(s.seed, S_KP), (B, s.Hkv, Lcap, s.D), dt)
        vc = _normal(stream(s.seed, S_VP), (B, s.Hkv, Lcap, s.D), dt)
        for b in range(B):
            vc[b, :, L[b]:, :] = POISON_V
        out["k_cache"], out["v_cache"] = kc, vc
        out["k_tree"] = _normal(stream(s.seed, S_KT), (B, s.Hkv, N, s.D), dt)
        out["v_tree"] = _normal(stream(s.seed, S_VT), (B, s.Hkv, N, s.D), dt)

    # ---- verification inputs
    if with_verify:
        if s.mode == "greedy":
            llm = stream(s.seed, S_LLM).standard_normal((B, N, V), dtype=np.float32)
            llm *= np.float32(s.logit_sigma)
            rp = stream(s.seed, S_PLANT)
            for b in range(B):
                for u in range(N):
                    kids = np.nonzero(par[b] == u)[0]
                    if len(kids) == 0 or rp.random() >= s.plant:
                        continue
                    c = kids[rp.integers(len(kids))]
                    llm[b, u, tok[b, c]] = llm[b, u].max() + 1.0
            out["llm"] = llm
        else:
            llm = _softmax_rows(stream(s.seed, S_LLM), (B, N, V), s.prob_sigma,
                                s.temperature)
            ssm = _softmax_rows(stream(s.seed, S_SSM), (B, N, V), s.prob_sigma,
                                s.temperature)
            # each non-root node's token is drawn from its own ssm row
            u = stream(s.seed, S_TOK).random((B, N))
            cdf = np.cumsum(ssm.astype(np.float64), axis=-1)
            cdf /= cdf[..., -1:]
            draw = (cdf < u[..., None]).sum(axis=-1).clip(0, V - 1).astype(np.int32)
            tok = out["tokens"].copy()
            tok[:, 1:] = draw[:, 1:]
            out["tokens"] = tok
            uni = philox_stream(s.seed, S_UNI)
            out["llm"], out["ssm"] = llm, ssm
            out["u_accept"] = uni.random((B, N), dtype=np.float32)
            out["u_bonus"] = uni.random(B, dtype=np.float32)
            # the seeded verifier draws its own uniforms (Philox4x64-10, key
            # (seed, 0)); the explicit ones above serve the explicit-uniform call
            out["seed"], out["step"] = s.seed, 0
    return out
