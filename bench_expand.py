"""Throughput of token-tree construction on one GPU: one level of
expansion-based construction (ttv_tree_expand, the default), or merge-based
construction (ttv_tree_merge, --op merge), probabilities from logits
(ttv_probs_from_logits, --op probs), stochastic verification fed with
logits (ttv_tree_verify_logits, --op verify_logits), or stochastic
verification of stored probabilities at any vocabulary size
(ttv_tree_verify, --op verify).

    python bench_expand.py [--steps K] [--warmup W] [--B 16] [--F 16] [--V 32000] [--k 4]
    python bench_expand.py --op merge [--B 4] [--S 4] [--Ls 16]
    python bench_expand.py --op probs [--B 16] [--F 64] [--V 32000] [--k 0] [--T 0.8] [--top-p 1]
    python bench_expand.py --op verify_logits [--k 0] [--T 0.8] [--top-p 1]
    python bench_expand.py --op verify [--V 32000]

Workload: B requests, each expanding F frontier nodes by the k most probable
tokens of their speculator rows of V fp32 probabilities (softmax of N(0,2)
logits at temperature 0.8, the stochastic workload's recipe).  Inputs are
resident in HBM and rotated over enough copies to exceed twice the 256 MB
MALL; exactly --steps calls are timed, each launched directly between two
HIP events on the launch stream.  One JSON line: value = frontier rows
expanded per second at the median call time; roofline = the rows' bytes
(B*F*V*4, each read once) per call over the call's average duration, against
the 8 TB/s HBM peak; cpu_baseline = the oracle on a bounded sample of the
same rows.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (timing and graph helpers)
import token_tree_verification_attn_amd as ttv  # noqa: E402

HBM_PEAK_GBS = 8000.0


def make_probs(B, F, V, seed=1005):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 11]))
    z = rng.normal(0.0, 2.0, (B, F, V)) / 0.8
    e = np.exp(z - z.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def cpu_baseline(probs, k, budget_s):
    """The oracle on whole requests until the budget is spent; rows/s."""
    import oracle
    B, F, V = probs.shape
    frontier = np.arange(F, dtype=np.int32)[None, :]
    par = np.full((1, 128), -1, np.int32)
    tok = np.zeros((1, 128), np.int32)
    n_in = np.array([F], np.int32)
    rows, t0 = 0, time.perf_counter()
    b = 0
    while True:
        oracle.tree_expand(probs[b:b + 1], frontier, n_in, k, par, tok)
        rows += F
        b = (b + 1) % B
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": rows / el, "unit": "frontier rows/s", "cores": 1, "kind": "oracle",
            "sample": "%d rows (%d requests of %d rows, V=%d, k=%d) in %.1f s of CPU work"
                      % (rows, rows // F, F, V, k, el)}


def time_calls(call, ncopies, steps, dev, stream):
    """Exactly `steps` calls call(i), i = 0..steps-1 (input copy i % ncopies),
    launched directly and timed one by one with HIP events on the launch
    stream (bench.timed_steps).  Returns (median ms, mean ms, launch kind)."""
    fns = [lambda i=i: call(i) for i in range(ncopies)]
    # ~40 ms of untimed calls ahead of the timed ones (see bench.timed_steps)
    t0 = time.perf_counter()
    call(0)
    torch.cuda.synchronize()
    preroll = int(min(4096, max(4, math.ceil(0.040 / max(time.perf_counter() - t0, 1e-6)))))
    t = bench.summary(bench.timed_steps(fns, steps, stream, preroll))
    return t["median"], t["mean"], "direct kernel launches"


def bench_merge(args):
    """Merge of S speculated sequences of Ls tokens per request (each repeats
    the first 0..3 tokens of the one before, vocabulary 32000): latency per
    call (the tree is built by one wavefront per request)."""
    B, S, Ls = args.B, args.S, args.Ls
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(np.random.SeedSequence([1004, 12]))
    seqs = rng.integers(0, 32000, (B, S, Ls)).astype(np.int32)
    for b in range(B):
        for s in range(1, S):
            d = int(rng.integers(0, 4))
            seqs[b, s, :d] = seqs[b, s - 1, :d]
    t_seqs = torch.from_numpy(seqs).to(dev)
    t_len = torch.full((B, S), Ls, dtype=torch.int32, device=dev)
    t_root = torch.zeros(B, dtype=torch.int32, device=dev)
    outs = [torch.full((B, 128), -1, dtype=torch.int32, device=dev) for _ in range(3)]
    n_out = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)

    def call(i):
        ttv.tree_merge(t_seqs, t_len, t_root, 128, *outs, n_out=n_out, dev_status=st)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    ms, ms_mean, launch = time_calls(call, 1, args.steps, dev, stream)
    assert int(st.abs().sum()) == 0
    print(json.dumps({
        "metric": "tree_merge trees/s", "value": B / (ms * 1e-3), "unit": "trees/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_mean": ms_mean, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "merge", "B": B, "S": S, "Ls": Ls,
                   "nodes": n_out.cpu().tolist(), "launch": launch},
        "roofline": None}), flush=True)


def bench_probs(args):
    """Probabilities from logits for B*F rows of V logits (N(0,2), the
    stochastic workload's recipe) at temperature T, top-k k (0: all tokens),
    top-p (1: off);
    each row read once and written once: 8V bytes per row."""
    B, F, V = args.B, args.F, args.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rng = np.random.default_rng(np.random.SeedSequence([1005, 13]))
    z = torch.from_numpy(rng.normal(0.0, 2.0, (B * F, V)).astype(np.float32)).to(dev)
    per_copy = 2 * z.numel() * 4
    ncopies = max(1, min(64, -(-2 * bench.MALL_BYTES // per_copy)))
    ins = [z] + [z.clone() for _ in range(ncopies - 1)]
    outs = [torch.empty_like(z) for _ in range(ncopies)]

    def call(i):
        ttv.probs_from_logits(ins[i % ncopies], args.T, args.k, out=outs[i % ncopies],
                              top_p=args.top_p)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    ms, ms_mean, launch = time_calls(call, ncopies, args.steps, dev, stream)
    nbytes = B * F * V * 8
    gbs = nbytes / (ms_mean * 1e-3) / 1e9
    print(json.dumps({
        "metric": "probs_from_logits rows/s", "value": B * F / (ms * 1e-3), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_mean": ms_mean,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "probs", "rows": B * F, "V": V, "T": args.T, "topk": args.k,
                   "top_p": args.top_p,
                   "input_copies": ncopies, "launch": launch,
                   "inputs": "rotated, HBM-resident"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "probs_kernel",
                     "per_launch_algorithmic": nbytes, "avg_launch_us": ms_mean * 1e3}}),
          flush=True)


def bench_verify_logits(args):
    """Multi-step speculative sampling from raw logits on the stochastic
    workload's trees (16 requests x 64 nodes, V = 32000; LLM and speculator
    logits N(0,2), temperature T; each node's token drawn from its
    speculator distribution): ttv_tree_verify_logits (one statistics pass
    per tensor, then the walk) against the unfused route, probabilities of
    both tensors written by ttv_probs_from_logits and then ttv_tree_verify.
    Both routes give the same paths (checked)."""
    import synth
    spec = synth.WORKLOADS["c5"]
    B, N, V = spec.B, spec.N, spec.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tree = synth.make(spec, with_kv=False, with_verify=False)
    rng = np.random.default_rng(np.random.SeedSequence([spec.seed, 14]))
    z_llm = rng.normal(0.0, 2.0, (B, N, V)).astype(np.float32)
    z_ssm = rng.normal(0.0, 2.0, (B, N, V)).astype(np.float32)
    q = np.exp((z_ssm - z_ssm.max(-1, keepdims=True)).astype(np.float64) / args.T)
    cdf = np.cumsum(q, -1)
    u = rng.random((B, N, 1)) * cdf[..., -1:]
    tokens = np.minimum((cdf < u).sum(-1), V - 1).astype(np.int32)
    tokens[:, 0] = 0
    parents = torch.from_numpy(tree["parents"]).to(dev)
    tok = torch.from_numpy(tokens).to(dev)
    per_copy = 2 * z_llm.nbytes
    ncopies = max(1, min(64, -(-2 * bench.MALL_BYTES // per_copy)))
    zl = [torch.from_numpy(z_llm).to(dev)]
    zs = [torch.from_numpy(z_ssm).to(dev)]
    for _ in range(ncopies - 1):
        zl.append(zl[0].clone())
        zs.append(zs[0].clone())
    pl = [torch.empty_like(zl[0]) for _ in range(ncopies)]
    ps = [torch.empty_like(zs[0]) for _ in range(ncopies)]
    outs = [ttv._verify_outputs(B, N, dev, None, None, None, None) for _ in range(2)]
    ws = torch.empty(ttv.lib().ttv_tree_verify_logits_workspace_size(B, N, V), dtype=torch.uint8,
                     device=dev)
    nv = ttv.tree_verify_workspace_size(ttv.STOCHASTIC, B, N, V)
    wsv = torch.empty(nv, dtype=torch.uint8, device=dev) if nv else None
    seed = spec.seed

    def fused(i):
        c = i % ncopies
        path, plen, otok, st = outs[0]
        ttv.tree_verify_logits(parents, tok, zl[c], zs[c], args.T, args.k, args.top_p, seed, 0,
                               path=path, path_len=plen, out_tokens=otok, dev_status=st,
                               workspace=ws)

    def two_pass(i):
        c = i % ncopies
        ttv.probs_from_logits(zl[c], args.T, args.k, out=pl[c], top_p=args.top_p)
        ttv.probs_from_logits(zs[c], args.T, args.k, out=ps[c], top_p=args.top_p)
        path, plen, otok, st = outs[1]
        ttv.tree_verify(ttv.STOCHASTIC, parents, tok, pl[c], ps[c], seed, 0, path=path,
                        path_len=plen, out_tokens=otok, dev_status=st, workspace=wsv)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        fused(i)
        two_pass(i)
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b), "the fused and the two-pass routes disagree"
    assert int(outs[0][3].abs().sum()) == 0
    ms_f, mean_f, launch = time_calls(fused, ncopies, args.steps, dev, stream)
    ms_t, mean_t, _ = time_calls(two_pass, ncopies, args.steps, dev, stream)
    nbytes = 2 * B * N * V * 4  # both logit tensors read once
    gbs = nbytes / (mean_f * 1e-3) / 1e9
    print(json.dumps({
        "metric": "tree_verify_logits trees/s", "value": B / (ms_f * 1e-3), "unit": "trees/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_f,
        "ms_per_step_mean": mean_f, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "verify_logits", "B": B, "N": N, "V": V, "T": args.T,
                   "topk": args.k, "top_p": args.top_p, "input_copies": ncopies,
                   "launch": launch, "inputs": "rotated, HBM-resident",
                   "path_len_mean": float(outs[0][1].float().mean())},
        "two_pass_ms_per_step": ms_t, "two_pass_ms_per_step_mean": mean_t,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "ttv_tree_verify_logits (statistics passes + walk)",
                     "per_launch_algorithmic": nbytes, "avg_launch_us": mean_f * 1e3}}),
          flush=True)


def bench_verify(args):
    """Multi-step speculative sampling (ttv_tree_verify, stochastic) on the
    stochastic workload's trees and probability rows (16 requests x 64 nodes,
    softmax of N(0,2) logits at temperature 0.8, each node's token drawn from
    its speculator row) at vocabulary size --V; past 36864 entries the
    residual lives in the workspace.  Checked against the oracle on the first
    request."""
    import dataclasses
    import oracle
    import synth
    spec = dataclasses.replace(synth.WORKLOADS["c5"], V=args.V)
    B, N, V = spec.B, spec.N, spec.V
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = synth.make(spec, with_kv=False)
    per_copy = 2 * d["llm"].nbytes
    ncopies = max(1, min(16, -(-2 * bench.MALL_BYTES // per_copy)))
    parents = torch.from_numpy(d["parents"]).to(dev)
    tok = torch.from_numpy(d["tokens"]).to(dev)
    pl = [torch.from_numpy(d["llm"]).to(dev)]
    ps = [torch.from_numpy(d["ssm"]).to(dev)]
    for _ in range(ncopies - 1):
        pl.append(pl[0].clone())
        ps.append(ps[0].clone())
    path, plen, otok, st = ttv._verify_outputs(B, N, dev, None, None, None, None)
    nv = ttv.tree_verify_workspace_size(ttv.STOCHASTIC, B, N, V)
    ws = torch.empty(nv, dtype=torch.uint8, device=dev) if nv else None

    def call(i):
        c = i % ncopies
        ttv.tree_verify(ttv.STOCHASTIC, parents, tok, pl[c], ps[c], d["seed"], 0, path=path,
                        path_len=plen, out_tokens=otok, dev_status=st, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    ref = oracle.verify_mss_seeded(d["parents"][:1], d["tokens"][:1], d["llm"][:1],
                                   d["ssm"][:1], d["seed"], 0)
    for g, r in zip((path, plen, otok, st), ref):
        assert np.array_equal(g[:1].cpu().numpy(), r), "differs from the oracle"
    ms, mean, launch = time_calls(call, ncopies, args.steps, dev, stream)
    print(json.dumps({
        "metric": "tree_verify stochastic trees/s", "value": B / (ms * 1e-3), "unit": "trees/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_mean": mean, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "verify", "B": B, "N": N, "V": V, "input_copies": ncopies,
                   "launch": launch, "inputs": "rotated, HBM-resident",
                   "residual": "workspace" if nv else "LDS",
                   "path_len_mean": float(plen.float().mean())}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--op", choices=["expand", "merge", "probs", "verify_logits", "verify"],
                    default="expand")
    ap.add_argument("--T", type=float, default=0.8)
    ap.add_argument("--S", type=int, default=4)
    ap.add_argument("--Ls", type=int, default=16)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--B", type=int, default=16)
    ap.add_argument("--F", type=int, default=None,
                    help="frontier rows per request (expand: 16) or rows per request (probs: 64)")
    ap.add_argument("--V", type=int, default=32000)
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--top-p", type=float, default=1.0)
    ap.add_argument("--cpu-budget", type=float, default=3.0)
    args = ap.parse_args()
    if args.F is None:
        args.F = 64 if args.op == "probs" else 16
    if args.op == "merge":
        return bench_merge(args)
    if args.op == "probs":
        return bench_probs(args)
    if args.op == "verify":
        return bench_verify(args)
    if args.op == "verify_logits":
        if args.k == 4 and "--k" not in sys.argv:
            args.k = 0
        return bench_verify_logits(args)
    B, F, V, k = args.B, args.F, args.V, args.k
    assert F + F * k <= 128, "the expanded tree must fit 128 nodes"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probs = make_probs(B, F, V)
    per_copy = probs.nbytes
    ncopies = max(1, min(64, -(-2 * bench.MALL_BYTES // per_copy)))
    pt = torch.from_numpy(probs).to(dev)
    copies = [pt] + [pt.clone() for _ in range(ncopies - 1)]
    frontier = torch.arange(F, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
    n_in = torch.full((B,), F, dtype=torch.int32, device=dev)
    parents = torch.full((B, 128), -1, dtype=torch.int32, device=dev)
    tokens = torch.zeros((B, 128), dtype=torch.int32, device=dev)
    src = torch.full((B, 128), -1, dtype=torch.int32, device=dev)
    n_out = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)

    def call(i):
        ttv.tree_expand(copies[i % ncopies], frontier, n_in, k, parents, tokens, src_row=src,
                        n_out=n_out, dev_status=st)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    steps = args.steps
    ms, ms_mean, launch = time_calls(call, ncopies, steps, dev, stream)
    assert int(st.abs().sum()) == 0 and int((n_out != F + F * k).sum()) == 0
    rows = B * F
    gbs = rows * V * 4 / (ms_mean * 1e-3) / 1e9
    res = {
        "metric": "tree_expand frontier rows/s (one expansion level)", "value": rows / (ms * 1e-3),
        "unit": "frontier rows/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": ms, "ms_per_step_mean": ms_mean, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "expand", "B": B, "F": F, "V": V, "k": k,
                   "input_copies": ncopies, "launch": launch, "inputs": "rotated, HBM-resident"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "tree_expand_kernel", "per_launch_algorithmic": rows * V * 4,
                     "avg_launch_us": ms_mean * 1e3},
    }
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(probs, k, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
