"""Helpers of the GPU parity tests: seeded inputs to the device, the library
call, the oracle on the same host arrays, and the comparison.

Tolerances: attention outputs within atol 2e-2 / rtol 1e-2 of the fp64 oracle
for bf16 inputs (fp32 accumulation, bf16 output); fp32 inputs use 1e-4 /
1e-4.  Tree masks, paths, tokens, lengths and committed KV bytes must match
exactly."""
import numpy as np
import torch

import oracle
import synth
import token_tree_verification_attn_amd as ttv

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
ATTN_TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def announce(msg):
    print("[gpu case] " + msg, flush=True)


def to_dev(d, dev="cuda"):
    t = {}
    dt = TDT[d.get("dtype", "f32")]
    for k in ("q", "k_cache", "v_cache", "k_tree", "v_tree"):
        if k in d:
            t[k] = torch.from_numpy(d[k]).to(dev).to(dt)  # bf16-exact values
    for k in ("parents", "tokens", "cache_len", "llm", "ssm", "u_accept", "u_bonus"):
        if k in d:
            t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
    return t


def sample_rows(d, n, seed=0):
    """n random (b, i, hq) rows plus, for every request, the root and the
    deepest node of each request under every query head of group 0."""
    rng = np.random.default_rng(seed)
    B, N, Hq = d["B"], d["N"], d["Hq"]
    rows = [(int(rng.integers(B)), int(rng.integers(N)), int(rng.integers(Hq)))
            for _ in range(n)]
    depth, _, _ = oracle.topology(d["parents"])
    G = Hq // d["Hkv"]
    for b in range(B):
        deepest = int(np.argmax(depth[b]))
        for g in range(G):
            rows.append((b, 0, g))
            rows.append((b, deepest, g))
    return np.unique(np.array(rows, np.int32), axis=0)


def block_rows(d, per_block, rows_per_block, seed=0):
    """per_block random query rows from every (request, kv head, block of
    rows_per_block packed rows r = node*G + g) -- the unit one attention
    workgroup (or, with a split prefix, each of its chunks' workgroups)
    computes -- so that every workgroup of the launch has outputs compared."""
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv = d["B"], d["N"], d["Hq"], d["Hkv"]
    G = Hq // Hkv
    R = N * G
    rows = []
    for b in range(B):
        for h in range(Hkv):
            for r0 in range(0, R, rows_per_block):
                n = min(rows_per_block, R - r0)
                for r in r0 + rng.choice(n, size=min(per_block, n), replace=False):
                    rows.append((b, int(r) // G, h * G + int(r) % G))
    return np.unique(np.array(rows, np.int32), axis=0)


def run_attn(d, t, **hints):
    out, lse, st = ttv.tree_attn(t["q"], t["k_cache"], t["v_cache"], t["cache_len"],
                                 t["k_tree"], t["v_tree"], t["parents"], d["Lmax"],
                                 scale=d["scale"], **hints)
    torch.cuda.synchronize()
    return out, lse, st


def check_attn(d, t=None, rows=None, repeat=True, **hints):
    """GPU tree_attn vs the oracle on all rows (rows=None) or the given rows;
    a second identical launch must reproduce the first bit for bit."""
    t = t if t is not None else to_dev(d)
    out, lse, st = run_attn(d, t, **hints)
    if repeat:
        out2, lse2, _ = run_attn(d, t, **hints)
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                           out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2)
        assert torch.equal(lse, lse2)
    if rows is None:
        rows = oracle.all_rows(d["B"], d["N"], d["Hq"])
    ref, ref_lse, ref_st = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"],
                                                 d["cache_len"], d["k_tree"], d["v_tree"],
                                                 d["parents"], d["scale"], rows)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    got_lse = l[rows[:, 0], rows[:, 1], rows[:, 2]]
    atol, rtol = ATTN_TOL[d["dtype"]]
    np.testing.assert_allclose(got, ref, atol=atol, rtol=rtol)
    np.testing.assert_allclose(got_lse, ref_lse, atol=1e-3, rtol=1e-4)
    # per-request status agrees with the oracle's per-row status
    st = st.cpu().numpy()
    for (b, _, _), s in zip(rows, ref_st):
        assert st[b] == s, (b, st[b], s)
    return out, lse, st


def check_verify(d, t=None, uniforms=False):
    """GPU tree_verify vs the oracle, bit for bit.  Stochastic inputs are
    verified with the uniforms drawn from (seed, step) on both sides, or with
    uniforms=True with the explicit uniforms of the inputs
    (tree_verify_uniforms)."""
    t = t if t is not None else to_dev(d)
    greedy = d["mode"] == "greedy"
    if greedy:
        path, plen, outt, st = ttv.tree_verify(ttv.GREEDY, t["parents"], t["tokens"], t["llm"])
        ref = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
    elif uniforms:
        path, plen, outt, st = ttv.tree_verify_uniforms(t["parents"], t["tokens"], t["llm"],
                                                        t["ssm"], t["u_accept"], t["u_bonus"])
        ref = oracle.verify_mss(d["parents"], d["tokens"], d["llm"], d["ssm"], d["u_accept"],
                                d["u_bonus"])
    else:
        path, plen, outt, st = ttv.tree_verify(ttv.STOCHASTIC, t["parents"], t["tokens"],
                                               t["llm"], t["ssm"], seed=d["seed"],
                                               step=d["step"])
        ref = oracle.verify_mss_seeded(d["parents"], d["tokens"], d["llm"], d["ssm"],
                                       d["seed"], d["step"])
    torch.cuda.synchronize()
    for name, g, r in zip(("path", "path_len", "out_tokens", "status"),
                          (path, plen, outt, st), ref):
        g = g.cpu().numpy()
        assert np.array_equal(g, r), "%s differs:\n gpu %s\n ref %s" % (name, g, r)
    return path, plen, outt, st


def check_commit(d, t, path, plen, in_place=False):
    """kv_commit on device copies of the cache vs the oracle's byte copy; with
    in_place the new lengths overwrite the input lengths (one workgroup per
    request), else they go to their own array (one per request and kv head)."""
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    lens = t["cache_len"].clone()
    clo, src, st = ttv.kv_commit(t["k_tree"], t["v_tree"], kc, vc, lens, path, plen, d["Lmax"],
                                 cache_len_out=lens if in_place else None)
    torch.cuda.synchronize()
    view = torch.int16 if kc.dtype == torch.bfloat16 else torch.int32
    np_dt = np.int16 if kc.dtype == torch.bfloat16 else np.int32
    kt = t["k_tree"].view(view).cpu().numpy()
    vt = t["v_tree"].view(view).cpu().numpy()
    kc0 = t["k_cache"].view(view).cpu().numpy()
    vc0 = t["v_cache"].view(view).cpu().numpy()
    rk, rv, rclo, rsrc, rst = oracle.kv_commit(kt, vt, kc0, vc0, d["cache_len"],
                                               path.cpu().numpy(), plen.cpu().numpy(),
                                               d["Lmax"])
    assert np.array_equal(clo.cpu().numpy(), rclo)
    assert np.array_equal(src.cpu().numpy(), rsrc)
    assert np.array_equal(st.cpu().numpy(), np.where(rst == 0, 0, ttv.E_SHAPE))
    assert np.array_equal(kc.view(view).cpu().numpy(), rk.astype(np_dt))
    assert np.array_equal(vc.view(view).cpu().numpy(), rv.astype(np_dt))
    return clo


def make(spec_or_name, **over):
    s = synth.spec(spec_or_name, **over) if isinstance(spec_or_name, str) else spec_or_name
    return synth.make(s)
