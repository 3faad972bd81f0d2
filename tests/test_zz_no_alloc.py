"""ttv_tree_attn_noalloc (the split partials in the library's static device
array instead of a caller's workspace) against ttv_tree_attn /
ttv_tree_attn_tuned with a workspace: bit-identical outputs, lse and statuses
on consecutive calls -- a split workload, then a smaller one (the array then
holds the first call's partials), then the first again -- and within the
attention tolerance of the fp64 oracle on sampled rows."""
import numpy as np
import pytest
import torch

import synth
import token_tree_verification_attn_amd as ttv
from gpu_case import ATTN_TOL, announce, sample_rows, to_dev
import oracle

pytestmark = pytest.mark.gpu


def small_spec(**kw):
    base = dict(name="na", B=3, N=48, Hq=16, Hkv=4, D=128, L=(100, 900), dtype="bf16", V=64,
                mode="greedy", tree="random", seed=4243)
    base.update(kw)
    return synth.Spec(**base)


def bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x


def compare(d, rows_per_block=0, chunk_keys=0):
    t = to_dev(d)
    B, N, Hq, D = t["q"].shape
    args = (t["q"], t["k_cache"], t["v_cache"], t["cache_len"], t["k_tree"], t["v_tree"],
            t["parents"], d["Lmax"])
    hints = dict(rows_per_block=rows_per_block, chunk_keys=chunk_keys)
    assert ttv.tree_attn_workspace_size(t["q"].dtype, B, N, Hq, d["Hkv"], D, d["Lmax"],
                                        **hints) > 0, "the case must use the scratch"
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device="cuda")
    out, lse, st = ttv.tree_attn_noalloc(*args, scale=d["scale"], lse=lse, **hints)
    ref_out, ref_lse, ref_st = ttv.tree_attn(*args, scale=d["scale"], **hints)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(ref_out))
    assert torch.equal(lse, ref_lse) and torch.equal(st, ref_st)
    rows = sample_rows(d, 64, seed=3)
    r_out, r_lse, _ = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                            d["k_tree"], d["v_tree"], d["parents"], d["scale"],
                                            rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    atol, rtol = ATTN_TOL[d["dtype"]]
    np.testing.assert_allclose(got, r_out, atol=atol, rtol=rtol)
    return st


def test_noalloc_matches_workspace_entry_point():
    big = synth.make("c3")
    small = synth.make(small_spec())
    announce("attn noalloc: c3 (split planned on the device)")
    assert (compare(big).cpu().numpy() == 0).all()
    announce("attn noalloc: smaller batch, 128-key chunks")
    assert (compare(small, chunk_keys=128).cpu().numpy() == 0).all()
    announce("attn noalloc: smaller batch, automatic shape")
    compare(small)
    announce("attn noalloc: c3 again")
    compare(big)


def test_noalloc_fp32_and_rejected_requests():
    """The FMA path (fp32) with a forced split, and requests the kernels
    reject (a malformed tree, a prefix past the promise)."""
    announce("attn noalloc: fp32 split + rejected requests")
    d = synth.make(small_spec(dtype="f32", B=4, N=20, Hq=8, Hkv=2, L=(50, 400)))
    d["parents"] = d["parents"].copy()
    d["parents"][1, 7] = 9
    st = compare(d, chunk_keys=64)
    assert st.cpu().numpy().tolist() == [0, ttv.E_TREE, 0, 0]
