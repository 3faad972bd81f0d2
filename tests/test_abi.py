"""The C-ABI library loads without a GPU, exports every function include/ttv.h
declares, and rejects bad arguments on the host before any HIP call (so each
error status below is produced here, on a machine with no GPU).  Fake device
pointers are used only in calls that must fail validation."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import token_tree_verification_attn_amd as ttv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttv.h")
A = 0x10000          # a 16-byte aligned fake pointer (never dereferenced)
MIS = 0x10008        # a misaligned fake pointer
SZ_ERR = ctypes.c_size_t(-1).value


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(ttv_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ttv_tree_topology", "ttv_tree_attn", "ttv_tree_attn_workspace_size",
              "ttv_tree_attn_tuned", "ttv_tree_attn_tuned_workspace_size",
              "ttv_tree_verify", "ttv_tree_verify_workspace_size", "ttv_tree_verify_uniforms",
              "ttv_kv_commit",
              "ttv_tree_expand", "ttv_tree_merge", "ttv_probs_from_logits", "ttv_kv_commit_inplace", "ttv_tree_verify_commit", "ttv_status_string",
              "ttv_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ttv.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ttv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\S+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    # the C ABI is the only exported interface of the library
    assert all(n.startswith("ttv_") for n in exported), sorted(exported)


def test_library_links_no_torch():
    out = subprocess.run(["ldd", ttv.LIB_PATH], capture_output=True, text=True).stdout
    assert "torch" not in out and "python" not in out


def test_status_strings():
    for s in range(10):
        assert ttv.status_string(s) != "unknown status"
    assert ttv.status_string(99) == "unknown status"


def attn(**kw):
    """ttv_tree_attn_tuned with these arguments; with the launch shape left
    automatic the same call through ttv_tree_attn must give the same status."""
    args = dict(dt=1, B=1, N=8, Hq=4, Hkv=2, D=64, scale=0.125, q=A, kc=A, vc=A, Lcap=128,
                cl=A, Lmax=100, kt=A, vt=A, par=A, out=A, lse=None, anc=None, depth=None,
                st=None, ws=A, wsb=1 << 30, rpb=0, ck=0)
    args.update(kw)
    v = list(args.values())
    st = ttv.lib().ttv_tree_attn_tuned(*v, None)
    if args["rpb"] == 0 and args["ck"] == 0:
        assert ttv.lib().ttv_tree_attn(*v[:-2], None) == st
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), ttv.E_DTYPE),
    (dict(q=None), ttv.E_NULL), (dict(kc=None), ttv.E_NULL), (dict(par=None), ttv.E_NULL),
    (dict(out=None), ttv.E_NULL), (dict(cl=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(N=0), ttv.E_SHAPE), (dict(Lmax=129), ttv.E_SHAPE),
    (dict(Lmax=-1), ttv.E_SHAPE), (dict(scale=float("nan")), ttv.E_SHAPE),
    (dict(scale=0.0), ttv.E_SHAPE), (dict(scale=-0.125), ttv.E_SHAPE),
    (dict(N=129), ttv.E_UNSUPPORTED), (dict(D=96), ttv.E_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), ttv.E_UNSUPPORTED), (dict(rpb=96), ttv.E_UNSUPPORTED),
    (dict(ck=100), ttv.E_UNSUPPORTED), (dict(dt=0, rpb=64), ttv.E_UNSUPPORTED),
    (dict(q=MIS), ttv.E_ALIGN), (dict(vt=MIS), ttv.E_ALIGN), (dict(out=MIS), ttv.E_ALIGN),
    (dict(ws=None, ck=64), ttv.E_WORKSPACE), (dict(wsb=16, ck=64), ttv.E_WORKSPACE),
    (dict(kt=None), ttv.E_NULL), (dict(vt=None), ttv.E_NULL),
    (dict(kt=None, vt=None, Lmax=125), ttv.E_SHAPE),   # tree in the cache: Lmax + N > Lcap
])
def test_tree_attn_host_validation(kw, status):
    assert attn(**kw) == status


def test_tree_attn_workspace_size_matches_plan():
    f = ttv.lib().ttv_tree_attn_tuned_workspace_size
    # 2 chunks of 64 keys -> per (pair, chunk, row): the partial output (D bf16
    # values for bf16, D fp32 sums for fp32) and its (max, sum) in fp32
    assert f(1, 1, 8, 4, 2, 64, 100, 0, 64) == 1 * 2 * 2 * 16 * (64 * 2 + 8)
    assert f(0, 1, 8, 4, 2, 64, 100, 0, 64) == 1 * 2 * 2 * 16 * (64 * 4 + 8)
    assert f(1, 1, 8, 4, 2, 64, 64, 0, 64) == 0                          # one chunk
    assert f(1, 1, 129, 4, 2, 64, 64, 0, 0) == SZ_ERR
    assert f(9, 1, 8, 4, 2, 64, 64, 0, 0) == SZ_ERR
    # the binding allocates exactly that much
    assert ttv.tree_attn_workspace_size(torch.bfloat16, 1, 8, 4, 2, 64, 100, 0, 64) == 8704
    # the automatic shape: no split up to 256 keys, one shape for both entry points
    g = ttv.lib().ttv_tree_attn_workspace_size
    assert g(1, 1, 8, 4, 2, 64, 100) == 0 == f(1, 1, 8, 4, 2, 64, 100, 0, 0)
    assert g(1, 4, 128, 64, 8, 128, 32768) == f(1, 4, 128, 64, 8, 128, 32768, 0, 0) > 0
    # one request of 32 kv heads x 64 rows x 512 keys: four 128-key chunks
    assert g(1, 1, 64, 32, 32, 128, 512) == 32 * 4 * 64 * (128 * 2 + 8)
    assert g(1, 1, 64, 32, 32, 128, 256) == 0
    assert g(1, 1, 129, 4, 2, 64, 64) == SZ_ERR


def verify(**kw):
    args = dict(mode=0, B=2, N=8, V=100, par=A, tok=A, llm=A, ssm=None, seed=1, step=2**63,
                path=A, plen=A, outt=A, st=None, ws=A, wsb=1 << 30)
    args.update(kw)
    return ttv.lib().ttv_tree_verify(*args.values(), None)


@pytest.mark.parametrize("kw,status", [
    (dict(mode=2), ttv.E_DTYPE),
    (dict(par=None), ttv.E_NULL), (dict(llm=None), ttv.E_NULL), (dict(path=None), ttv.E_NULL),
    (dict(mode=1), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(V=0), ttv.E_SHAPE),
    (dict(N=200), ttv.E_UNSUPPORTED),
    (dict(mode=1, ssm=A, V=40001), ttv.E_UNSUPPORTED),   # residual in memory: V % 4 == 0
    (dict(mode=1, ssm=A, V=(1 << 18) + 4), ttv.E_UNSUPPORTED),
    (dict(mode=1, ssm=A, V=40000, ws=None), ttv.E_WORKSPACE),
    (dict(mode=1, ssm=A, V=40000, wsb=2 * 40000 * 4 - 4), ttv.E_WORKSPACE),
    (dict(mode=1, ssm=A, V=40000, ws=MIS), ttv.E_ALIGN),
    (dict(llm=MIS), ttv.E_ALIGN), (dict(mode=1, ssm=MIS), ttv.E_ALIGN),
    (dict(ws=None), ttv.E_WORKSPACE), (dict(wsb=8), ttv.E_WORKSPACE),
])
def test_tree_verify_host_validation(kw, status):
    assert verify(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(par=None), ttv.E_NULL), (dict(ssm=None), ttv.E_NULL), (dict(ua=None), ttv.E_NULL),
    (dict(ub=None), ttv.E_NULL), (dict(outt=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(N=0), ttv.E_SHAPE), (dict(V=0), ttv.E_SHAPE),
    (dict(N=129), ttv.E_UNSUPPORTED), (dict(V=40000), ttv.E_UNSUPPORTED),
    (dict(llm=MIS), ttv.E_ALIGN), (dict(ssm=MIS), ttv.E_ALIGN),
])
def test_tree_verify_uniforms_host_validation(kw, status):
    args = dict(B=2, N=8, V=100, par=A, tok=A, llm=A, ssm=A, ua=A, ub=A, path=A, plen=A,
                outt=A, st=None)
    args.update(kw)
    assert ttv.lib().ttv_tree_verify_uniforms(*args.values(), None) == status


def test_tree_verify_workspace_size():
    f = ttv.lib().ttv_tree_verify_workspace_size
    assert f(1, 4, 64, 32000) == 0           # stochastic: the residual on chip
    assert f(1, 4, 64, 36864) == 0
    assert f(1, 4, 64, 40000) == 4 * 40000 * 4          # beyond it: B*V floats
    assert f(1, 3, 64, 1 << 18) == 3 * (1 << 18) * 4
    assert f(1, 4, 64, 40001) == SZ_ERR      # V % 4 != 0
    assert f(1, 4, 64, (1 << 18) + 4) == SZ_ERR
    assert f(0, 1, 64, 32000) > 0
    assert f(0, 1, 200, 32000) == SZ_ERR
    assert f(5, 1, 8, 32) == SZ_ERR


def commit(**kw):
    args = dict(dt=1, B=2, N=8, Hkv=2, D=64, Lcap=100, kt=A, vt=A, kc=A, vc=A, cli=A, clo=A,
                Lmax=50, path=A, plen=A, src=None, st=None)
    args.update(kw)
    return ttv.lib().ttv_kv_commit(*args.values(), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), ttv.E_DTYPE),
    (dict(kt=None), ttv.E_NULL), (dict(clo=None), ttv.E_NULL), (dict(plen=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(Lmax=93), ttv.E_SHAPE), (dict(Lcap=-1), ttv.E_SHAPE),
    (dict(N=129, Lcap=1000), ttv.E_UNSUPPORTED), (dict(D=32), ttv.E_UNSUPPORTED),
    (dict(kc=MIS), ttv.E_ALIGN),
])
def test_kv_commit_host_validation(kw, status):
    assert commit(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(par=None), ttv.E_NULL), (dict(B=0), ttv.E_SHAPE), (dict(N=129), ttv.E_UNSUPPORTED),
])
def test_tree_topology_host_validation(kw, status):
    args = dict(B=1, N=8, par=A, anc=None, depth=None, st=None)
    args.update(kw)
    assert ttv.lib().ttv_tree_topology(*args.values(), None) == status


def test_binding_checks_tensors_before_calling():
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        ttv.tree_attn(q, torch.zeros(1, 1, 8, 64), torch.zeros(1, 1, 8, 64),
                      torch.zeros(1, dtype=torch.int32), torch.zeros(1, 1, 4, 64),
                      torch.zeros(1, 1, 5, 64), torch.zeros(1, 4, dtype=torch.int32), Lmax=4)
    with pytest.raises(TypeError):
        ttv.tree_verify(ttv.GREEDY, torch.zeros(1, 4, dtype=torch.int64),
                        torch.zeros(1, 4, dtype=torch.int32), torch.zeros(1, 4, 10))


@pytest.mark.parametrize("kw,status", [
    (dict(probs=None), ttv.E_NULL), (dict(fr=None), ttv.E_NULL), (dict(nout=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(F=0), ttv.E_SHAPE), (dict(k=0), ttv.E_SHAPE),
    (dict(V=4, k=5), ttv.E_SHAPE), (dict(Ncap=0), ttv.E_SHAPE),
    (dict(k=17), ttv.E_UNSUPPORTED), (dict(F=129), ttv.E_UNSUPPORTED),
    (dict(Ncap=129), ttv.E_UNSUPPORTED),
])
def test_tree_expand_host_validation(kw, status):
    args = dict(B=2, F=4, V=100, k=3, probs=A, fr=A, nin=A, Ncap=64, par=A, tok=A, src=None,
                nout=A, st=None)
    args.update(kw)
    assert ttv.lib().ttv_tree_expand(*args.values(), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(seqs=None), ttv.E_NULL), (dict(ln=None), ttv.E_NULL), (dict(root=None), ttv.E_NULL),
    (dict(par=None), ttv.E_NULL), (dict(B=0), ttv.E_SHAPE), (dict(S=0), ttv.E_SHAPE),
    (dict(Ls=0), ttv.E_SHAPE), (dict(Ncap=0), ttv.E_SHAPE),
    (dict(S=65), ttv.E_UNSUPPORTED), (dict(Ls=129), ttv.E_UNSUPPORTED),
    (dict(Ncap=129), ttv.E_UNSUPPORTED),
])
def test_tree_merge_host_validation(kw, status):
    args = dict(B=2, S=4, Ls=16, seqs=A, ln=A, root=A, Ncap=64, par=A, tok=A, src=None, nout=A,
                st=None)
    args.update(kw)
    assert ttv.lib().ttv_tree_merge(*args.values(), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), ttv.E_NULL), (dict(p=None), ttv.E_NULL), (dict(R=0), ttv.E_SHAPE),
    (dict(V=0), ttv.E_SHAPE), (dict(T=0.0), ttv.E_SHAPE), (dict(T=float("inf")), ttv.E_SHAPE),
    (dict(T=float("nan")), ttv.E_SHAPE), (dict(k=-1), ttv.E_SHAPE),
    (dict(k=513), ttv.E_UNSUPPORTED), (dict(top_p=0.0), ttv.E_SHAPE),
    (dict(top_p=1.5), ttv.E_SHAPE), (dict(top_p=float("nan")), ttv.E_SHAPE),
    (dict(T=1e-39), ttv.E_SHAPE),
])
def test_probs_from_logits_host_validation(kw, status):
    args = dict(R=4, V=1000, T=0.8, k=50, top_p=1.0, z=A, p=A)
    args.update(kw)
    assert ttv.lib().ttv_probs_from_logits(*args.values(), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), ttv.E_DTYPE), (dict(kc=None), ttv.E_NULL), (dict(clo=None), ttv.E_NULL),
    (dict(path=None), ttv.E_NULL), (dict(B=0), ttv.E_SHAPE), (dict(Lmax=93), ttv.E_SHAPE),
    (dict(Lcap=-1), ttv.E_SHAPE), (dict(N=129, Lcap=1000), ttv.E_UNSUPPORTED),
    (dict(D=32), ttv.E_UNSUPPORTED), (dict(kc=MIS), ttv.E_ALIGN),
])
def test_kv_commit_inplace_host_validation(kw, status):
    args = dict(dt=1, B=2, N=8, Hkv=2, D=64, Lcap=100, kc=A, vc=A, cli=A, clo=A, Lmax=50,
                path=A, plen=A, src=None, st=None)
    args.update(kw)
    assert ttv.lib().ttv_kv_commit_inplace(*args.values(), None) == status


def verify_commit(**kw):
    args = dict(mode=0, dt=1, B=2, N=8, V=64, Hkv=2, D=64, Lcap=100, par=A, tok=A, llm=A,
                ssm=None, seed=7, step=0, kt=A, vt=A, kc=A, vc=A, cli=A, clo=A + 0x100, Lmax=50,
                path=A, plen=A, outt=A, src=None, st=None, ws=A, wsb=1 << 20)
    args.update(kw)
    return ttv.lib().ttv_tree_verify_commit(*args.values(), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), ttv.E_DTYPE), (dict(par=None), ttv.E_NULL), (dict(llm=None), ttv.E_NULL),
    (dict(kc=None), ttv.E_NULL), (dict(clo=None), ttv.E_NULL), (dict(outt=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(V=0), ttv.E_SHAPE), (dict(Lmax=93), ttv.E_SHAPE),
    (dict(N=129, Lcap=1000), ttv.E_UNSUPPORTED), (dict(D=32), ttv.E_UNSUPPORTED),
    (dict(llm=MIS), ttv.E_ALIGN), (dict(kt=MIS), ttv.E_ALIGN), (dict(ws=None), ttv.E_WORKSPACE),
    (dict(wsb=64), ttv.E_WORKSPACE), (dict(ws=MIS), ttv.E_ALIGN), (dict(mode=2), ttv.E_DTYPE),
    (dict(mode=1), ttv.E_NULL),                                  # stochastic without ssm
    (dict(mode=1, ssm=A, V=40002), ttv.E_UNSUPPORTED),  # residual in memory: V % 4 == 0
    (dict(mode=1, ssm=A, V=40000, ws=None), ttv.E_WORKSPACE),
    (dict(mode=1, ssm=A, V=40000, wsb=64), ttv.E_WORKSPACE),
    (dict(mode=1, ssm=MIS), ttv.E_ALIGN),
])
def test_tree_verify_commit_host_validation(kw, status):
    assert verify_commit(**kw) == status


def test_tree_verify_commit_takes_every_commit_shape():
    """Shared length arrays and the largest rows reach the workspace check."""
    assert verify_commit(clo=A, ws=None) == ttv.E_WORKSPACE
    assert verify_commit(dt=0, D=128, N=128, Lcap=1000, ws=None) == ttv.E_WORKSPACE


def noalloc(**kw):
    args = dict(dt=1, B=1, N=8, Hq=4, Hkv=2, D=64, scale=0.125, q=A, kc=A, vc=A, Lcap=128,
                cl=A, Lmax=100, kt=A, vt=A, par=A, out=A, lse=None, anc=None, depth=None,
                st=None, rpb=0, ck=0)
    args.update(kw)
    return ttv.lib().ttv_tree_attn_noalloc(*args.values(), None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), ttv.E_DTYPE), (dict(q=None), ttv.E_NULL), (dict(kt=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(Lmax=129), ttv.E_SHAPE), (dict(scale=0.0), ttv.E_SHAPE),
    (dict(N=129), ttv.E_UNSUPPORTED), (dict(D=96), ttv.E_UNSUPPORTED), (dict(q=MIS), ttv.E_ALIGN),
    (dict(rpb=96), ttv.E_UNSUPPORTED), (dict(ck=100), ttv.E_UNSUPPORTED),
    # 4 requests x 8 kv heads x 1024 rows x 32768 keys in 128-key chunks: 4.3 GB of partials
    (dict(B=4, N=128, Hq=64, Hkv=8, D=128, Lcap=32768 + 128, Lmax=32768, ck=128),
     ttv.E_SCRATCH),
])
def test_tree_attn_noalloc_host_validation(kw, status):
    """The no-allocation entry point validates like ttv_tree_attn and refuses
    a call whose partials exceed its static scratch before any HIP call."""
    assert noalloc(**kw) == status


def test_noalloc_scratch_limit_is_the_stated_one():
    f = ttv.lib().ttv_tree_attn_tuned_workspace_size
    assert f(1, 4, 128, 64, 8, 128, 32768, 0, 128) > ttv.NOALLOC_SCRATCH_BYTES
    # the automatic shape of the long-context workload fits
    assert 0 < f(1, 4, 128, 64, 8, 128, 32768, 0, 0) <= ttv.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define TTV_NOALLOC_SCRATCH_BYTES (48u << 20)" in text
    assert ttv.NOALLOC_SCRATCH_BYTES == 48 << 20


def test_varlen_entry_points_need_node_counts():
    """The _varlen entry points validate like their fixed-size forms and
    refuse a NULL node-count array."""
    L = ttv.lib()
    attn_args = [1, 1, 8, 4, 2, 64, 0.125, A, A, A, 128, A, 100, A, A, A]
    tail = [A, None, None, None, None, A, 1 << 30, None]
    assert L.ttv_tree_attn_varlen(*attn_args, None, *tail) == ttv.E_NULL
    assert L.ttv_tree_attn_varlen(*attn_args, A, *tail[:0], MIS, *tail[1:]) == ttv.E_ALIGN
    assert L.ttv_tree_attn_varlen(1, 1, 129, 4, 2, 64, 0.125, A, A, A, 1280, A, 100, A, A, A, A,
                                  *tail) == ttv.E_UNSUPPORTED
    ver = lambda n, **kw: L.ttv_tree_verify_varlen(
        kw.get("mode", 0), 2, 8, 100, A, A, n, A, kw.get("ssm"), 1, 2, A, A, A, None, A, 1 << 30,
        None)
    assert ver(None) == ttv.E_NULL
    assert ver(A, mode=1) == ttv.E_NULL and ver(A, mode=3) == ttv.E_DTYPE
    vc = lambda n, **kw: L.ttv_tree_verify_commit_varlen(
        0, 1, 2, 8, 64, 2, 64, 100, A, A, n, A, None, 7, 0, A, A, A, A, A, A + 0x100,
        kw.get("Lmax", 50), A, A, A, None, None, A, 1 << 20, None)
    assert vc(None) == ttv.E_NULL and vc(A, Lmax=93) == ttv.E_SHAPE


@pytest.mark.parametrize("kw,status", [
    (dict(par=None), ttv.E_NULL), (dict(zl=None), ttv.E_NULL), (dict(zs=None), ttv.E_NULL),
    (dict(B=0), ttv.E_SHAPE), (dict(T=0.0), ttv.E_SHAPE), (dict(top_p=0.0), ttv.E_SHAPE),
    (dict(V=1002), ttv.E_UNSUPPORTED), (dict(V=(1 << 18) + 4), ttv.E_UNSUPPORTED),
    (dict(N=129), ttv.E_UNSUPPORTED), (dict(k=600), ttv.E_UNSUPPORTED),
    (dict(zl=MIS), ttv.E_ALIGN), (dict(ws=None), ttv.E_WORKSPACE),
    (dict(wsb=2 * 2 * 8 * 16 - 1), ttv.E_WORKSPACE),
    # past 32768 entries the residual joins the workspace (B*V floats)
    (dict(V=32772, wsb=2 * 2 * 8 * 16 + 2 * 32772 * 4 - 4), ttv.E_WORKSPACE),
    (dict(V=32772, ws=MIS), ttv.E_ALIGN),
])
def test_tree_verify_logits_host_validation(kw, status):
    args = dict(B=2, N=8, V=1000, par=A, tok=A, nn=None, zl=A, zs=A, T=0.8, k=0, top_p=0.9,
                seed=1, step=0, path=A, plen=A, outt=A, st=None, ws=A, wsb=1 << 20)
    args.update(kw)
    assert ttv.lib().ttv_tree_verify_logits(*args.values(), None) == status
    f = ttv.lib().ttv_tree_verify_logits_workspace_size
    assert f(2, 8, 1000) == 2 * 2 * 8 * 16
    assert f(2, 8, 32768) == 2 * 2 * 8 * 16
    assert f(2, 8, 32772) == 2 * 2 * 8 * 16 + 2 * 32772 * 4
    assert f(2, 8, 1 << 18) == 2 * 2 * 8 * 16 + 2 * (1 << 18) * 4
    assert f(2, 8, 1002) == SZ_ERR and f(2, 8, (1 << 18) + 4) == SZ_ERR and f(2, 129, 1000) == SZ_ERR
