"""GPU tree attention vs the fp64 oracle on the same seeded inputs.

The five workloads at full size in the launch configuration the benchmark
uses (every row; the long-context one on rows from every workgroup's unit),
plus edge cases: N = 1, empty prefix,
chains and stars, N = 64/65/128 (bitset word boundary), GQA group sizes 1..16,
ragged prefix lengths, the FMA path in bf16 (fewer than 16 rows per kv head)
and fp32, head dim 64, every row-block size and forced KV splits, and
rejected requests (malformed tree, prefix longer than the promise).  Batches
of 2..64 requests take the split planned on the device from the actual
lengths; explicit length mixes (empty, one key, tile boundaries, the maximum)
check that every key is covered exactly once."""
import numpy as np
import pytest
import torch

import synth
import oracle
from gpu_case import announce, block_rows, check_attn, make, run_attn, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_workload_full(name):
    announce("attn workload %s (all rows)" % name)
    check_attn(make(name))


def test_long_context_every_workgroup():
    """The long-context workload at full size, in the launch the benchmark
    times (256-row blocks, the prefix split planned on the device): 16 rows
    from every (request, kv head, row block) unit -- each of its chunk
    workgroups contributes to all of them -- plus the roots and deepest
    nodes."""
    announce("attn workload c4 (16 rows of every row block)")
    d = make("c4")
    rows = np.unique(np.concatenate([block_rows(d, 16, 256), sample_rows(d, 0)]), axis=0)
    assert len({(b, h // 8, ((i * 8 + h % 8) // 256)) for b, i, h in rows}) == 4 * 8 * 4
    check_attn(d, rows=rows)


def spec(**kw):
    base = dict(name="edge", B=2, N=16, Hq=8, Hkv=2, D=128, L=200, dtype="bf16", V=64,
                mode="greedy", tree="random", seed=4242, dmax=8, max_children=4)
    base.update(kw)
    return synth.Spec(**base)


EDGE = {
    "decode_N1_fma": dict(B=3, N=1, Hq=8, Hkv=1, L=300),
    "decode_N1_mfma_G16": dict(B=2, N=1, Hq=16, Hkv=1, L=257),
    "empty_prefix": dict(B=2, N=64, Hq=8, Hkv=2, L=0),
    "chain128_two_words": dict(B=1, N=128, Hq=4, Hkv=2, L=100, tree="chain"),
    "star65": dict(B=2, N=65, Hq=2, Hkv=2, L=70, tree="star"),
    "random64": dict(B=2, N=64, Hq=8, Hkv=8, L=129),
    "random65": dict(B=2, N=65, Hq=8, Hkv=4, L=1),
    "random128_G8": dict(B=1, N=128, Hq=16, Hkv=2, L=333, dmax=16),
    "ragged_prefix": dict(B=5, N=24, Hq=8, Hkv=2, L=(1, 700)),
    "bf16_fma_path": dict(B=3, N=3, Hq=8, Hkv=2, L=(5, 90)),
    "fp32_D128_multi_rowblock": dict(B=2, N=20, Hq=4, Hkv=2, L=150, dtype="f32"),
    "fp32_D64": dict(B=1, N=9, Hq=2, Hkv=1, D=64, L=77, dtype="f32"),
    "bf16_D64_mfma": dict(B=2, N=32, Hq=8, Hkv=2, D=64, L=300),
    "G1_mha": dict(B=1, N=40, Hq=4, Hkv=4, L=64),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    announce("attn edge %s" % case)
    check_attn(synth.make(spec(**EDGE[case])))


@pytest.mark.parametrize("rpb,ck", [(64, 0), (128, 0), (256, 0), (64, 64), (128, 128),
                                    (256, 64), (128, 192), (64, 1024)])
def test_launch_shapes(rpb, ck):
    announce("attn rows_per_block=%d chunk_keys=%d" % (rpb, ck))
    d = synth.make(spec(B=3, N=48, Hq=16, Hkv=4, L=(100, 900)))
    check_attn(d, rows_per_block=rpb, chunk_keys=ck)


@pytest.mark.parametrize("ck", [0, 64])
def test_rejected_requests(ck):
    announce("attn rejected requests chunk_keys=%d" % ck)
    d = synth.make(spec(B=4, N=20, Hq=8, Hkv=2, L=(50, 300)))
    d["parents"] = d["parents"].copy()
    d["parents"][1, 7] = 9                      # forward reference: malformed
    t = to_dev(d)
    t["cache_len"][2] = d["Lmax"] + 1           # breaks the host's promise
    out, lse, st = run_attn(d, t, chunk_keys=ck)
    assert list(st.cpu().numpy()) == [0, 7, 2, 0]
    assert torch.all(out[1] == 0) and torch.all(out[2] == 0)
    assert torch.all(lse[1] == 0) and torch.all(lse[2] == 0)
    # the other requests are unaffected
    rows = np.array([r for r in oracle.all_rows(4, 20, 8) if r[0] in (0, 3)], np.int32)
    ref, _, _ = oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                      d["k_tree"], d["v_tree"], d["parents"], d["scale"], rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    np.testing.assert_allclose(got, ref, atol=2e-2, rtol=1e-2)


BALANCED = {
    # name: (spec, explicit prefix lengths or None)
    "mixed_lengths": (dict(B=8, N=32, Hq=16, Hkv=4, L=4096), [0, 1, 63, 64, 65, 3000, 17, 4096]),
    "one_long_many_short": (dict(B=12, N=24, Hq=8, Hkv=2, L=6000), [6000] + [40] * 11),
    "tree_tiles_split_n128": (dict(B=3, N=128, Hq=8, Hkv=4, L=(10, 600)), None),
    "b64_lane_limit": (dict(B=64, N=16, Hq=8, Hkv=2, L=(0, 700)), None),
    "b65_host_split": (dict(B=65, N=16, Hq=8, Hkv=2, L=(0, 700)), None),
    "many_row_blocks": (dict(B=2, N=64, Hq=64, Hkv=8, L=(300, 1200)), None),
}


@pytest.mark.parametrize("case", sorted(BALANCED))
def test_balanced_split(case):
    announce("attn balanced split %s" % case)
    kw, lengths = BALANCED[case]
    d = synth.make(spec(**kw))
    if lengths is not None:
        d["cache_len"] = np.array(lengths, np.int32)
    check_attn(d)


@pytest.mark.parametrize("L,ck", [(0, 0), (191, 0), (192, 0), (193, 0), (1000, 0), (4096, 0),
                                  (191, 256), (450, 256), (4095, 256)])
def test_prefix_shorter_than_promise(L, ck):
    """One request (fixed split), promised 4096 keys, holding L: the first
    tiles of a chunk are copied before L is read, so every cache row at or
    past L is NaN here -- a copy of such a row reaching the math would turn
    the outputs into NaN."""
    announce("attn prefix %d of promised 4096, chunk_keys=%d" % (L, ck))
    d = synth.make(spec(B=1, N=48, Hq=16, Hkv=4, L=4096))
    d["cache_len"] = np.array([L], np.int32)
    for k in ("k_cache", "v_cache"):
        d[k] = d[k].copy()
        d[k][:, :, L:, :] = np.nan
    check_attn(d, chunk_keys=ck)
