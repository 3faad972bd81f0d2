"""Properties of the compiled kernels that their correctness or speed rests on
but that no numeric test can pin down reliably (CPU only: hipcc
cross-compiles gfx950 assembly without a GPU).

The query and parent loads of attn_mfma.hip are issued as inline assembly
ahead of the tile copies and waited for by one `s_waitcnt vmcnt(N)` statement
that names their registers in a trailing comment.  The compiler does not know
those registers are still being written: if it read or copied one before that
wait, the kernel would use stale data.  So, for every attention kernel:
  * exactly one such wait, guarding exactly the async loads' destinations;
  * on every control-flow path from the loads to the wait, no instruction
    touches a register whose load is still in flight.
And no kernel of the library uses private (scratch) memory: scratch accesses
are vector memory operations, so each one waits on every load in flight (the
tile copies, the row passes).
"""
import os
import re
import shutil
import subprocess

import pytest

from token_tree_verification_attn_amd import build as ttv_build

SRC = os.path.join(ttv_build.CSRC, "attn_mfma.hip")
KERNEL = re.compile(r"^(_ZN3ttv17attn_mfma2_kernel\w+):")
ASYNC_LOAD = re.compile(r"^global_load_dword(x4)? v.*,\s*off$")


def vregs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(ttv_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "attn_mfma.s")
    flags = [f for f in ttv_build.FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run([ttv_build.HIPCC] + flags + ["--cuda-device-only", "-S", "-o", out, SRC],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return open(out).read().split("\n")


def kernels(lines):
    """name -> (instructions, label -> instruction index)"""
    res = {}
    starts = [(i, KERNEL.match(l).group(1)) for i, l in enumerate(lines) if KERNEL.match(l)]
    for i, name in starts:
        ins, labels = [], {}
        j = i + 1
        while not lines[j].startswith(".Lfunc_end"):  # (a kernel may end early too)
            m = re.match(r"^(\.LBB\w+):", lines[j])
            t = lines[j].strip()
            if m:
                labels[m.group(1)] = len(ins)
            elif lines[j].startswith("\t") and t and not t.startswith(";") and not t.startswith("."):
                ins.append(t)
            j += 1
        res[name] = (ins, labels)
    return res


def test_every_shape_compiled(asm):
    names = kernels(asm)
    assert len(names) == 6, sorted(names)


@pytest.mark.parametrize("src", ["attn_mfma.hip", "attn.hip", "verify.hip", "commit.hip",
                                 "topology.hip"])
def test_no_private_memory(src, tmp_path):
    # every kernel of the library: private (scratch) accesses are vector
    # memory operations, so each one also waits on the loads in flight
    if not os.path.exists(ttv_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "k.s")
    flags = [f for f in ttv_build.FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run([ttv_build.HIPCC] + flags + ["--cuda-device-only", "-S", "-o", out,
                          os.path.join(ttv_build.CSRC, src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = open(out).read().split("\n")
    assert not [l for l in lines if l.strip().startswith("scratch_")], src
    assert not [l for l in lines if re.search(r"\.private_segment_fixed_size:\s*[1-9]", l)], src


def test_copies_padded_after_their_base(asm):
    # each tile copy reads its base address from SGPRs that v_readfirstlane
    # (VALU) wrote just before; a vector-memory read of an SGPR needs 5 wait
    # states after a VALU write of it, and the compiler cannot add them inside
    # inline assembly (without them a copy took a stale base and faulted)
    for name, (ins, _) in kernels(asm).items():
        copies = [i for i, t in enumerate(ins) if t.startswith("global_load_lds")]
        assert copies, name
        assert all(ins[i - 1].startswith("s_nop 4") for i in copies), name


def guard_violations(ins, labels):
    """Instructions that touch a register of an async load before its wait,
    on any control-flow path from the first load to the wait."""
    loads = [i for i, t in enumerate(ins) if ASYNC_LOAD.match(t.split(";")[0].strip())]
    pins = [i for i, t in enumerate(ins) if t.startswith("s_waitcnt vmcnt") and ";" in t]
    assert loads and len(pins) == 1
    pin = pins[0]
    dst = set()
    for i in loads:
        dst |= vregs(ins[i].split(None, 1)[1].split(",")[0])
    assert vregs(ins[pin].split(";", 1)[1]) == dst
    seen, bad, stack = set(), [], [(loads[0], frozenset())]
    while stack:
        pc, pend = stack.pop()
        while (pc, pend) not in seen and pc != pin and pc < len(ins):
            seen.add((pc, pend))
            t = ins[pc]
            op, _, rest = t.partition(" ")
            rest = rest.split(";")[0]
            if pc in loads:
                d, _, addr = rest.partition(",")
                if vregs(addr) & pend:
                    bad.append(t)
                pend = pend | frozenset(vregs(d))
                pc += 1
                continue
            if vregs(rest) & pend:
                bad.append(t)
            if op == "s_endpgm":
                break
            if op == "s_branch":
                pc = labels[rest.strip()]
                continue
            if op.startswith("s_cbranch"):
                stack.append((labels[rest.strip()], pend))
            pc += 1
    return bad


def test_async_loads_guarded(asm):
    for name, (ins, labels) in kernels(asm).items():
        assert not guard_violations(ins, labels), name


def test_guard_check_sees_a_read_before_the_wait(asm):
    # the check itself: a copy of a loaded register placed right after its
    # load must be reported
    name, (ins, labels) = sorted(kernels(asm).items())[0]
    i = [k for k, t in enumerate(ins) if t.startswith("global_load_dwordx4") and t.endswith("off")][0]
    reg = sorted(vregs(ins[i].split(None, 1)[1].split(",")[0]))[0]
    planted = ins[:i + 1] + ["v_mov_b32_e32 v255, v%d" % reg] + ins[i + 1:]
    shifted = {k: (v + 1 if v > i else v) for k, v in labels.items()}
    assert guard_violations(planted, shifted) == ["v_mov_b32_e32 v255, v%d" % reg]
