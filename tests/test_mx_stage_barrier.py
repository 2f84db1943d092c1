"""Static check of the MXFP4 prefill kernel's stage barriers (CPU only).

The kernel's workgroup barrier is `s_waitcnt vmcnt(N) lgkmcnt(0); s_barrier`
with N the number of operand loads of one step: the wave's share of the next B
stage was issued before the previous barrier, so it has landed once at most N
operations remain in flight, provided the wave issued at least N since that
barrier.  That only holds if the compiler keeps every step's loads between its
two barriers.  This test compiles mx_gemm.hip for gfx950, rebuilds each
instance's control-flow graph from the assembly and checks that on every path
from one barrier to the next at least N vector-memory operations are issued (a
load that some waves skip, inside an exec-mask branch, counts only on the path
that runs it; a load the compiler dropped does not count at all).
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "rotation_w4a4_quantization_amd", "csrc", "mx_gemm.hip")
INSTANCES = {  # mangled name -> operand loads per step (A loads + B loads of one wave)
    "_ZN4w4a414mx_gemm_kernelILi8ELi2ELi2EEEvNS_12MxGemmParamsE": 3,
    "_ZN4w4a414mx_gemm_kernelILi4ELi1ELi2EEEvNS_12MxGemmParamsE": 3,
}
VMEM = re.compile(r"^\s*(buffer_load|buffer_store|buffer_atomic|global_load|global_store|global_atomic|"
                  r"flat_load|flat_store|scratch_load|scratch_store)\w*")
LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)")
END = re.compile(r"^\s*(s_endpgm|s_setpc_b64)")


def _hip_flags():
    spec = importlib.util.spec_from_file_location(
        "w4a4_build", os.path.join(ROOT, "rotation_w4a4_quantization_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [f for f in mod.HIP_FLAGS if f not in ("-shared", "-fPIC")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("mx") / "mx_gemm.s")
    cmd = [hipcc, *_hip_flags(), "-S", "--cuda-device-only", "-I", os.path.join(ROOT, "include"), "-o", out, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


def _function(text, name):
    lines = text.splitlines()
    start = next(i for i, ln in enumerate(lines) if ln.startswith(name + ":"))
    body = []
    for ln in lines[start + 1:]:
        body.append(ln)
        if END.match(ln):
            break
    return body


def _blocks(body):
    """Basic blocks [label, events, successors]; an event is 'v' for a
    vector-memory operation or ('bar', N) for a barrier (N: the vmcnt of the
    inline-asm stage barrier, None for any other s_barrier)."""
    blocks, cur, events, in_asm, asm_vm = [], "entry", [], False, None

    def close(succ):
        nonlocal events
        blocks.append([cur, events, succ])
        events = []

    for ln in body:
        s = ln.strip()
        m = LABEL.match(ln)
        if m:
            close(None)                 # fall through into the labelled block
            cur = m.group(1)
        elif s.startswith(";;#ASMSTART"):
            in_asm, asm_vm = True, None
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm:
            mv = re.match(r"s_waitcnt\s+vmcnt\((\d+)\)", s)
            if mv:
                asm_vm = int(mv.group(1))
            if s.startswith("s_barrier"):
                events.append(("bar", asm_vm))
        elif s.startswith("s_barrier"):
            events.append(("bar", None))
        elif VMEM.match(ln):
            events.append("v")
        elif BRANCH.match(ln):
            b = BRANCH.match(ln)
            close([b.group(2)] + (["<next>"] if b.group(1) != "s_branch" else []))
            cur = f"after_{len(blocks)}"
        elif END.match(ln):
            close([])
            cur = f"after_{len(blocks)}"
    close([])
    for i, blk in enumerate(blocks):
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        succ = [nxt] if blk[2] is None else [nxt if t == "<next>" else t for t in blk[2]]
        blk[2] = [t for t in succ if t is not None]
    return blocks


def _check(body):
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks)}
    preds = {i: [] for i in range(len(blocks))}
    for i, b in enumerate(blocks):
        for s in b[2]:
            if s in index:
                preds[index[s]].append(i)
    NONE = -1          # no barrier yet on some path into this point
    INF = 10 ** 6      # not reached yet
    out = [INF] * len(blocks)

    def run(i, cnt, check):
        checked = []
        for ev in blocks[i][1]:
            if ev == "v":
                cnt = cnt if cnt == NONE else min(cnt + 1, 999)
            else:
                n = ev[1]
                if check and n is not None and cnt != NONE:
                    checked.append((blocks[i][0], cnt, n))
                cnt = 0
        return cnt, checked

    changed = True
    while changed:
        changed = False
        for i in range(len(blocks)):
            ins = [out[p] for p in preds[i] if out[p] != INF]
            if i == 0:
                cin = NONE
            elif not ins:
                continue
            else:
                cin = NONE if NONE in ins else min(ins)
            c, _ = run(i, cin, False)
            if c != out[i]:
                out[i] = c
                changed = True
    results = []
    for i in range(len(blocks)):
        ins = [out[p] for p in preds[i] if out[p] != INF]
        cin = NONE if i == 0 or NONE in ins or not ins else min(ins)
        results += run(i, cin, True)[1]
    return results


@pytest.mark.parametrize("name", sorted(INSTANCES))
def test_stage_barrier_counts(asm, name):
    ks = INSTANCES[name]
    res = _check(_function(asm, name))
    assert len(res) >= 8, f"expected the loop's stage barriers, found {res}"
    bad = [r for r in res if r[1] < r[2]]
    assert not bad, f"fewer vector-memory operations than the barrier's vmcnt on some path: {bad}"
    assert {n for _, _, n in res} == {ks}, res
