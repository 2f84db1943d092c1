"""Static check of the 32x32-block GEMMs' A-stage waits (CPU only).

gemm_asym_x32_kernel streams each group's activation codes into a per-wave
LDS stage with buffer_load ... lds, two groups ahead, and reads the stage
only after an explicit `s_waitcnt vmcnt(6)` at the top of the group's step:
vector-memory operations complete in order, and the kernel issues six of
them after a group's codes, zero-point and scale (B rows of two groups, the
next group's codes and its zero-point and scale; 8 in the 4-wave instance,
whose threads stage two B chunks each).  That only holds if the
compiler keeps that issue order.  This test compiles gemm.hip for gfx950,
rebuilds the kernel's control-flow graph from the assembly and walks every
path (loop iterations, the tail steps for any group count) with the queue of
vector-memory operations in flight, each labelled with the group it belongs
to, applying only the kernel's explicit waits (the compiler's own tracking of
writes into LDS is not relied upon; its waits could only retire operations
sooner).  At every read of an A stage, the codes of the group being read
must no longer be in flight.  (Its zero-point and scale are loaded into registers,
which the compiler itself waits for before their first use.)
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "rotation_w4a4_quantization_amd", "csrc", "gemm.hip")
# mangled name -> the explicit wait that opens a step: 2 x (B chunks per
# thread and group) + 4
# (the symmetric 4-wave kernel has no zero-point and scale loads: 2 x 2 + 2)
KERNELS = {"_ZN4w4a420gemm_asym_x32_kernelILi8EEEvNS_10GemmParamsE": 6,
           "_ZN4w4a420gemm_asym_x32_kernelILi4EEEvNS_10GemmParamsE": 8,
           "_ZN4w4a419gemm_sym_x32_kernelILi4EEEvNS_10GemmParamsE": 6}
LABEL = re.compile(r"^(\.LBB\w+):")
BRANCH = re.compile(r"^\s*(s_branch|s_cbranch_\w+)\s+(\.LBB\w+)")
END = re.compile(r"^\s*(s_endpgm|s_setpc_b64)")
VMEM = re.compile(r"^\s*(buffer|global|flat|scratch)_(load|store|atomic)\w*")
WAIT = re.compile(r"s_waitcnt\s+.*vmcnt\((\d+)\)")


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
    out = str(tmp_path_factory.mktemp("gemm") / "gemm.s")
    cmd = [hipcc, *_hip_flags(), "-S", "--cuda-device-only", "-I", os.path.join(ROOT, "include"), "-o", out, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read().splitlines()


def _function(lines, name):
    start = next(i for i, ln in enumerate(lines) if ln.startswith(name + ":"))
    fn = []
    for ln in lines[start + 1:]:
        fn.append(ln)
        if END.match(ln):
            break
    return fn


def _events(line, in_asm, step_wait):
    """Events of one instruction: ('W', n) the explicit wait opening a step,
    ('w', n) another explicit wait, 'step' (the explicit wait that opens a group's step), 'dma', 'zs'
    (a zero-point or scale load), 'v' (other vector-memory op), 'lds_read'.
    The first two LDS reads of a step are its A-stage reads: the step reads
    both A chunks before anything else (the weight fragments' reads follow a
    scheduling barrier)."""
    s = line.strip()
    m = WAIT.search(s)
    if m and s.startswith("s_waitcnt"):
        if not in_asm:
            return []                # the compiler's own waits are not relied upon
        n = int(m.group(1))
        return [("W", n), "step"] if n == step_wait else [("w", n)]
    if VMEM.match(line):
        if re.search(r"\blds\b", s.split(";")[0]):
            return ["dma"]
        if s.startswith("buffer_load_ubyte") or re.match(r"buffer_load_dword\s", s):
            return ["zs"]
        return ["v"]
    if s.startswith("ds_read"):
        return ["lds_read"]
    return []


def _cfg(fn, step_wait):
    blocks, cur, evs, in_asm = [], "entry", [], False

    def close(succ):
        nonlocal evs
        blocks.append([cur, evs, succ])
        evs = []

    for ln in fn:
        s = ln.strip()
        lab = LABEL.match(ln)
        if lab:
            close(None)
            cur = lab.group(1)
        elif s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif BRANCH.match(ln):
            b = BRANCH.match(ln)
            close([b.group(2)] + (["<next>"] if b.group(1) != "s_branch" else []))
            cur = f"after_{len(blocks)}"
        elif END.match(ln):
            close([])
            cur = f"after_{len(blocks)}"
        else:
            evs += _events(ln, in_asm, step_wait)
    close([])
    for i, blk in enumerate(blocks):
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        succ = [nxt] if blk[2] is None else [nxt if t == "<next>" else t for t in blk[2]]
        blk[2] = [t for t in succ if t is not None]
    return blocks


def _walk(blocks):
    """Every path from the entry, with the in-flight queue as state.  Labels
    are kept relative to the current step (group - step), so the states are
    finite and the walk ends.  Returns (reads checked, violations, steps)."""
    index = {b[0]: i for i, b in enumerate(blocks)}
    seen, stack = set(), [(0, (), 0, 0, 0, 0)]
    reads, bad, steps = 0, [], 0
    while stack:
        bi, queue, pro_dma, pro_zs, started, a_left = stack.pop()
        key = (bi, queue, pro_dma, pro_zs, started, a_left)
        if key in seen:
            continue
        seen.add(key)
        q = list(queue)
        for ev in blocks[bi][1]:
            if ev == "step":                # a step opens: its group is relative 0
                steps += 1
                if started:
                    q = [(t, None if g is None else g - 1) for t, g in q]
                started = 1
                a_left = 2
            elif ev == "lds_read":
                if a_left:
                    a_left -= 1
                    ev = "read"
            if isinstance(ev, tuple):
                while len(q) > ev[1]:
                    q.pop(0)
            elif ev in ("dma", "zs"):
                if not started:        # prologue: groups 0 and 1, two operations each
                    n = pro_dma if ev == "dma" else pro_zs
                    q.append((ev, n // 2))
                    if ev == "dma":
                        pro_dma += 1
                    else:
                        pro_zs += 1
                else:
                    q.append((ev, 2))  # a step requests the codes, zero-point and scale of group + 2
            elif ev == "v":
                q.append(("v", None))
            elif ev == "read":
                reads += 1
                pending = [e for e in q if e[0] == "dma" and e[1] == 0]
                if pending:
                    bad.append((blocks[bi][0], list(q)))
            assert len(q) <= 512, "vector-memory queue grows without a wait"
        for succ in blocks[bi][2]:
            if succ in index:
                stack.append((index[succ], tuple(q), pro_dma, pro_zs, started, a_left))
    return reads, bad, steps


@pytest.mark.parametrize("name", sorted(KERNELS))
def test_a_stage_reads_wait_for_their_group(asm, name):
    blocks = _cfg(_function(asm, name), KERNELS[name])
    reads, bad, steps = _walk(blocks)
    assert steps >= 8 and reads >= 16, (steps, reads)
    assert not bad, f"an A stage is read while its group's loads may be in flight: {bad[:3]}"
