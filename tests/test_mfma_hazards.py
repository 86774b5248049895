"""Static check of the MFMA result hazard in the library's own gfx950 code.

With MFMA results in architectural VGPRs, the hardware does not hold back a
VALU or memory instruction that reads (or overwrites) a VGPR an MFMA is still
writing: the program must leave enough wait states (instructions issued in
between, or s_nop cycles) after the MFMA.  The compiler pads straight-line
code; this test checks every path of the compiled kernels, across basic
blocks and loop back edges, so that a change of the filter's loop structure
that leaves a path short fails here instead of returning wrong indices.

It compiles each source that issues MFMAs to gfx950 assembly with the
library's own flags (no GPU needed) and walks the control-flow graph forward
from every MFMA."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from dynamic_top_sparse_amd import build  # noqa: E402

# Wait states the compiler itself inserts before a VALU read of a 32x32x16
# (8-pass) XDL result on gfx950: passes + 3, plus one on this chip.
REQUIRED = 12
SOURCES = ["scorer.hip", "proj.hip"]

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_BRANCH = re.compile(r"^s_(c)?branch(_\w+)?$")


def _vregs(text):
    regs = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def _assembly(src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    cmd = [hipcc, *build.FLAGS, "-S", "--cuda-device-only", os.path.join(build.CSRC, src),
           "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def _functions(asm):
    """name -> list of ('label', name) / ('insn', mnemonic, operands)."""
    funcs = {}
    cur = None
    for raw in asm.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.startswith(".type") and "@function" in line:
            cur = line.split()[1].split(",")[0]
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
            continue
        if line.endswith(":"):
            funcs[cur].append(("label", line[:-1]))
            continue
        if line.startswith("."):
            continue
        parts = line.split(None, 1)
        funcs[cur].append(("insn", parts[0], parts[1] if len(parts) > 1 else ""))
    return {k: v for k, v in funcs.items() if any(x[0] == "insn" for x in v)}


def _blocks(body):
    """Basic blocks as (instructions, successor block indices)."""
    blocks, labels, cur = [], {}, []
    for item in body:
        if item[0] == "label":
            if cur:
                blocks.append(cur)
                cur = []
            labels[item[1]] = len(blocks)
            continue
        cur.append(item)
        if _BRANCH.match(item[1]) or item[1] == "s_endpgm":
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    succ = []
    for i, b in enumerate(blocks):
        last = b[-1]
        s = []
        if _BRANCH.match(last[1]):
            s.append(labels[last[2].strip()])
            if last[1] != "s_branch" and i + 1 < len(blocks):
                s.append(i + 1)
        elif last[1] != "s_endpgm" and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def _wait_states(insn):
    if insn[1] == "s_nop":
        return int(insn[2].strip(), 0) + 1
    return 1


def _shortest_unsafe(blocks, succ, bi, ii):
    """Smallest number of wait states between the MFMA at blocks[bi][ii] and
    an instruction that uses its destination other than as the next MFMA's
    accumulator input (None if every path is at least REQUIRED long)."""
    mfma = blocks[bi][ii]
    dst_text = mfma[2].split(",")[0]
    dst = _vregs(dst_text)
    worst = None
    best_seen = {}
    stack = [(bi, ii + 1, 0)]
    while stack:
        b, i, n = stack.pop()
        if i == 0:
            # a block reached before with no more wait states is covered
            if best_seen.get(b, REQUIRED + 1) <= n:
                continue
            best_seen[b] = n
        stop = False
        while i < len(blocks[b]):
            insn = blocks[b][i]
            if n >= REQUIRED:
                stop = True
                break
            ops = insn[2]
            if insn[1].startswith("v_mfma"):
                fields = [f.strip() for f in ops.split(",")]
                srcs_ab = _vregs(",".join(fields[1:3]))
                if srcs_ab & dst:
                    worst = n if worst is None else min(worst, n)
                # the accumulator input of a chained MFMA, or a new result
                # written over the same registers, is ordered by the matrix
                # pipe itself
            elif _vregs(ops) & dst:
                worst = n if worst is None else min(worst, n)
                stop = True
                break
            n += _wait_states(insn)
            i += 1
        if not stop:
            for s in succ[b]:
                stack.append((s, 0, n))
    return worst


@pytest.mark.parametrize("src", SOURCES)
def test_mfma_results_are_read_after_enough_wait_states(src):
    funcs = _functions(_assembly(src))
    checked = 0
    problems = []
    for name, body in funcs.items():
        blocks, succ = _blocks(body)
        for bi, b in enumerate(blocks):
            for ii, insn in enumerate(b):
                if not insn[1].startswith("v_mfma"):
                    continue
                checked += 1
                short = _shortest_unsafe(blocks, succ, bi, ii)
                if short is not None:
                    problems.append((name[:90], insn[1], short))
    assert checked > 0, f"no MFMA found in {src}"
    assert not problems, problems[:10]


def test_checker_sees_a_short_path():
    """The walker finds a read placed too early, across a branch."""
    asm = """
    .type k,@function
k:
    v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], v[20:23], v[0:15]
    s_cbranch_execz .L1
    v_add_f32 v30, v1, v1
.L1:
    s_nop 3
    v_max_i32 v31, v2, v3
    s_endpgm
.Lfunc_end0:
"""
    funcs = _functions(asm)
    blocks, succ = _blocks(funcs["k"])
    assert _shortest_unsafe(blocks, succ, 0, 0) == 1
    # the same read after a full pad is fine on both paths
    asm_ok = asm.replace("s_nop 3", "s_nop 15")
    funcs = _functions(asm_ok)
    blocks, succ = _blocks(funcs["k"])
    assert _shortest_unsafe(blocks, succ, 0, 0) is not None   # v30 path still short
    asm_ok2 = asm_ok.replace("v_add_f32 v30, v1, v1", "v_add_f32 v30, v40, v40")
    funcs = _functions(asm_ok2)
    blocks, succ = _blocks(funcs["k"])
    assert _shortest_unsafe(blocks, succ, 0, 0) is None
