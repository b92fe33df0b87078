"""Compiles the fast kernel to gfx950 assembly and checks the wait states in front of
every inline-asm memory instruction (CPU only: hipcc cross-compiles).

The direct-to-LDS loads and the scalar descriptor load are inline asm, which the
compiler's hazard recognizer does not look into. On gfx9-family chips a VMEM or SMEM
instruction reading an SGPR that a VALU instruction wrote (v_readlane when the compiler
restores a spilled SGPR, v_readfirstlane, v_cmp into an SGPR pair) needs 5 wait states
first, and an LDS-DMA load needs 1 after an SALU write of M0. Missing wait states let the
load use a stale base address; this test pins the fix (every such asm statement opens
with s_nop 4) against the code the compiler actually emits.
"""
import os
import re
import shutil
import subprocess

import pytest

from ff_input_projection_amd import build as fpbuild

HIPCC = fpbuild.HIPCC


def _asm(tmp_path):
    src = os.path.join(fpbuild.CSRC, "fused_proj_fast.hip")
    out = os.path.join(tmp_path, "fast.s")
    flags = [f for f in fpbuild.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-x", "hip", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return open(out).read()


def _kernels(asm):
    for name in re.findall(r"^(_Z\S*fused_proj_fast_kernel\S*):", asm, re.M):
        a = asm.index(name + ":")
        b = asm.index(".Lfunc_end", a)
        yield name, asm[a:b].split("\n")


def _sgprs(text):
    regs = set()
    for m in re.finditer(r"s\[(\d+):(\d+)\]", text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", text):
        regs.add(int(m.group(1)))
    return regs


def _valu_sgpr_defs(inst):
    m = re.match(r"(v_readlane_b32|v_readfirstlane_b32)\s+s(\d+)", inst)
    if m:
        return {int(m.group(2))}
    m = re.match(r"v_\w+_e64\s+s\[(\d+):(\d+)\]", inst)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_inline_asm_memory_instructions_have_their_wait_states(tmp_path):
    asm = _asm(str(tmp_path))
    checked = 0
    problems = []
    for name, lines in _kernels(asm):
        insts = []   # (text, inside inline asm)
        in_asm = False
        for l in lines:
            t = l.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if l.startswith("\t") and t and not t.startswith((".", ";")):
                insts.append((t, in_asm))
        for i, (t, inside) in enumerate(insts):
            if not inside or not (t.startswith("global_load_lds") or t.startswith("s_load_dword")):
                continue
            checked += 1
            operands = t.split(None, 1)[1] if " " in t else ""
            # the destination of a scalar load is written, not read
            if t.startswith("s_load_dword"):
                operands = operands.split(",", 1)[1]
            reads = _sgprs(operands)
            waits, k = 0, i - 1
            while k >= 0 and waits < 5:
                p = insts[k][0]
                if p.startswith("s_nop"):
                    waits += int(p.split()[1], 0) + 1
                    k -= 1
                    continue
                if _valu_sgpr_defs(p) & reads:
                    problems.append(f"{name}: '{p}' then '{t}' after {waits} wait states")
                    break
                if t.startswith("global_load_lds") and waits < 1 and re.match(r"s_\w+\s+m0,", p):
                    problems.append(f"{name}: '{p}' then '{t}' with no wait state")
                    break
                waits += 1
                k -= 1
    assert checked > 100, "no inline-asm memory instructions found"
    assert not problems, "\n".join(problems[:20])
