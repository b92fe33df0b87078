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


def _start_asm(src, out, part):
    flags = [f for f in fpbuild.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, f"-DFP_FAST_PART={part}", "-I", fpbuild.CSRC, "--cuda-device-only", "-S", "-x", "hip",
           src, "-o", out]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish_asm(proc, out):
    _, err = proc.communicate()
    assert proc.returncode == 0, err[-4000:]
    return open(out).read()


# The form of scalar_load16 that once sign-extended the descriptor address: readfirstlane
# returns int, and widening the low half straight to 64 bits copies its bit 31 into the
# high half.
_GOOD_WIDEN = ("((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32)) << 32) |\n"
               "                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)a)")
_BAD_WIDEN = ("((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32)) << 32) |\n"
              "                        (uint64_t)__builtin_amdgcn_readfirstlane((unsigned)a)")


@pytest.fixture(scope="module")
def fast_asm(tmp_path_factory):
    """The fast kernel's gfx950 assembly (every part of its instantiations, as the build
    compiles them), and that of part 0 of a copy with the sign-extending widening planted
    in scalar_load16 (all compiled at once)."""
    d = tmp_path_factory.mktemp("isa")
    src = os.path.join(fpbuild.CSRC, "fused_proj_fast.hip")
    text = open(src).read()
    assert text.count(_GOOD_WIDEN) == 1, "scalar_load16's widening changed: update this test"
    bad_src = os.path.join(d, "fast_bad.hip")
    with open(bad_src, "w") as f:
        f.write(text.replace(_GOOD_WIDEN, _BAD_WIDEN))
    good = [(os.path.join(d, f"fast.part{k}.s"), k) for k in range(fpbuild.FAST_PARTS)]
    bad_out = os.path.join(d, "fast_bad.s")
    procs = [(_start_asm(src, out, k), out) for out, k in good]
    pb = _start_asm(bad_src, bad_out, 0)
    good_asm = "\n".join(_finish_asm(p, out) for p, out in procs)
    return good_asm, _finish_asm(pb, bad_out)


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
def test_inline_asm_memory_instructions_have_their_wait_states(fast_asm):
    asm = fast_asm[0]
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


_SGPR_PAIR = re.compile(r"s\[(\d+):(\d+)\]")


def _dest_and_sources(inst):
    """Scalar registers an instruction writes (its first operand) and reads (the rest)."""
    if " " not in inst:
        return set(), set()
    ops = [o.strip() for o in inst.split(None, 1)[1].split(",")]
    return _sgprs(ops[0]), _sgprs(",".join(ops[1:]))


def _sign_extension(inst):
    return (re.match(r"s_ashr_i(32|64)\s.*,\s*(31|63)$", inst) is not None or inst.startswith("s_bfe_i64")
            or inst.startswith("s_sext_"))


def _address_slice_problems(asm):
    """For every inline-asm s_load_dwordx16, follow the scalar registers its address pair
    is computed from back through its basic block; report any sign extension among them."""
    problems, checked = [], 0
    for name, lines in _kernels(asm):
        insts = [l.strip() for l in lines]
        for i, t in enumerate(insts):
            if not t.startswith("s_load_dwordx16"):
                continue
            checked += 1
            m = _SGPR_PAIR.findall(t.split(",", 1)[1])[0]
            needed = set(range(int(m[0]), int(m[1]) + 1))
            for p in reversed(insts[max(0, i - 200):i]):
                if p.startswith(".LBB") or p.startswith("s_cbranch") or p.startswith("s_branch"):
                    break
                if not p or p.startswith((";", ".")) or not p.startswith("s_"):
                    if p.startswith("v_readlane") or p.startswith("v_readfirstlane"):
                        needed -= _dest_and_sources(p)[0]
                    continue
                dst, src = _dest_and_sources(p)
                if not dst & needed:
                    continue
                if _sign_extension(p):
                    problems.append(f"{name}: '{p}' feeds the address of '{t}'")
                    break
                needed = (needed - dst) | src
    return checked, problems


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_descriptor_address_is_not_sign_extended(fast_asm):
    """The column-descriptor address reaching s_load_dwordx16 (scalar_load16) is formed
    from the table's 64-bit address and an unsigned index: no sign extension anywhere in
    the scalar registers it is computed from. A sign-extended low half once turned the
    address into garbage whenever its bit 31 was set; a copy of the kernel with that
    widening planted back must be caught by the same check."""
    good, bad = fast_asm
    checked, problems = _address_slice_problems(good)
    assert checked >= 8, "no descriptor loads found"
    assert not problems, "\n".join(problems[:10])
    checked_bad, problems_bad = _address_slice_problems(bad)
    assert checked_bad >= 8 and problems_bad, "the planted sign extension was not detected"
