"""Checks on the gfx950 assembly of the matrix-core kernels (CPU only).

The compiler inserts the wait states that gfx9 matrix instructions need
around vector instructions, but it cannot see inside inline asm. Every kernel
is compiled to assembly and checked two ways, against the requirements of the
CDNA3 ISA's table of independent instructions between dependent matrix (XDL)
and vector instructions (the same numbers LLVM's hazard recognizer encodes
for gfx940 and gfx950):
 - each v_mfma's A, B and C sources are traced back to the last instruction
   that wrote them: if that was a vector instruction (in or out of inline
   asm), at least two wait states (instructions or s_nop slots) must separate
   the two (the table's VALU write -> XDL source read);
 - each vector instruction inside inline asm that reads a register a v_mfma
   wrote, or writes a register a v_mfma read as its accumulator, must come at
   least MFMA_TO_ASM wait states after that v_mfma, scanning back in layout
   order across block boundaries. The table asks for the instruction's pass
   count plus 3 (one more on gfx950) between an XDL instruction and a vector
   read or overwrite of its registers: 12 for the 8-pass 16x16x32 f16 and
   bf16 instructions, the only matrix instructions the kernels use (a
   16-pass 32x32 instruction would need 20, more than MFMA_TO_ASM).
"""

import os
import re
import shutil
import subprocess

import pytest

from quantized_kv_cache_quantize_amd import build as B

MIN_WAIT = 2
MFMA_TO_ASM = 18


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[:])v(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _kernels(asm, keep_asm_marks=False):
    for m in re.finditer(r"^(_Z\S*_kernel\S*):", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        out = []
        for ln in asm[m.end():end].split("\n"):
            t = ln.strip()
            if keep_asm_marks and t.startswith((";;#ASMSTART", ";;#ASMEND")):
                out.append(t)
                continue
            t = t.split(";")[0].strip()
            if t and not t.startswith("."):
                out.append(t)
        yield name, out


def _asm_after_mfma(lines):
    """Smallest count of wait states between a v_mfma and a later vector
    instruction inside inline asm that reads one of its results or writes
    one of its accumulator sources."""
    worst = None
    inside = False
    for i, ln in enumerate(lines):
        if ln.startswith(";;#ASMSTART"):
            inside = True
            continue
        if ln.startswith(";;#ASMEND"):
            inside = False
            continue
        if not inside or not ln.startswith("v_") or ln.startswith("v_mfma"):
            continue
        ops = ln.split(None, 1)[1].split(",")
        reads, writes = _regs(",".join(ops[1:])), _regs(ops[0])
        waits = 0
        for j in range(i - 1, -1, -1):
            prev = lines[j]
            if prev.startswith(";;#") or prev.endswith(":"):
                continue
            if waits >= MFMA_TO_ASM:
                break
            if prev.startswith("v_mfma"):
                mops = prev.split(None, 1)[1].split(",")
                if _regs(mops[0]) & reads or _regs(mops[3]) & writes:
                    worst = waits if worst is None else min(worst, waits)
                    break
            waits += int(prev.split()[1]) + 1 if prev.startswith("s_nop") else 1
    return worst


def _min_wait(lines):
    """Smallest count of wait states between a vector write and an MFMA
    read of that register, scanning back within one basic block."""
    worst = None
    for i, ln in enumerate(lines):
        if not ln.startswith("v_mfma"):
            continue
        ops = ln.split(None, 1)[1].split(",")
        srcs = _regs(ops[1]) | _regs(ops[2]) | _regs(ops[3])
        waits = 0
        for j in range(i - 1, max(-1, i - 16), -1):
            prev = lines[j]
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            if prev.endswith(":") or prev.startswith(("s_cbranch", "s_branch")):
                break
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                if _regs(prev.split(None, 1)[1].split(",")[0]) & srcs:
                    worst = waits if worst is None else min(worst, waits)
                    break
            waits += 1
    return worst


MFMA_SOURCES = ("sdpa_mfma.hip", "sdpa_prefill.hip")  # every source with matrix instructions


@pytest.fixture(scope="module")
def mfma_asm(tmp_path_factory):
    hipcc = B.hipcc()
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    texts = []
    for src in MFMA_SOURCES:
        out = d / (src + ".s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
               os.path.join(B.CSRC, src), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True)
        texts.append(out.read_text())
    return "\n".join(texts)


def test_every_matrix_source_is_checked():
    """A source added later with matrix instructions must join the list."""
    for src in B.sources():
        if os.path.basename(src) not in MFMA_SOURCES:
            assert "__builtin_amdgcn_mfma" not in open(src).read(), "%s uses matrix instructions but is not checked" % src


def test_vector_write_to_mfma_read_wait_states(mfma_asm):
    kernels = list(_kernels(mfma_asm))
    assert kernels, "no kernels found in the assembly"
    for name, lines in kernels:
        w = _min_wait(lines)
        if w is not None:
            assert w >= MIN_WAIT, "%s: MFMA reads a vector result after %d wait states" % (name, w)


def test_mfma_result_to_inline_asm_wait_states(mfma_asm):
    for name, lines in _kernels(mfma_asm, keep_asm_marks=True):
        w = _asm_after_mfma(lines)
        if w is not None:
            assert w >= MFMA_TO_ASM, "%s: inline asm reads a matrix result after %d wait states" % (name, w)


def test_checker_flags_asm_after_mfma():
    lines = ["v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[0:3]", ";;#ASMSTART",
             "v_mul_f32 v1, v1, v40", ";;#ASMEND"]
    assert _asm_after_mfma(lines) == 0
    lines = ["v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[0:3]", ";;#ASMSTART", "s_nop 7", "s_nop 7",
             "s_nop 3", ";;#ASMEND", ".LBB0_1:", ";;#ASMSTART", "v_mul_f32 v1, v1, v40", ";;#ASMEND"]
    assert _asm_after_mfma(lines) is None  # 20 wait states: the scan stops before the MFMA
    # an asm write into the accumulator source of a v_mfma just issued
    lines = ["v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[4:7]", "s_nop 0", ";;#ASMSTART",
             "v_lshlrev_b32 v5, 4, v40", ";;#ASMEND"]
    assert _asm_after_mfma(lines) == 1


def test_checker_flags_a_close_write():
    # the checker itself: a vector write right before the MFMA that reads it
    lines = ["v_and_or_b32 v10, v1, s2, v3", "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], 0"]
    assert _min_wait(lines) == 0
    lines = ["v_and_or_b32 v10, v1, s2, v3", "s_nop 1", "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], 0"]
    assert _min_wait(lines) == 2
    lines = ["v_mul_f32 v2, v2, v9", "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], v[0:3]"]
    assert _min_wait(lines) == 0  # an accumulator source counts too


def test_only_eight_pass_matrix_instructions(mfma_asm):
    """MFMA_TO_ASM covers the 8-pass 16x16x32 instructions only; a longer
    matrix instruction would need a larger threshold."""
    ops = set(re.findall(r"^\s*(v_mfma\w+)", mfma_asm, re.M))
    assert ops and ops <= {"v_mfma_f32_16x16x32_f16", "v_mfma_f32_16x16x32_bf16"}, ops
