"""Checks on the gfx950 assembly of the matrix-core kernels (CPU only).

The compiler inserts the wait states that gfx9 matrix instructions need after
a vector instruction writes one of their A/B source registers, but it cannot
see inside inline asm. Every kernel is compiled to assembly and each
v_mfma's A/B sources are traced back to the last instruction that wrote them:
if that was a vector instruction (in or out of inline asm), at least two
wait states (instructions or s_nop slots) must separate the two.
"""

import os
import re
import shutil
import subprocess

import pytest

from quantized_kv_cache_quantize_amd import build as B

MIN_WAIT = 2


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[:])v(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _kernels(asm):
    for m in re.finditer(r"^(_Z\S*_kernel\S*):", asm, re.M):
        name = m.group(1)
        end = asm.index(".Lfunc_end", m.end())
        lines = [ln.split(";")[0].strip() for ln in asm[m.end():end].split("\n")]
        yield name, [ln for ln in lines if ln and not ln.startswith(".")]


def _min_wait(lines):
    """Smallest count of wait states between a vector write and an MFMA
    read of that register, scanning back within one basic block."""
    worst = None
    for i, ln in enumerate(lines):
        if not ln.startswith("v_mfma"):
            continue
        ops = ln.split(None, 1)[1].split(",")
        srcs = _regs(ops[1]) | _regs(ops[2])
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


@pytest.fixture(scope="module")
def mfma_asm(tmp_path_factory):
    hipcc = B.hipcc()
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "sdpa_mfma.s"
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC,
           os.path.join(B.CSRC, "sdpa_mfma.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def test_vector_write_to_mfma_read_wait_states(mfma_asm):
    kernels = list(_kernels(mfma_asm))
    assert kernels, "no kernels found in the assembly"
    for name, lines in kernels:
        w = _min_wait(lines)
        if w is not None:
            assert w >= MIN_WAIT, "%s: MFMA reads a vector result after %d wait states" % (name, w)


def test_checker_flags_a_close_write():
    # the checker itself: a vector write right before the MFMA that reads it
    lines = ["v_and_or_b32 v10, v1, s2, v3", "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], 0"]
    assert _min_wait(lines) == 0
    lines = ["v_and_or_b32 v10, v1, s2, v3", "s_nop 1", "v_mfma_f32_16x16x32_f16 v[0:3], v[10:13], v[20:23], 0"]
    assert _min_wait(lines) == 2
