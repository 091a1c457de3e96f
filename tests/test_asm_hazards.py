"""Wait states around the inline-assembly MFMAs of the mid-size tile kernel.

The mid-size kernel issues its MFMAs as inline assembly, with the
accumulators pinned to AGPRs.  The compiler inserts the wait states that the
hardware does not interlock only around MFMAs it issued itself, so the kernel
relies on rules of its own: no VALU instruction writes an MFMA operand within
two wait states before the MFMA, and nothing but another MFMA touches an MFMA
result within 19 wait states after it (18 is the gfx950 figure for the
longest 16-pass MFMAs reading back into VALU; one more for margin).  This test
compiles the kernel's source for gfx950 and scans the generated code for a
break of either rule -- on the straight-line order and across each loop's back
edge.  The scanner itself is checked on planted cases.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_backward_gemm_amd", "csrc")
KERNELS = ["_ZN3nf417grad_a_mid_kernelILi1EEEvPKvPKfPKjPfiiiiii",
           "_ZN3nf417grad_a_mid_kernelILi3EEEvPKvPKfPKjPfiiiiii"]
VALU_BEFORE = 2
AFTER = 19


def _regs(tok):
    m = re.fullmatch(r"([av])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([av])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(line):
    parts = line.split(None, 1)
    ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def _wait_states(line):
    op, ops = _parse(line)
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def scan(instrs):
    """Rule breaks in a list of instruction lines (executed in order)."""
    bad = []
    for i, line in enumerate(instrs):
        op, ops = _parse(line)
        if "mfma" not in op:
            continue
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(t) for t in ops[1:4]))
        w = 0
        for j in range(i - 1, max(-1, i - 8), -1):
            opj, aj = _parse(instrs[j])
            if w >= VALU_BEFORE:
                break
            if opj.startswith("v_") and "mfma" not in opj and aj and _regs(aj[0]) & srcs:
                bad.append(("valu-before-mfma", w, instrs[j], line))
            w += _wait_states(instrs[j])
        w = 0
        for j in range(i + 1, min(len(instrs), i + 64)):
            if w >= AFTER:
                break
            opj, aj = _parse(instrs[j])
            touched = set().union(*(_regs(t) for t in aj)) if aj else set()
            if "mfma" in opj:
                if _regs(aj[0]) & dst:
                    break  # a later MFMA of the same chain takes over the registers
            elif touched & dst:
                bad.append(("access-after-mfma", w, line, instrs[j]))
            w += _wait_states(instrs[j])
    return bad


def kernel_sequences(asm, name):
    """The kernel's instructions in order, plus each loop's end followed by its head (the back edge)."""
    m = re.search(r"^" + re.escape(name) + r":(.*?)s_endpgm", asm, re.S | re.M)
    assert m, name
    lines, labels = [], {}
    for raw in m.group(1).split("\n"):
        line = raw.split(";")[0].strip()
        if not line or line.startswith("."):
            if re.fullmatch(r"\.LBB\w+:", line):
                labels[line[:-1]] = len(lines)
            continue
        lines.append(line)
    seqs = [lines]
    for i, line in enumerate(lines):
        op, ops = _parse(line)
        if op.startswith("s_cbranch") or op == "s_branch":
            tgt = labels.get(ops[0]) if ops else None
            if tgt is not None and tgt <= i:
                seqs.append(lines[max(tgt, i - 64):i + 1] + lines[tgt:tgt + 64])
    return seqs


def test_scanner_flags_planted_breaks():
    ok = ["v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]",
          "v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]",
          "s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v0, a0"]
    assert scan(ok) == []
    early_read = ok[:2] + ["s_nop 7", "v_accvgpr_read_b32 v0, a1"]
    assert [b[0] for b in scan(early_read)] == ["access-after-mfma"]
    early_write = ["v_accvgpr_write_b32 a2, 0", "v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]"]
    assert [b[0] for b in scan(early_write)] == ["valu-before-mfma"]
    operand = ["v_mov_b32_e32 v9, v1", "s_nop 1", "v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]"]
    assert scan(operand) == []  # two wait states
    operand_close = ["v_mov_b32_e32 v9, v1", "v_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]"]
    assert [b[0] for b in scan(operand_close)] == ["valu-before-mfma"]


@pytest.fixture(scope="module")
def mid_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "wide.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fno-gpu-flush-denormals-to-zero",
           "-fno-strict-aliasing", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "nf4_grad_a_wide.hip"),
           "--offload-device-only", "-S", "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.mark.parametrize("name", KERNELS)
def test_mid_kernel_has_no_mfma_hazard(mid_asm, name):
    seqs = kernel_sequences(mid_asm, name)
    n_mfma = sum("mfma" in s for s in seqs[0])
    assert n_mfma >= 128  # the loop body's MFMAs are there to scan
    assert len(seqs) > 1  # and at least one loop back edge
    bad = [b for s in seqs for b in scan(s)]
    assert bad == [], bad[:5]


@pytest.mark.parametrize("name", KERNELS)
def test_mid_kernel_keeps_accumulators_in_place(mid_asm, name):
    """No spills and no accumulator copies inside the main loop (the point of the AGPR pinning)."""
    m = re.search(r"^" + re.escape(name) + r":(.*?)s_endpgm", mid_asm, re.S | re.M)
    body = m.group(1)
    assert "scratch_" not in body
    head = body.index("Loop Header")
    loop = body[head:]
    loop = loop[:loop.index("s_cbranch_scc1")]
    assert "v_accvgpr_read" not in loop and "v_accvgpr_mov" not in loop
