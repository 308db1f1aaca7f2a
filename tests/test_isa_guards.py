"""Compiled-code guard for the one kernel whose LDS reads are inline assembly
with the wait in a separate statement: the heads' hidden-state projection
GEMM issues a stage's operand reads one stage ahead and waits for them later,
so that the compiler does not wait for every direct-to-LDS copy in flight.
That is only safe while the compiler leaves the reads' destination registers
alone until the wait: no compiler-generated instruction between an asm read
and the asm wait after it may read or write them, and the kernel may not
spill (a spill or a copy would take a register whose load is still in flight,
and a register the compiler thought free could be handed to an address).
Compiles the source to gfx950 assembly with hipcc; no GPU is needed."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "semi_autoregressive_block_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _regs(operands):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|\bv(\d+)\b", operands):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _kernel_body(asm, name_part):
    m = re.search(r"^(_Z\S*" + re.escape(name_part) + r"\S*):", asm, re.M)
    assert m, f"{name_part} not found in the assembly"
    end = asm.find(".Lfunc_end", m.end())
    return asm[m.end():end]


def _violations(body):
    """Non-asm instructions that touch a register of an asm ds_read before
    the asm s_waitcnt lgkmcnt(0) that completes it."""
    in_asm, pending, bad = False, set(), []
    for line in body.splitlines():
        t = line.strip()
        if "ASMSTART" in t:
            in_asm = True
            continue
        if "ASMEND" in t:
            in_asm = False
            continue
        if in_asm:
            if t.startswith("ds_read"):
                pending |= _regs(t.split(None, 1)[1].split(",")[0])
            elif t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
                pending = set()
            continue
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        parts = t.split(None, 1)
        if pending and len(parts) > 1 and _regs(parts[1].split(";")[0]) & pending:
            bad.append(t)
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_projection_gemm_asm_reads_keep_their_registers(tmp_path):
    out = tmp_path / "markov_heads.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, "markov_heads.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    body = _kernel_body(out.read_text(), "head_proj_gemm")
    assert "ds_read_b128" in body and "ASMSTART" in body  # the pattern this guards is still there
    assert "scratch_" not in body, "head_proj_gemm spills"
    bad = _violations(body)
    assert not bad, f"{len(bad)} instructions touch in-flight asm read registers, first: {bad[:3]}"


def test_guard_flags_a_touch_before_the_wait():
    """The checker itself: a copy of an in-flight register is flagged, the
    same copy after the asm wait is not."""
    issue = "\t;;#ASMSTART\n\tds_read_b128 v[4:7], v1\n\t;;#ASMEND\n"
    wait = "\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n"
    touch = "\tv_mov_b32_e32 v20, v5\n"
    assert _violations(issue + touch + wait) == ["v_mov_b32_e32 v20, v5"]
    assert _violations(issue + wait + touch) == []
    assert _violations(issue + "\tv_add_u32_e32 v8, v9, v10\n" + wait) == []
