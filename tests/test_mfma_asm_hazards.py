"""The hand-scheduled MFMA phase of the forward kernel (inline asm) against the gfx950 hazard rules.

The compiler inserts wait states for the matrix-core instructions it emits itself, but not for
those written as inline asm. This test builds the forward kernels' gfx950 assembly (CPU only) and
walks every inline-asm MFMA:
  * no later instruction other than an MFMA accumulating into exactly the same registers may read
    or write the MFMA's destination registers within 20 wait states (a 16-pass XDL result read by
    the VALU, memory or another MFMA's A/B operand needs passes + 4 on gfx950), and the window
    may not run into a branch;
  * no VALU instruction in the 2 wait states before the MFMA may write one of its source registers.
An s_nop N counts N + 1 wait states, any other instruction 1.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_forward_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
XDL_WRITE_WAIT_STATES = 20
VALU_WRITE_MFMA_READ_WAIT_STATES = 2

REG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def operands(text):
    """Register sets of the comma-separated operands of one instruction."""
    parts = text.split(None, 1)
    if len(parts) < 2:
        return []
    return [regs(op) for op in re.split(r",(?![^\[]*\])", parts[1])]


def instructions(func_text):
    """(text, from_inline_asm) for every instruction of one function, in order."""
    out, in_asm = [], False
    for ln in func_text.splitlines():
        t = ln.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        for piece in t.split("\\n"):
            piece = piece.strip()
            if piece:
                out.append((piece, in_asm))
    return out


def wait_states(instr):
    m = re.match(r"s_nop\s+(\d+)", instr)
    return int(m.group(1)) + 1 if m else 1


@pytest.fixture(scope="module")
def forward_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "fwd_mfma.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           os.path.join(CSRC, "fwd_mfma.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    funcs = re.split(r"\n(?=_Z\S*fwd_mfma_kernel\S*:)", text)
    return [f for f in funcs if re.match(r"_Z\S*fwd_mfma_kernel\S*:", f)]


def test_every_forward_kernel_variant_was_found(forward_asm):
    # head dim {64, 128} x dtype {bf16, fp16} x {sum-checked, running max} x {causal, not}
    assert len(forward_asm) == 16


def test_inline_asm_mfma_results_are_not_touched_inside_the_wait_window(forward_asm):
    checked = 0
    for func in forward_asm:
        name = func.split(":", 1)[0]
        ins = instructions(func)
        for i, (text, from_asm) in enumerate(ins):
            if not (from_asm and text.startswith("v_mfma")):
                continue
            ops = operands(text)
            dst = ops[0]
            ws, j = 0, i + 1
            while ws < XDL_WRITE_WAIT_STATES:
                assert j < len(ins), f"{name}: function ends inside the wait window of '{text}'"
                nxt = ins[j][0]
                assert not re.match(r"s_(c?branch|setpc|endpgm|barrier)", nxt), \
                    f"{name}: '{nxt}' inside the {XDL_WRITE_WAIT_STATES}-wait-state window of '{text}'"
                if nxt.startswith("v_mfma"):
                    nops = operands(nxt)
                    same_acc = nops[0] == dst and nops[3] == dst
                    assert same_acc or not (dst & (nops[0] | nops[1] | nops[2] | nops[3])), \
                        f"{name}: '{nxt}' uses the result of '{text}' after {ws} wait states"
                else:
                    assert not (dst & regs(nxt)), f"{name}: '{nxt}' touches the result of '{text}' after {ws} wait states"
                ws += wait_states(nxt)
                j += 1
            checked += 1
    assert checked >= 4 * 32, checked     # the d = 64 phase: 32 MFMAs in each of its 4 kernel variants


def test_no_valu_write_just_before_an_inline_asm_mfma_reads_it(forward_asm):
    for func in forward_asm:
        name = func.split(":", 1)[0]
        ins = instructions(func)
        for i, (text, from_asm) in enumerate(ins):
            if not (from_asm and text.startswith("v_mfma")):
                continue
            srcs = set().union(*operands(text)[1:])
            ws, j = 0, i - 1
            while ws < VALU_WRITE_MFMA_READ_WAIT_STATES and j >= 0:
                prev = ins[j][0]
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    written = operands(prev)[0] if operands(prev) else set()
                    assert not (written & srcs), f"{name}: '{prev}' writes an operand of '{text}' {ws} wait states before it"
                ws += wait_states(prev)
                j -= 1
