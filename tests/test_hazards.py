"""The matrix-core operand hazard, checked in the device assembly of this library's own build.

A VALU result needs two wait states before a matrix-core (MFMA) instruction reads it as an
operand.  The compiler inserts them for the code it schedules, but it does not see what an
inline-asm statement writes, and the P operands of the P V products come from inline-asm
v_fma_mix instructions (kvq_attn_block.h, kvq_prefill.hip), protected by a hand-placed s_nop.
This test compiles the attention kernels to gfx950 assembly with the library's own flags and
walks every kernel in layout order: each MFMA's A, B and C registers must have been written by
a VALU instruction at least two wait states earlier (an instruction issued counts one, s_nop N
counts N + 1).  It runs on the CPU; only hipcc is needed.

Control flow: besides the text in order (the fall-through paths), every branch's taken path is
walked as well, the instructions up to the branch followed by those at its target, so a write
before a loop's back-edge is checked against the reads at the loop's head.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from long_context_decode_flash_amd import build as B

WAIT_STATES = 2

_REG = re.compile(r"\b([vas])(\d+)\b|\b([vas])\[(\d+):(\d+)\]")


def _regs(operand: str, kind: str = "v") -> set[int]:
    out = set()
    for m in _REG.finditer(operand):
        if m.group(1):
            if m.group(1) == kind:
                out.add(int(m.group(2)))
        elif m.group(3) == kind:
            out.update(range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _split_operands(text: str) -> list[str]:
    # operands are comma-separated; register ranges contain ':' but no ','
    return [t.strip() for t in text.split(",") if t.strip()]


def kernels(asm: str) -> dict[str, list[str]]:
    """Instruction lines of every function in an assembly listing, labels kept as ('label:')."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        body = []
        for line in asm[m.end():end].splitlines():
            t = line.split(";")[0].strip() if not line.strip().startswith(";;#") else ""
            if not t or t.startswith("."):
                if re.match(r"^\.LBB\S+:", line.strip()):
                    body.append(line.strip().split()[0])
                continue
            body.append(t)
        out[name] = body
    return out


def violations(lines: list[str], need: int = WAIT_STATES) -> list[tuple[int, str, str, int]]:
    """(index, writer, reader, wait states) for every MFMA operand read too soon after a VALU
    write of one of its registers, in layout order."""
    last_write: dict[int, tuple[int, str]] = {}  # vgpr -> (issue clock after the write, writer)
    clock = 0
    found = []
    for i, t in enumerate(lines):
        if t.endswith(":"):
            continue  # a label issues nothing
        op, _, rest = t.partition(" ")
        ops = _split_operands(rest)
        if op.startswith("v_mfma"):
            srcs = set()
            for o in ops[1:4]:
                srcs |= _regs(o)
            for r in srcs:
                if r in last_write:
                    at, writer = last_write[r]
                    if clock - at < need:
                        found.append((i, writer, t, clock - at))
        if op == "s_nop":
            clock += int(rest.strip(), 0) + 1
            continue
        clock += 1
        if op.startswith("v_") and not op.startswith("v_mfma") and ops:
            written = _regs(ops[0])
            if "_swap_" in op and len(ops) > 1:  # the permlane swaps write both operands
                written |= _regs(ops[1])
            for r in written:
                last_write[r] = (clock, t)
    return found


def all_violations(lines: list[str], need: int = WAIT_STATES, window: int = 8):
    """violations() on the fall-through order and on every branch's taken path: the `window`
    instructions up to and including the branch, then the instructions at its target (the
    hazard spans two wait states, so a few instructions either side decide it)."""
    found = [(writer, reader, ws) for _, writer, reader, ws in violations(lines, need)]
    labels = {t[:-1]: i for i, t in enumerate(lines) if t.endswith(":")}
    for i, t in enumerate(lines):
        op, _, rest = t.partition(" ")
        if not (op.startswith("s_cbranch") or op == "s_branch"):
            continue
        target = rest.strip().split()[0] if rest.strip() else ""
        if target not in labels:
            continue
        before = [x for x in lines[max(0, i - window):i + 1] if not x.endswith(":")]
        after = lines[labels[target]:labels[target] + 4 * window]
        for k, writer, reader, ws in violations(before + after, need):
            if k >= len(before):
                found.append((writer, reader, ws))
    return found


def _assemble(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".s"))
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC,
           "-o", out, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and not shutil.which(B.HIPCC):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    return {f: open(_assemble(os.path.join(B.CSRC, f), d)).read() for f in ("kvq_decode.hip", "kvq_prefill.hip")}


def test_checker_finds_a_planted_hazard():
    lines = ["v_fma_mixlo_f16 v10, v1, v2, 0", "v_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]"]
    assert violations(lines) and violations(lines)[0][3] == 0
    assert violations(["v_fma_mixlo_f16 v10, v1, v2, 0", "s_nop 0",
                       "v_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]"])
    assert not violations(["v_fma_mixlo_f16 v10, v1, v2, 0", "s_nop 1",
                           "v_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]"])
    assert not violations(["v_fma_mixlo_f16 v10, v1, v2, 0", "v_add_u32_e32 v3, v4, v5", "s_add_i32 s1, s1, 1",
                           "v_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]"])
    # a taken branch counts as one wait state: a write before a loop's back-edge meets the read
    # at the loop's head
    loop = [".LBB0_1:", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0", "v_add_u32_e32 v1, v1, v2",
            "s_nop 4", "v_fma_mixlo_f16 v5, v1, v2, 0", "s_cbranch_scc1 .LBB0_1"]
    assert not violations(loop) and all_violations(loop)
    # a register range, the C operand and a swap's second operand all count
    assert violations(["v_mov_b32_e32 v22, 0", "v_mfma_f32_16x16x32_f16 v[20:23], v[4:7], v[8:11], v[20:23]"])
    assert violations(["v_permlane16_swap_b32_e32 v3, v5", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0"])
    assert not violations(["v_mov_b32_e32 v40, 0", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0"])


@pytest.mark.parametrize("src", ["kvq_decode.hip", "kvq_prefill.hip"])
def test_mfma_operands_have_their_wait_states(listings, src):
    ks = kernels(listings[src])
    checked = 0
    bad = []
    for name, lines in ks.items():
        n = sum(1 for t in lines if t.startswith("v_mfma"))
        if not n:
            continue
        checked += n
        for writer, reader, ws in all_violations(lines):
            bad.append(f"{name[:60]}: {writer!r} -> {reader!r} after {ws} wait states")
    assert checked > 100, f"{src}: only {checked} MFMA instructions found"
    assert not bad, "\n".join(bad[:20])


def test_checker_sees_the_nop_taken_out(tmp_path):
    """The same check on a copy of the sources with the hand-placed nop of the decode's P V step
    removed (compiled only, never run): the checker then finds MFMAs that read a P half one wait
    state after its inline-asm v_fma_mix write, the stale read the nop prevents.  (Which kernels
    depend on the nop is the schedule's business: with these sources 16 of the 18 one-row-block
    kernels do; in the two-row-block kernels the second row block's P split and the V operands'
    own work fall between the first P writes and the first product, and the nop is a guard.)"""
    if not os.path.exists(B.HIPCC) and not shutil.which(B.HIPCC):
        pytest.skip("hipcc not available")
    src = tmp_path / "csrc"
    shutil.copytree(B.CSRC, src)
    hdr = src / "kvq_attn_block.h"
    text = hdr.read_text()
    text, n = re.subn(r'asm\("s_nop 1"[^;]*;', ";", text)
    assert n == 1
    hdr.write_text(text)
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")]
    out = str(tmp_path / "dec.s")
    res = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"),
                          "-I", str(src), "-o", out, str(src / "kvq_decode.hip")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    ks = kernels(open(out).read())
    found = {k: all_violations(v) for k, v in ks.items() if "decode_kernel" in k}
    flagged = {k: v for k, v in found.items() if v}
    assert flagged, "no decode kernel reads a P half too early without the nop"
    writers = {w.split()[0] for v in flagged.values() for w, _, _ in v}
    assert writers <= {"v_fma_mixlo_f16", "v_fma_mixhi_f16"}, writers
