"""Wait-state hazards in the gfx950 code of every kernel source, read from the
assembly hipcc writes for it (the same flags as the library build).

On CDNA a vector-ALU instruction that writes a scalar register (v_readfirstlane,
v_readlane, v_cmp into an SGPR pair, a carry out) must be followed by 5 wait
states before a vector memory instruction reads that register (as a buffer
descriptor, an offset or a base), and by 4 before v_readlane / v_writelane use
it as the lane select; the hardware does not interlock these.  The compiler's
hazard recognizer inserts the wait states for the instructions it generates,
but an instruction inside inline asm is opaque to it, so whatever the scheduler
places after such an instruction is unprotected unless the asm block pads
itself.  These tests walk every control-flow path (fall-through and branch
targets) from each such write:

* after a write inside inline asm, no vector-memory, vector-ALU or lane-select
  read of the register within 5 wait states;
* after any vector-ALU write of a scalar register, no vector-memory read of it
  within 5 wait states and no lane-select use within 4.

The checker is itself checked on planted sequences.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from frame_wise_delta_02_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]
WAIT = 5          # VALU writes SGPR -> VMEM reads it
LANE_SELECT = 4   # VALU writes SGPR -> v_readlane / v_writelane lane select

_VMEM = re.compile(r"^(buffer_|global_|flat_|scratch_)")
_LABEL = re.compile(r"^(\.LBB\w+):")


def _sregs(text: str) -> set[int]:
    out: set[int] = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _operands(inst: str) -> tuple[str, list[str]]:
    op = inst.split()[0]
    return op, [o.strip() for o in inst[len(op):].split(",")] if inst[len(op):].strip() else []


def _valu_sgpr_writes(inst: str) -> set[int]:
    op, ops = _operands(inst)
    if not op.startswith("v_") or not ops:
        return set()
    w = _sregs(ops[0]) if not ops[0].startswith("v") else set()
    if len(ops) > 1 and any(k in op for k in ("_co_", "div_scale", "mad_u64_u32", "mad_i64_i32")):
        w |= _sregs(ops[1])
    return w


def _instructions(asm: str):
    """(line index, instruction text, inside inline asm) for every line, plus
    the label table; comments and directives come back as empty text."""
    rows, labels, in_asm = [], {}, False
    for i, line in enumerate(asm.splitlines()):
        if "ASMSTART" in line:
            in_asm = True
        elif "ASMEND" in line:
            in_asm = False
        m = _LABEL.match(line)
        if m:
            labels[m.group(1)] = i
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            t = ""
        rows.append((i, t, in_asm))
    return rows, labels


def hazards(asm: str) -> list[str]:
    """Every read of a VALU-written scalar register that comes too soon."""
    rows, labels = _instructions(asm)
    found = []
    for i, inst, in_asm in rows:
        if not inst:
            continue
        regs = _valu_sgpr_writes(inst)
        if not regs:
            continue
        stack, seen = [(i + 1, 0)], set()
        while stack:
            j, ws = stack.pop()
            while j < len(rows) and ws < WAIT:
                if (j, ws) in seen:
                    break
                seen.add((j, ws))
                _, u, _ = rows[j]
                j += 1
                if not u:
                    continue
                op, ops = _operands(u)
                reads = _sregs(",".join(ops[1:])) if ops else set()  # a VALU's sources
                if _VMEM.match(op) and regs & _sregs(",".join(ops)):
                    found.append(f"{inst!r} -> {u!r} after {ws} wait states (vector memory)")
                elif op.startswith(("v_readlane", "v_writelane")) and len(ops) >= 3 and ws < LANE_SELECT \
                        and regs & _sregs(ops[2]):
                    found.append(f"{inst!r} -> {u!r} after {ws} wait states (lane select)")
                elif in_asm and op.startswith("v_") and regs & reads:
                    found.append(f"{inst!r} (inline asm) -> {u!r} after {ws} wait states (vector ALU)")
                ws += int(u.split()[1], 0) + 1 if op == "s_nop" else 1
                if op.startswith("s_cbranch") or op == "s_branch":
                    target = ops[0] if ops else ""
                    if target in labels:
                        stack.append((labels[target] + 1, ws))
                    if op == "s_branch":
                        break
                if op in ("s_endpgm", "s_setpc_b64"):
                    break
    return found


# ---- the checker on planted sequences -----------------------------------------

def _asm(*lines):
    return "\n".join("\t" + l if not l.endswith(":") else l for l in lines) + "\n"


PLANTED = {
    "offset right after an inline-asm readfirstlane": _asm(
        ";;#ASMSTART", "v_readfirstlane_b32 s25, v2", ";;#ASMEND",
        "s_mov_b32 s3, 0", "buffer_load_dwordx4 v[0:3], v4, s[8:11], s25 offen", "s_endpgm"),
    "descriptor word inside an SGPR range": _asm(
        "v_readlane_b32 s10, v7, 3", "s_nop 1", "buffer_load_dword v0, v4, s[8:11], 0 offen", "s_endpgm"),
    "read on the branch target": _asm(
        ";;#ASMSTART", "v_readfirstlane_b32 s4, v1", ";;#ASMEND", "s_cbranch_scc0 .LBB0_2",
        "s_endpgm", ".LBB0_2:", "global_load_dword v0, v1, s[4:5]", "s_endpgm"),
    "lane select": _asm(
        "v_cmp_gt_u32_e64 s[6:7], v1, v2", "v_readlane_b32 s8, v3, s6", "s_endpgm"),
    "vector ALU read after an inline-asm write": _asm(
        ";;#ASMSTART", "v_readfirstlane_b32 s21, v3", ";;#ASMEND", "v_mov_b32_e32 v2, s21", "s_endpgm"),
}

CLEAN = {
    "padded inside the asm block": _asm(
        ";;#ASMSTART", "v_readfirstlane_b32 s25, v2", "s_nop 4", ";;#ASMEND",
        "buffer_load_dwordx4 v[0:3], v4, s[8:11], s25 offen", "s_endpgm"),
    "five instructions between": _asm(
        "v_readfirstlane_b32 s25, v2", "s_mov_b32 s1, 0", "s_mov_b32 s2, 0", "s_mov_b32 s3, 0",
        "s_add_i32 s6, s6, 1", "s_add_i32 s7, s7, 1", "buffer_load_dword v0, v4, s[8:11], s25 offen", "s_endpgm"),
    "scalar ALU read": _asm(
        ";;#ASMSTART", "v_readfirstlane_b32 s24, v2", ";;#ASMEND", "s_add_i32 s24, s24, s4", "s_endpgm"),
    "another register": _asm(
        "v_readfirstlane_b32 s25, v2", "buffer_load_dword v0, v4, s[8:11], s26 offen", "s_endpgm"),
}


@pytest.mark.parametrize("name", list(PLANTED))
def test_checker_reports_planted_hazard(name):
    assert hazards(PLANTED[name]), name


@pytest.mark.parametrize("name", list(CLEAN))
def test_checker_passes_padded_or_unrelated_reads(name):
    assert not hazards(CLEAN[name]), hazards(CLEAN[name])


# ---- the library's kernels -------------------------------------------------------

def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return open(out).read()


@pytest.fixture(scope="module")
def device_asm():
    if shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(min(len(HIP_SOURCES), 8)) as ex:
            texts = list(ex.map(lambda s: _device_asm(s, d), HIP_SOURCES))
    return dict(zip(HIP_SOURCES, texts))


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_wait_state_hazard_in_kernel_code(device_asm, src):
    asm = device_asm[src]
    assert "s_endpgm" in asm, f"{src}: no kernel code in the assembly"
    found = hazards(asm)
    assert not found, f"{src}: " + "\n".join(found[:10])


def test_inline_asm_scalar_writes_are_padded(device_asm):
    """Every inline-asm v_readfirstlane in the kernels is followed inside its own
    asm block by an s_nop of at least 4 (5 wait states)."""
    n = 0
    for src, asm in device_asm.items():
        rows, _ = _instructions(asm)
        for k, (_, inst, in_asm) in enumerate(rows):
            if in_asm and inst.startswith("v_readfirstlane_b32"):
                n += 1
                nxt = next((u for _, u, a in rows[k + 1:] if u or not a), "")
                assert nxt.startswith("s_nop") and int(nxt.split()[1], 0) >= 4, (src, inst, nxt)
    assert n > 0, "no inline-asm readfirstlane found: the sgpr() helper changed"
