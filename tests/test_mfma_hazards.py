"""Static check of the MFMA kernels' gfx950 assembly (no GPU needed).

A VALU instruction (or a store) that reads an MFMA result must issue enough
wait states after the MFMA; the compiler inserts s_nop for this, and in
straight-line code it keeps at least 8 between a 16x16x32 (or 16x16x16)
bf16 MFMA and the first read of its result.  Its hazard pass has been seen
to under-count when an if-block without an else sits between the MFMA and
the read: it counted only the path through the block, so the path that
jumps over it read a stale accumulator register (wrong results that depend
on timing).  The kernels avoid runtime branches at such points; this test
compiles them to assembly and checks, along the shortest path in layout
order, that every read of an MFMA result reached across a branch is at
least 8 wait states after the MFMA.  It also checks that no inline-assembly
instruction writes a register that an MFMA issued just before still reads as
its accumulator input, over every path into the write, and that no MFMA
reads a register an inline-assembly instruction wrote just before: the
compiler inserts the wait states for both only around its own
instructions.

A third check covers the DPP forms written as inline assembly (the
v_fmac_f32_dpp row broadcasts of the diagonal triangular solve).  A DPP
instruction reads its first source through the lane permutation, and on
gfx9 a VALU write of that VGPR must come at least 2 wait states before the
DPP read.  The compiler inserts them before its own DPP instructions, not
before inline assembly, so the check finds, for every inline DPP
instruction, the last VALU write of its permuted source and requires 2 wait
states in between (a label or branch inside that window is flagged too,
since another path could end in a write there).
"""

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc")
SOURCES = ["chunk_fwd_bf16.hip", "chunk_fwd_kda.hip"]
MIN_WAIT_STATES = 8
WINDOW = 64          # instructions scanned after each MFMA

_REG = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _assembly(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read().splitlines()


def short_reads(lines, min_ws=MIN_WAIT_STATES):
    """(mfma line, reader line, wait states) for reads of an MFMA result
    reached across a branch with fewer than min_ws wait states on the
    shortest layout-order path."""
    found = []
    inf = 10 ** 6
    for i, line in enumerate(lines):
        s = line.strip()
        if not s.startswith("v_mfma"):
            continue
        dst = _vregs(s.split()[1])
        ws, crossed, pending = 0, False, {}
        for j in range(i + 1, min(i + 1 + WINDOW, len(lines))):
            t = lines[j].strip()
            if t.startswith(".LBB") and t.endswith(":"):
                ws = min(ws, pending.pop(t[:-1], inf))
                continue
            if not t or t.startswith((";", ".")):
                continue
            if t.startswith("s_endpgm"):
                break
            if t.startswith(("s_cbranch", "s_branch")):
                crossed = True
                label = t.split()[1]
                pending[label] = min(pending.get(label, inf), ws + 1)
                ws = inf if t.startswith("s_branch") else ws + 1
                continue
            if t.startswith("s_nop"):
                ws += int(t.split()[1]) + 1
                continue
            parts = t.split(None, 1)
            if len(parts) == 2:
                ops = parts[1]
                if t.startswith("v_mfma"):
                    if _vregs(ops.split(",", 1)[1]) & dst:
                        break       # an accumulator chain: not a VALU read
                elif t.startswith(("ds_write", "buffer_store", "global_store")):
                    if _vregs(ops) & dst:
                        if crossed and ws < min_ws:
                            found.append((i + 1, j + 1, ws))
                        break
                elif t.startswith("v_") and "," in ops:
                    if _vregs(ops.split(",", 1)[1]) & dst:
                        if crossed and ws < min_ws:
                            found.append((i + 1, j + 1, ws))
                        break
            ws += 1
    return found


# A VALU write of a register that an in-flight 16x16x32 (or 16x16x16) bf16
# MFMA reads as its accumulator input needs 3 wait states after the MFMA on
# gfx950: the compiler's own code for these kernels keeps exactly 3 (an
# s_nop 2 where nothing else fills them); the scan asks for 4.
ACC_WAR_WAIT_STATES = 4
# an MFMA may read a VALU result 2 wait states after it is written (the
# compiler's own code keeps 2)
VALU_MFMA_RAW_WAIT_STATES = 2


def _branch_sources(lines):
    """label -> indices of the branch instructions that jump to it"""
    out = {}
    for i, line in enumerate(lines):
        t = line.strip()
        if t.startswith(("s_cbranch", "s_branch")):
            out.setdefault(t.split()[1], []).append(i)
    return out


def _falls_through_into(lines, i):
    """whether the instruction before line i (a label) can fall through to it"""
    k = i - 1
    while k >= 0:
        t = lines[k].strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            return not t.startswith(("s_branch", "s_endpgm", "s_setpc"))
        if t.endswith(":") and not t.startswith(";"):
            return True
        k -= 1
    return False


def asm_writes_after_mfma(lines, min_ws=ACC_WAR_WAIT_STATES):
    """(mfma line, asm line, wait states) where an inline-assembly instruction
    writes a VGPR that an MFMA reads as its accumulator input fewer than
    min_ws wait states earlier, on any path into the write (fall-through and
    every branch to each label crossed, walked backwards).  The compiler
    protects that read only from its own instructions.  The first operand of
    each instruction in an inline block is taken as its destination."""
    found = []
    sources = _branch_sources(lines)
    inside = False
    for j, line in enumerate(lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        if not inside or not s.startswith("v_"):
            continue
        parts = s.split(None, 1)
        if len(parts) < 2:
            continue
        dst = _vregs(parts[1].split(",")[0])
        stack, seen, near = [(j - 1, 0)], set(), {}
        while stack:
            i, ws = stack.pop()
            while i >= 0 and ws < min_ws and (i, ws) not in seen:
                seen.add((i, ws))
                t_ = lines[i].strip()
                if t_.endswith(":") and not t_.startswith(";"):
                    stack.extend((b, ws) for b in sources.get(t_[:-1], []))
                    if not _falls_through_into(lines, i):
                        break
                elif t_ and not t_.startswith((";", ".")):
                    if t_.startswith("s_endpgm"):
                        break
                    if t_.startswith("v_mfma"):
                        ops = t_.split(None, 1)[1].split(",")
                        if len(ops) >= 4 and _vregs(ops[3]) & dst:
                            near[i + 1] = min(near.get(i + 1, ws), ws)
                    ws += int(t_.split()[1]) + 1 if t_.startswith("s_nop") else 1
                i -= 1
        found.extend((m, j + 1, w) for m, w in sorted(near.items()))
    return found


def _labels(lines):
    return {l.strip()[:-1]: i for i, l in enumerate(lines)
            if l.strip().endswith(":") and not l.strip().startswith(";")}


def mfma_reads_after_asm_write(lines, min_ws=VALU_MFMA_RAW_WAIT_STATES):
    """(asm line, mfma line, wait states) where an MFMA reads a VGPR that an
    inline-assembly instruction wrote fewer than min_ws wait states before,
    on any path out of the write (fall-through and branch targets, walked
    forwards until the register is written again)."""
    found = []
    labels = _labels(lines)
    inside = False
    for j, line in enumerate(lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        if not inside or not s.startswith("v_"):
            continue
        parts = s.split(None, 1)
        if len(parts) < 2:
            continue
        dst = _vregs(parts[1].split(",")[0])
        stack, seen = [(j + 1, 0)], set()
        while stack:
            i, ws = stack.pop()
            while i < len(lines) and ws < min_ws and (i, ws) not in seen:
                seen.add((i, ws))
                t_ = lines[i].strip()
                if not t_ or t_.startswith((";", ".")) or t_.endswith(":"):
                    i += 1
                    continue
                if t_.startswith("s_endpgm"):
                    break
                if t_.startswith("v_mfma"):
                    ops = t_.split(None, 1)[1].split(",")
                    if any(_vregs(o) & dst for o in ops[1:]):
                        found.append((j + 1, i + 1, ws))
                        break
                if t_.startswith(("s_cbranch", "s_branch")):
                    tgt = labels.get(t_.split()[1])
                    if tgt is not None:
                        stack.append((tgt + 1, ws + 1))
                    if t_.startswith("s_branch"):
                        break
                elif t_.startswith("v_") and len(t_.split(None, 1)) == 2 and \
                        _vregs(t_.split(None, 1)[1].split(",")[0]) >= dst:
                    break       # written again
                ws += int(t_.split()[1]) + 1 if t_.startswith("s_nop") else 1
                i += 1
    return found


DPP_MIN_WAIT_STATES = 2


def dpp_reads_after_valu_write(lines, min_ws=DPP_MIN_WAIT_STATES):
    """(writer line, dpp line, wait states) where an inline-assembly DPP
    instruction reads its permuted source fewer than min_ws wait states
    after a VALU write of that register (writer line None: a label or branch
    came first, so the window is not known to be clear)."""
    found = []
    inside = False
    for j, line in enumerate(lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            inside = True
            continue
        if s.startswith(";;#ASMEND"):
            inside = False
            continue
        if not inside or not s.startswith("v_") or "_dpp" not in s.split()[0]:
            continue
        ops = s.split(None, 1)[1].split(",")
        if len(ops) < 2:
            continue
        src = _vregs(ops[1])          # src0: the operand the DPP control permutes
        ws = 0
        for i in range(j - 1, max(j - 1 - WINDOW, -1), -1):
            if ws >= min_ws:
                break
            t_ = lines[i].strip()
            if not t_ or t_.startswith((";", ".")):
                continue
            if t_.startswith(("s_cbranch", "s_branch")) or t_.endswith(":"):
                found.append((None, j + 1, ws))
                break
            if t_.startswith("s_nop"):
                ws += int(t_.split()[1]) + 1
                continue
            if t_.startswith("v_"):
                parts = t_.split(None, 1)
                if len(parts) == 2 and _vregs(parts[1].split(",")[0]) & src:
                    found.append((i + 1, j + 1, ws))
                    break
            ws += 1
    return found


def test_scanner_flags_a_dpp_read_right_after_a_valu_write():
    lines = """
    v_mul_f32_e32 v40, v41, v42
    ;;#ASMSTART
    v_fmac_f32_dpp v10, v40, v11 row_newbcast:3 row_mask:0xf bank_mask:0xf
    ;;#ASMEND
""".splitlines()
    assert [f[2] for f in dpp_reads_after_valu_write(lines)] == [0]
    # two wait states in between, a write of the other (unpermuted) source,
    # or a load (not a VALU write) are fine
    assert dpp_reads_after_valu_write(lines[:2] + ["    s_nop 1"] + lines[2:]) == []
    assert dpp_reads_after_valu_write([l.replace("v40, v41", "v11, v41") for l in lines]) == []
    assert dpp_reads_after_valu_write(
        [l.replace("v_mul_f32_e32 v40, v41, v42", "ds_read_b32 v40, v41") for l in lines]) == []
    # one unrelated instruction is one wait state: still short
    one = lines[:2] + ["    v_add_f32_e32 v50, v51, v52"] + lines[2:]
    assert [f[2] for f in dpp_reads_after_valu_write(one)] == [1]


def test_scanner_flags_an_asm_write_of_an_mfma_accumulator_input():
    lines = """
    v_mfma_f32_16x16x32_bf16 v[12:15], v[162:165], v[56:59], v[142:145]
    ;;#ASMSTART
    v_dot2_f32_bf16 v142, v154, s23, v170
    ;;#ASMEND
""".splitlines()
    assert len(asm_writes_after_mfma(lines)) == 1
    # far enough after the MFMA, or writing another register, it is fine
    late = lines[:2] + ["    s_nop 3"] + lines[2:]
    assert asm_writes_after_mfma(late) == []
    other = [l.replace("v142,", "v150,") for l in lines]
    assert asm_writes_after_mfma(other) == []
    # a later MFMA in between does not hide the earlier one
    two = lines[:2] + ["    v_mfma_f32_16x16x32_bf16 v[20:23], v[2:5], v[6:9], v[20:23]"] + lines[2:]
    assert len(asm_writes_after_mfma(two)) == 1


def test_scanner_flags_an_mfma_read_right_after_an_asm_write():
    lines = """
    ;;#ASMSTART
    v_cvt_pk_bf16_f32 v40, v41, v42
    ;;#ASMEND
    v_mfma_f32_16x16x32_bf16 v[12:15], v[162:165], v[40:43], v[12:15]
""".splitlines()
    assert [f[2] for f in mfma_reads_after_asm_write(lines)] == [0]
    padded = lines[:4] + ["    s_nop 1"] + lines[4:]
    assert mfma_reads_after_asm_write(padded) == []
    # a write of another register in between is not a read of v40
    other = [l.replace("v[40:43]", "v[44:47]") for l in lines]
    assert mfma_reads_after_asm_write(other) == []


def test_scanner_follows_branches_into_an_asm_write():
    # the write sits at a loop head: the path from the back edge ends in an
    # MFMA that reads v142 as its accumulator input
    lines = """
    s_branch .LBB0_2
.LBB0_1:
    v_mfma_f32_16x16x32_bf16 v[12:15], v[162:165], v[56:59], v[142:145]
    s_cbranch_scc1 .LBB0_3
.LBB0_2:
    s_mov_b32 s4, 0
    ;;#ASMSTART
    v_dot2_f32_bf16 v142, v154, s23, v170
    ;;#ASMEND
    s_branch .LBB0_1
.LBB0_3:
    s_endpgm
""".splitlines()
    assert [f[2] for f in asm_writes_after_mfma(lines)] == [2]
    # padded on the back-edge path it is fine
    fixed = [l.replace("s_cbranch_scc1 .LBB0_3", "s_nop 7\n    s_nop 7\n    s_nop 7\n    s_cbranch_scc1 .LBB0_3")
             for l in lines]
    assert asm_writes_after_mfma("\n".join(fixed).splitlines()) == []


def test_scanner_flags_a_read_that_skips_an_if_block():
    # the shape the check exists for: the MFMA result v6 is read two
    # instructions after the MFMA on the path that jumps over the block
    lines = """
    v_mfma_f32_16x16x32_bf16 v[6:9], v[14:17], v[14:17], v[6:9]
    s_cbranch_vccnz .LBB0_2
    ds_read_b128 v[14:17], v14 offset:19712
    v_mul_f32_e32 v2, v2, v14
    v_mul_f32_e32 v3, v3, v15
    v_mul_f32_e32 v4, v4, v16
    v_mul_f32_e32 v5, v5, v17
    v_mul_f32_e32 v2, v2, v18
    v_mul_f32_e32 v3, v3, v18
    v_mul_f32_e32 v4, v4, v18
.LBB0_2:
    ds_read_b128 v[14:17], v12 offset:4096
    v_mul_f32_e32 v2, v6, v2
""".splitlines()
    assert [f[2] for f in short_reads(lines)] == [2]
    # enough wait states before the branch cover both paths
    mfma = next(i for i, l in enumerate(lines) if "v_mfma" in l)
    padded = lines[:mfma + 1] + ["    s_nop 7"] + lines[mfma + 1:]
    assert short_reads(padded) == []
    # so does a read inside the block, whose only way in is from the MFMA
    inside = lines[:mfma + 2] + ["    s_nop 6", "    v_mul_f32_e32 v2, v6, v2"] + lines[mfma + 2:]
    assert short_reads(inside) == []


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_mfma_results_are_not_read_early_across_branches():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            asm = dict(zip(SOURCES, ex.map(lambda s: _assembly(s, tmp), SOURCES)))
    problems = {src: short_reads(lines)[:5] for src, lines in asm.items()}
    assert all(not p for p in problems.values()), problems
    asm_problems = {src: asm_writes_after_mfma(lines)[:5] for src, lines in asm.items()}
    assert all(not p for p in asm_problems.values()), asm_problems
    raw_problems = {src: mfma_reads_after_asm_write(lines)[:5] for src, lines in asm.items()}
    assert all(not p for p in raw_problems.values()), raw_problems
    dpp_problems = {src: dpp_reads_after_valu_write(lines)[:5] for src, lines in asm.items()}
    assert all(not p for p in dpp_problems.values()), dpp_problems
    # the scan saw the solve's inline DPP instructions (it is not vacuous)
    for src, lines in asm.items():
        assert sum("v_fmac_f32_dpp" in l for l in lines) >= 120, src
