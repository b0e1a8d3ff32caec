"""The LDS-direct loads of the GEMM kernels are written as inline asm, so the
compiler's hazard handling does not see them. This test compiles the kernels
to gfx950 assembly (no GPU needed) and checks the one hazard that applies to
them: a vector memory instruction that reads an SGPR written by a VALU op
(v_readlane, v_readfirstlane, a VOPC with an SGPR result, ...) needs 5 wait
states in between on gfx9. A descriptor restored from VGPR lanes right before
such a load would be read stale."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_expert_ffn_amd import buildlib

WAIT_STATES = 5


def _sgprs(text):
    regs = set()
    for a, b in re.findall(r"\bs\[(\d+):(\d+)\]", text):
        regs.update(range(int(a), int(b) + 1))
    for a in re.findall(r"\bs(\d+)\b", text):
        regs.add(int(a))
    return regs


def _blocks(body: str):
    """Basic blocks of one kernel's assembly: [(label or None, [instruction])]."""
    blocks = [[None, []]]
    for line in body.split("\n"):
        t = line.strip()
        if re.match(r"^[.\w$]+:", t):  # a label (.LBB0_1: and the like)
            blocks.append([t.split(":")[0], []])
            continue
        t = t.split(";")[0].strip()
        if not t or t.startswith("."):
            continue
        blocks[-1][1].append(t)
        op = t.split()[0]
        if op in ("s_branch", "s_endpgm", "s_setpc_b64") or op.startswith("s_cbranch"):
            blocks.append([None, []])  # a branch ends its block
    return blocks


def _effect(t: str):
    """(wait states the instruction takes, SGPRs it writes if it is a VALU op)."""
    op = t.split()[0]
    n = 1
    mm = re.match(r"s_nop\s+(\d+)", t)
    if mm:
        n = int(mm.group(1)) + 1
    written = set()
    if op.startswith("v_"):
        operands = t[len(op):].split(",")
        if operands and re.match(r"\s*s(\[|\d)", operands[0]):
            written = _sgprs(operands[0])
    return n, written


def _kernel_hazards(kernel: str, body: str):
    blocks = _blocks(body)
    index = {lab: i for i, (lab, _) in enumerate(blocks) if lab}
    preds = {i: set() for i in range(len(blocks))}
    for i, (_, ins) in enumerate(blocks):
        for t in ins:
            op = t.split()[0]
            if op == "s_branch" or op.startswith("s_cbranch"):
                target = t.split()[1]
                if target in index:
                    preds[index[target]].add(i)
        last = ins[-1].split()[0] if ins else None
        if last not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            preds[i + 1].add(i)

    def fewest(bi, end, srd, budget, seen):
        """Fewest wait states between a VALU write of srd and instruction
        `end` of block bi over every path into it, or None if none within
        budget."""
        ins = blocks[bi][1]
        w = 0
        for k in range(end - 1, -1, -1):
            n, written = _effect(ins[k])
            if written & srd:
                return w
            w += n
            if w >= budget:
                return None
        best = None
        for p in preds[bi]:
            if (p, budget - w) in seen:
                continue
            seen.add((p, budget - w))
            r = fewest(p, len(blocks[p][1]), srd, budget - w, seen)
            if r is not None and (best is None or r + w < best):
                best = r + w
        return best

    found = []
    for bi, (_, ins) in enumerate(blocks):
        for k, t in enumerate(ins):
            if t.startswith("buffer_load") and re.search(r"\slds\b", t) and "," in t:
                r = fewest(bi, k, _sgprs(t.split(",")[1]), WAIT_STATES, set())
                if r is not None and r < WAIT_STATES:
                    found.append((kernel, r, t))
    return found


def lds_load_hazards(asm: str):
    """(kernel, wait states, load) for every LDS-direct buffer load reading an
    SGPR written by a VALU op fewer than WAIT_STATES wait states before, over
    every path into the load: straight-line code, code that falls through
    into a label, and branches (forward and loop back-edges) to it."""
    found = []
    heads = list(re.finditer(r"^(_Z\S+):", asm, re.M))
    for n, m in enumerate(heads):
        end = heads[n + 1].start() if n + 1 < len(heads) else len(asm)
        found += _kernel_hazards(m.group(1), asm[m.end():end])
    return found


def test_scanner_catches_the_pattern():
    asm = """_Zk:
\tv_readlane_b32 s4, v184, 15
\tv_readlane_b32 s7, v184, 18
\tbuffer_load_dwordx4 v4, s[4:7], 0 offen lds
\tv_readlane_b32 s7, v184, 18
\ts_nop 4
\tbuffer_load_dword v2, s[4:7], 0 offen lds
"""
    found = lds_load_hazards(asm)
    assert len(found) == 1 and found[0][1] == 0


def test_scanner_follows_fall_through():
    """A VALU write of an SGPR at the end of one block, then a label that the
    code falls through into, then the load: still a hazard. After an
    unconditional branch the label starts a new path."""
    asm = """_Zk:
\tv_readfirstlane_b32 s8, v3
.LBB0_1:
\tbuffer_load_dwordx4 v4, s[8:11], 0 offen lds
\ts_branch .LBB0_3
\tv_readfirstlane_b32 s12, v3
\ts_branch .LBB0_1
.LBB0_2:
\tbuffer_load_dwordx4 v4, s[12:15], 0 offen lds
.LBB0_3:
\ts_endpgm
"""
    found = lds_load_hazards(asm)
    assert len(found) == 1 and "s[8:11]" in found[0][2] and found[0][1] == 0


def test_scanner_follows_branches_and_back_edges():
    """A loop whose last instructions write the descriptor with a VALU op and
    branch back to a load at the loop head; a forward branch from right after
    such a write to a load."""
    asm = """_Zk:
\ts_mov_b32 s4, 0
.LBB0_1:
\tbuffer_load_dwordx4 v4, s[4:7], 0 offen lds
\ts_nop 7
\tv_readlane_b32 s5, v9, 1
\ts_cbranch_scc1 .LBB0_1
\tv_readfirstlane_b32 s12, v3
\ts_cbranch_vccz .LBB0_3
\ts_nop 7
\ts_branch .LBB0_4
.LBB0_3:
\tbuffer_load_dwordx4 v4, s[12:15], 0 offen lds
.LBB0_4:
\ts_endpgm
"""
    found = sorted(lds_load_hazards(asm), key=lambda f: f[2])
    assert [(w, t.split(",")[1].strip()) for _, w, t in found] == [(1, "s[12:15]"),
                                                                    (1, "s[4:7]")]


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None,
                    reason="hipcc not available")
@pytest.mark.parametrize("source,variant", [("moe_gemm.hip", "plain"), ("moe_gemm.hip", "trace"),
                                            ("moe_gemm.hip", "mfma32"), ("moe_gemm.hip", "a64"),
                                            ("moe_mx.hip", "plain"), ("moe_mx.hip", "trace")])
def test_gemm_kernels_have_no_valu_sgpr_hazard(tmp_path, variant, source):
    """Every source with LDS-direct loads, in both library builds (the plain
    one and the one with timing records), and the GEMMs with the 32x32x16
    MFMA core option and with 64-K A stages on every 256-row up/gate tile."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    src = os.path.join(buildlib.PKG, "csrc", source)
    out = tmp_path / "kernels.s"
    flags = [f for f in buildlib.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    if variant == "trace":
        flags += buildlib.TRACE_FLAGS
    elif variant == "mfma32":
        flags += ["-DMOE_MFMA32=1"]
    elif variant == "a64":
        flags += ["-DMOE_A64=2"]
    cmd = [hipcc, *flags, "-I", os.path.join(buildlib.ROOT, "include"), "-I",
           os.path.join(buildlib.PKG, "csrc"), "-S", "--cuda-device-only", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert re.search(r"\slds\b", asm), "no LDS-direct loads found in the assembly"
    found = lds_load_hazards(asm)
    assert not found, "\n".join(f"{k}: {w} wait states before {t}" for k, w, t in found[:10])
