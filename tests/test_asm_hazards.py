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


def lds_load_hazards(asm: str):
    """(kernel, wait states, load) for every LDS-direct buffer load reading an
    SGPR written by a VALU op fewer than WAIT_STATES wait states before, in
    straight-line code (history restarts at each label)."""
    found = []
    kernel = None
    hist = []  # (wait states the instruction takes, SGPRs written by a VALU op)
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kernel, hist = m.group(1), []
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")):
            continue
        if t.endswith(":"):
            hist = []
            continue
        op = t.split()[0]
        if op.startswith("buffer_load") and re.search(r"\slds\b", t):
            srd = _sgprs(t.split(",")[1]) if "," in t else set()
            waits = 0
            for n, written in reversed(hist):
                if written & srd:
                    if waits < WAIT_STATES:
                        found.append((kernel, waits, t))
                    break
                waits += n
                if waits >= WAIT_STATES:
                    break
        n = 1
        mm = re.match(r"s_nop\s+(\d+)", t)
        if mm:
            n = int(mm.group(1)) + 1
        written = set()
        if op.startswith("v_"):
            operands = t[len(op):].split(",")
            if operands and re.match(r"\s*s(\[|\d)", operands[0]):
                written = _sgprs(operands[0])
        hist.append((n, written))
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


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None,
                    reason="hipcc not available")
def test_gemm_kernels_have_no_valu_sgpr_hazard(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    src = os.path.join(buildlib.PKG, "csrc", "moe_gemm.hip")
    out = tmp_path / "moe_gemm.s"
    flags = [f for f in buildlib.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "-I", os.path.join(buildlib.ROOT, "include"), "-I",
           os.path.join(buildlib.PKG, "csrc"), "-S", "--cuda-device-only", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert re.search(r"\slds\b", asm), "no LDS-direct loads found in the assembly"
    found = lds_load_hazards(asm)
    assert not found, "\n".join(f"{k}: {w} wait states before {t}" for k, w, t in found[:10])
