"""Build the HIP library (libmoe.so) for gfx950 in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")  # the build() target (not SPARSE_EXPERT_FFN_LIB)
# the same library with per-task timing records in the persistent kernels
TRACE_LIB = os.path.join(PKG, "libmoe_trace.so")
TRACE_FLAGS = ["-DMOE_TRACE=1"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-munsafe-fp-atomics",
    # keep hipcc from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed to one
    space (string literals kept as they are)."""
    import re
    string = r'"(?:\\.|[^"\\\n])*"'
    keep = lambda m: m.group(0) if m.group(0).startswith('"') else " "
    text = re.sub(string + r'|//[^\n]*|/\*.*?\*/', keep, text, flags=re.S)
    return re.sub(string + r'|\s+', keep, text).strip()


def source_digest() -> str:
    """SHA-256 over what determines the compiled kernels: the code of the HIP
    sources and headers under csrc/ and of the public header (comments and
    layout left out, so a comment edit keeps the digest) and the compiler
    flags. Measurement records (hardware counters) carry it, so that a record
    taken on other kernels is recognised as stale."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + \
        sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    noisy = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noisy and verbose:
        sys.stderr.write("\n".join(noisy) + "\n")


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB) -> str:
    """Each source compiled to an object side by side, then one link."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objdir = os.path.join(ROOT, "_build", os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in sources()]
    cmds = [[hipcc, *flags, *(extra or []), *inc, "-c", src, "-o", o]
            for src, o in zip(sources(), objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"],
         verbose)
    os.replace(out + ".tmp", out)
    return out


def build_trace(verbose: bool = False) -> str:
    return build(verbose=verbose, extra=TRACE_FLAGS, out=TRACE_LIB)


def build_all(verbose: bool = False) -> list[str]:
    """The library and its timing-record variant, compiled side by side."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(2) as ex:
        futs = [ex.submit(build, verbose), ex.submit(build_trace, verbose)]
        return [f.result() for f in futs]


if __name__ == "__main__":
    print(build_all(verbose=True))
