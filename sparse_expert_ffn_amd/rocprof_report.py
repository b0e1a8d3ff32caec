"""rocprofv3 harness for the MoE layer kernels: runs the benchmark under the
profiler passes and turns their CSV output into per-kernel figures.

Passes (each a separate rocprofv3 run of ``bench.py``, so that every counter
group fits the hardware's per-run limits):

  trace   --kernel-trace --stats           per-kernel calls and durations
  fetch   --pmc FETCH_SIZE                 HBM bytes read per dispatch
  write   --pmc WRITE_SIZE                 HBM bytes written per dispatch
  sq      --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE
                SQ_WAVE_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE GRBM_COUNT
                                           matrix-core and LDS utilisation, clock
  cfetch / cwrite  the two byte counters on a plain 1 GiB device copy
                   (``bench.py --copy-calibration``): the scale that turns a
                   counter reading into bytes

Derived figures per kernel (averages over its dispatches):
  - duration (kernel trace);
  - HBM read / write bytes = FETCH_SIZE / WRITE_SIZE (KiB) x 1024 x the copy's
    bytes-per-KiB-reading scale;
  - achieved TFLOP/s and GB/s from the algorithmic counts the caller gives;
  - MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs), cycles =
    GRBM_GUI_ACTIVE / XCDs (the GRBM counters are summed over the XCDs);
  - LDS active / bank-conflict share = counter / (cycles x CUs);
  - waves waiting on instruction issue = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES;
  - effective clock = GRBM_COUNT / XCDs / duration;
  - the cycle shares and the clock only for kernels of MIN_COUNTER_US or more
    (the counter window of a short dispatch is much longer than the kernel).

Usage (from the repository root, on a machine with the GPU):

  python -m sparse_expert_ffn_amd.rocprof_report run --workload prefill_bal --out DIR
  python -m sparse_expert_ffn_amd.rocprof_report report --workload prefill_bal --out DIR \\
      [--md FILE] [--traffic-json FILE]

``run`` starts each pass as a child process under a time limit (the profiler
is the child, the benchmark its program: nothing is exec'd from a process
that holds the GPU) and then writes the report. This module only reads what
the profiler wrote; it does not touch the GPU itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import shlex
import subprocess
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

XCDS = 8
SIMDS = 1024
CUS = 256
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# kernels shorter than this get no cycle-share or clock figures
MIN_COUNTER_US = 50.0

SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
               "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE", "GRBM_COUNT")

PASSES = {
    "trace": ["--kernel-trace", "--stats"],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
    "sq": ["--pmc", *SQ_COUNTERS],
}
CALIBRATION = {"cfetch": ["--pmc", "FETCH_SIZE"], "cwrite": ["--pmc", "WRITE_SIZE"]}


def short_name(kernel: str) -> str:
    """'void moe::upgate_kernel<unsigned short, 256, 128, false>(moe::ForwardParams)'
    -> 'upgate_kernel<unsigned short, 256, 128, false>'."""
    k = kernel.strip()
    k = re.sub(r"^void\s+", "", k)
    depth = 0
    for i, ch in enumerate(k):  # cut the argument list (outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            k = k[:i]
            break
    k = re.sub(r"\bmoe::", "", k)
    return k.strip()


def _col(row: dict, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def _find(dirpath: str, suffix: str):
    files = sorted(glob.glob(os.path.join(dirpath, "**", f"*{suffix}"), recursive=True))
    return files


def read_kernel_trace(dirpath: str):
    """{short kernel name: [duration ns, ...]} from *kernel_trace.csv."""
    out = defaultdict(list)
    for f in _find(dirpath, "kernel_trace.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = short_name(_col(row, "Kernel_Name", "KernelName", "Name"))
                t0 = int(_col(row, "Start_Timestamp", "BeginNs", "Start"))
                t1 = int(_col(row, "End_Timestamp", "EndNs", "End"))
                out[name].append(t1 - t0)
    return dict(out)


def read_counters(dirpath: str):
    """{short kernel name: {counter: [value per dispatch, ...]}, '_dur':
    [ns per dispatch]} from *counter_collection.csv (rows of one dispatch and
    counter are summed: some counters are reported per dimension)."""
    per = defaultdict(float)      # (dispatch, kernel, counter) -> value
    dur = {}                      # (dispatch, kernel) -> ns
    for f in _find(dirpath, "counter_collection.csv"):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = short_name(_col(row, "Kernel_Name", "KernelName", "Name"))
                disp = _col(row, "Dispatch_Id", "Correlation_Id", "Index")
                ctr = _col(row, "Counter_Name", "Counter")
                per[(f, disp, name, ctr)] += float(_col(row, "Counter_Value", "Value"))
                try:
                    t0 = int(_col(row, "Start_Timestamp", "BeginNs"))
                    t1 = int(_col(row, "End_Timestamp", "EndNs"))
                    dur[(f, disp, name)] = t1 - t0
                except KeyError:
                    pass
    out = defaultdict(lambda: defaultdict(list))
    for (f, disp, name, ctr), v in per.items():
        out[name][ctr].append(v)
    for (f, disp, name), ns in dur.items():
        out[name]["_dur"].append(ns)
    return {k: dict(v) for k, v in out.items()}


def _avg(xs):
    return sum(xs) / len(xs) if xs else None


def copy_scale(cal_dir: str, counter: str, nbytes: int = 1 << 30):
    """Bytes per KiB of counter reading, from the copy-calibration run: the
    largest per-dispatch reading among kernels whose name holds 'copy'
    (the device copy of nbytes), or None."""
    c = read_counters(cal_dir)
    best = None
    for name, ctrs in c.items():
        if "copy" not in name.lower() or counter not in ctrs:
            continue
        v = max(ctrs[counter])
        best = v if best is None else max(best, v)
    if not best:
        return None
    return nbytes / (best * 1024.0)


def digest(out_dir: str, algorithmic=None):
    """Per-kernel figures from the passes under out_dir. algorithmic:
    {short kernel name prefix: {"flops": F, "bytes": B}} per launch."""
    algorithmic = algorithmic or {}
    trace = read_kernel_trace(os.path.join(out_dir, "trace"))
    fetch = read_counters(os.path.join(out_dir, "fetch"))
    write = read_counters(os.path.join(out_dir, "write"))
    sq = read_counters(os.path.join(out_dir, "sq"))
    fscale = copy_scale(os.path.join(out_dir, "cfetch"), "FETCH_SIZE")
    wscale = copy_scale(os.path.join(out_dir, "cwrite"), "WRITE_SIZE")
    total_ns = sum(sum(v) for v in trace.values()) or 1
    rows = []
    for name, durs in sorted(trace.items(), key=lambda kv: -sum(kv[1])):
        r = {"kernel": name, "calls": len(durs), "avg_us": _avg(durs) / 1e3,
             "min_us": min(durs) / 1e3, "max_us": max(durs) / 1e3,
             "share": sum(durs) / total_ns}
        f = fetch.get(name, {}).get("FETCH_SIZE")
        w = write.get(name, {}).get("WRITE_SIZE")
        r["fetch_kib"] = _avg(f) if f else None
        r["write_kib"] = _avg(w) if w else None
        r["hbm_read_bytes"] = r["fetch_kib"] * 1024 * fscale if f and fscale else None
        r["hbm_write_bytes"] = r["write_kib"] * 1024 * wscale if w and wscale else None
        s = sq.get(name, {})
        cyc = _avg(s.get("GRBM_GUI_ACTIVE", [])) if s.get("GRBM_GUI_ACTIVE") else None
        if cyc:
            cyc /= XCDS
            mf = _avg(s.get("SQ_VALU_MFMA_BUSY_CYCLES", []))
            lds = _avg(s.get("SQ_LDS_IDX_ACTIVE", []))
            bc = _avg(s.get("SQ_LDS_BANK_CONFLICT", []))
            r["mfma_busy"] = mf / (cyc * SIMDS) if mf is not None else None
            r["lds_active"] = lds / (cyc * CUS) if lds is not None else None
            r["lds_bank_conflict"] = bc / (cyc * CUS) if bc is not None else None
        wc = _avg(s.get("SQ_WAVE_CYCLES", [])) if s.get("SQ_WAVE_CYCLES") else None
        wi = _avg(s.get("SQ_WAIT_INST_ANY", [])) if s.get("SQ_WAIT_INST_ANY") else None
        r["wait_issue"] = wi / wc if wc and wi is not None else None
        cnt = s.get("GRBM_COUNT")
        d = s.get("_dur")
        if cnt and d:
            r["clock_ghz"] = _avg([c / XCDS / ns for c, ns in zip(cnt, d) if ns > 0])
        if r["avg_us"] < MIN_COUNTER_US:
            # the counters' collection window is several µs longer than a
            # short dispatch: shares of its cycles and the clock say nothing
            for key in ("mfma_busy", "lds_active", "lds_bank_conflict", "clock_ghz"):
                r.pop(key, None)
        for prefix, alg in algorithmic.items():
            if name.startswith(prefix):
                sec = r["avg_us"] * 1e-6
                if alg.get("flops"):
                    r["tflops"] = alg["flops"] / sec / 1e12
                    r["mfma_frac"] = r["tflops"] / PEAK_BF16_TFLOPS
                if alg.get("bytes"):
                    r["gbs"] = alg["bytes"] / sec / 1e9
                    r["hbm_frac"] = r["gbs"] / PEAK_HBM_GBS
                r["alg_flops"] = alg.get("flops")
                r["alg_bytes"] = alg.get("bytes")
        rows.append(r)
    return {"kernels": rows, "fetch_scale": fscale, "write_scale": wscale}


def _fmt(v, spec, scale=1.0):
    return "" if v is None else format(v * scale, spec)


def markdown(d, title: str, commands) -> str:
    lines = [f"# {title}", "", "Commands (from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    fs, ws = d["fetch_scale"], d["write_scale"]
    lines += ["", "Byte counters scaled by a plain 1 GiB device copy's readings: "
              f"FETCH_SIZE x{_fmt(fs, '.4f')} bytes per KiB / 1024, "
              f"WRITE_SIZE x{_fmt(ws, '.4f')}." if fs or ws else "", ""]
    lines += ["| kernel | calls | avg µs | min µs | max µs | share | HBM read GB | HBM write GB "
              "| TFLOP/s | GB/s | MFMA busy | LDS active | LDS conflict | wait issue | clock GHz |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in d["kernels"]:
        lines.append("| `{}` | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} | {} |".format(
            r["kernel"], r["calls"], _fmt(r["avg_us"], ".1f"), _fmt(r["min_us"], ".1f"),
            _fmt(r["max_us"], ".1f"), _fmt(r["share"], ".1%"),
            _fmt(r.get("hbm_read_bytes"), ".3f", 1e-9), _fmt(r.get("hbm_write_bytes"), ".3f", 1e-9),
            _fmt(r.get("tflops"), ".0f"), _fmt(r.get("gbs"), ".0f"),
            _fmt(r.get("mfma_busy"), ".1%"), _fmt(r.get("lds_active"), ".1%"),
            _fmt(r.get("lds_bank_conflict"), ".1%"), _fmt(r.get("wait_issue"), ".1%"),
            _fmt(r.get("clock_ghz"), ".2f")))
    return "\n".join(lines) + "\n"


def bench_cmd(workload: str, steps, warmup, extra=()):
    """bench.py on one workload; steps / warmup None: the benchmark's own
    defaults (the timed run whose HIP-event figures the trace must match)."""
    counts = [] if steps is None else ["--steps", str(steps), "--warmup", str(warmup)]
    return [sys.executable, os.path.join(ROOT, "bench.py"), *counts, "--no-cpu-baseline",
            "--other", "", "--workload", workload, *extra]


def run_passes(workload: str, out_dir: str, steps: int, warmup: int, passes, limit: int,
               extra=()):
    """Each pass as a child process under a time limit; stops at the first
    failure (a pass that failed on the GPU must not be followed by more)."""
    env = dict(os.environ, TMPDIR="/tmp")
    cmds = []
    for p in passes:
        opts = PASSES.get(p) or CALIBRATION[p]
        # the kernel trace of the default timed run (its averages must agree
        # with the bench line's event timing); counters on a short run
        if p in CALIBRATION:
            prog = [sys.executable, os.path.join(ROOT, "bench.py"), "--copy-calibration"]
        elif p == "trace":
            prog = bench_cmd(workload, None, None, extra)
        else:
            prog = bench_cmd(workload, steps, warmup, extra)
        cmd = ["rocprofv3", *opts, "--output-format", "csv", "-d",
               os.path.abspath(os.path.join(out_dir, p)), "-o", p, "--", *prog]
        cmds.append(cmd)
        print(f"[rocprof] pass {p}: {shlex.join(cmd)}", flush=True)
        t0 = time.time()
        r = subprocess.run(cmd, cwd="/tmp", env=env, timeout=limit,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        with open(os.path.join(out_dir, f"{p}.log"), "w") as fh:
            fh.write(r.stdout)
        print(f"[rocprof] pass {p}: rc {r.returncode} in {time.time() - t0:.1f} s", flush=True)
        # rocprofv3 may end with SIGSEGV after the program finished and the
        # results were written; the program's own last line tells
        ok = r.returncode == 0 or (r.returncode in (-11, 139) and '"metric"' in r.stdout) or \
            (p in CALIBRATION and r.returncode in (-11, 139) and "copy_calibration" in r.stdout)
        if not ok:
            raise SystemExit(f"pass {p} failed with {r.returncode}; see {p}.log")
    return cmds


def algorithmic_counts(workload: str, out_dir: str):
    """Per-launch algorithmic flops / bytes of the GEMM kernels from the
    trace pass's bench line (kept rows of its routing)."""
    log = os.path.join(out_dir, "trace.log")
    if not os.path.exists(log):
        return {}
    line = None
    with open(log) as fh:
        for ln in fh:
            if ln.startswith("{") and '"metric"' in ln:
                line = ln
    if line is None:
        return {}
    b = json.loads(line)
    roof = b["roofline"]
    from sparse_expert_ffn_amd import workloads as wk
    wl = wk.WORKLOADS[workload]
    kept = b["layer"]["kept"]
    touched = b["layer"]["touched_experts"]
    e = wl.elem_bytes
    down_flops = 2.0 * wl.D * wl.H * kept + 2.0 * wl.D_shared * wl.H * wl.S
    down_bytes = touched * wl.D * wl.H * e + wl.D_shared * wl.H * e + \
        (kept + (wl.S if wl.D_shared else 0)) * wl.D * e
    up = {"flops": roof["flops_per_launch"], "bytes": roof["bytes_per_launch"]}
    down = {"flops": down_flops, "bytes": down_bytes}
    if wl.mxfp8:  # 1 code byte per element and one scale byte per 32
        down["bytes"] = down_bytes / e * 33 / 32
        return {"upgate_mx_kernel": up, "down_mx_kernel": down}
    return {"upgate_kernel": up, "down_kernel": down, "down_stream_kernel": down}


def bench_line(log: str):
    """The last bench.py JSON line in a pass log, or None."""
    if not os.path.exists(log):
        return None
    line = None
    with open(log) as fh:
        for ln in fh:
            if ln.startswith("{") and '"metric"' in ln:
                line = ln
    return json.loads(line) if line else None


def traffic_record(d, workload: str, block_size: int, commands):
    """The up/gate kernel's counter figures as bench.py's traffic record."""
    from sparse_expert_ffn_amd import buildlib
    up = [r for r in d["kernels"] if r["kernel"].startswith("upgate_kernel")]
    if not up or up[0].get("hbm_read_bytes") is None or up[0].get("hbm_write_bytes") is None:
        return None
    r = up[0]
    return {"kernel": r["kernel"], "workload": workload, "block_size": block_size,
            "source_sha256": buildlib.source_digest(), "dispatches": r["calls"],
            "fetch_size_kib_per_dispatch": r["fetch_kib"],
            "write_size_kib_per_dispatch": r["write_kib"],
            "fetch_scale": d["fetch_scale"], "write_scale": d["write_scale"],
            "hbm_read_bytes_per_launch": r["hbm_read_bytes"],
            "hbm_write_bytes_per_launch": r["hbm_write_bytes"],
            "hbm_bytes_per_launch": r["hbm_read_bytes"] + r["hbm_write_bytes"],
            "commands": commands}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("mode", choices=("run", "report"))
    ap.add_argument("--workload", default="prefill_bal")
    ap.add_argument("--out", required=True)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--passes", default="trace,fetch,write,sq,cfetch,cwrite")
    ap.add_argument("--limit", type=int, default=240, help="seconds per pass")
    ap.add_argument("--md", default=None, help="write the markdown report here")
    ap.add_argument("--traffic-json", default=None,
                    help="write the up/gate kernel's traffic record here")
    a = ap.parse_args(argv)
    os.makedirs(a.out, exist_ok=True)
    passes = [p for p in a.passes.split(",") if p]
    cmds_file = os.path.join(a.out, "commands.json")
    if a.mode == "run":
        cmds = run_passes(a.workload, a.out, a.steps, a.warmup, passes, a.limit)
        with open(cmds_file, "w") as fh:
            json.dump([shlex.join(c) for c in cmds], fh, indent=1)
    cmds = json.load(open(cmds_file)) if os.path.exists(cmds_file) else []
    rel = [re.sub(re.escape(ROOT) + "/", "", c).replace(sys.executable, "python3") for c in cmds]
    rel = [re.sub(r"-d \S+/(\w+) ", r"-d OUT/\1 ", c) for c in rel]
    alg = algorithmic_counts(a.workload, a.out)
    d = digest(a.out, alg)
    bm = None
    tl = os.path.join(a.out, "trace.log")
    if os.path.exists(tl):
        for ln in open(tl):
            if ln.startswith("{") and '"metric"' in ln:
                bm = json.loads(ln)["config"]["block_size"]
    head = [f"python -m sparse_expert_ffn_amd.rocprof_report run --workload {a.workload} "
            f"--out OUT --steps {a.steps} --warmup {a.warmup}",
            "which runs, from /tmp with TMPDIR=/tmp:"] + rel
    md = markdown(d, f"{a.workload}: kernel times and counters (MI355X, gfx950)", head)
    bl = bench_line(tl)
    if bl is not None:
        r = bl["roofline"]
        md += ("\nThe trace pass's own bench line (the default timed run, inputs resident): "
               f"{bl['value'] / 1e6:.3f} M tokens/s, {bl['ms_per_step']:.4f} ms per step; "
               f"{r['kernel']}, average launch by HIP events on its stream: "
               f"{r['avg_launch_ms'] * 1e3:.1f} µs, {r['achieved']:.0f} {r['unit']} = "
               f"{r['frac']:.3f} of {r['peak']:.0f} {r['unit']} (bound: {r['bound']}). "
               "The trace averages above also hold the warm-up launches and the "
               "profiler's own overhead.\n")
    print(md)
    if a.md:
        with open(a.md, "w") as fh:
            fh.write(md)
    if a.traffic_json and bm is not None:
        rec = traffic_record(d, a.workload, bm, head)
        if rec is not None:
            with open(a.traffic_json, "w") as fh:
                json.dump(rec, fh, indent=1)
    with open(os.path.join(a.out, "digest.json"), "w") as fh:
        json.dump(d, fh, indent=1)


if __name__ == "__main__":
    main()
