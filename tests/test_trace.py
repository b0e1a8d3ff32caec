"""Per-task timing records (MOE_TRACE build): the record layout the header
documents, the summary arithmetic on synthetic records (CPU), and on the GPU
the records of real launches: one per task, stamps in order, one exit per
workgroup, and the traced library's output equal to the plain one's."""
import os
import re

import numpy as np
import pytest

import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import buildlib
from sparse_expert_ffn_amd import trace as tr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_record_layout_matches_header():
    assert tr.REC.itemsize == 48 and tr.HEADER_BYTES == 64
    common = open(os.path.join(ROOT, "sparse_expert_ffn_amd", "csrc", "moe_common.h")).read()
    assert re.search(r"kTraceHeaderBytes\s*=\s*64", common)
    body = re.search(r"struct TraceRec \{(.*?)\};", common, re.S).group(1)
    fields = re.findall(r"(uint32_t|int64_t|uint64_t)\s+(\w+);", body)
    assert [f for _, f in fields] == ["kernel", "workgroup", "task", "t_claim", "t_rows",
                                      "t_kloop", "t_end"]


def _recs(rows):
    r = np.zeros(len(rows), dtype=tr.REC)
    for i, row in enumerate(rows):
        r[i] = row
    return r


def test_summary_arithmetic():
    # two workgroups of kernel 1: wg 0 runs tasks 0 and 2 (100 ticks each), wg 1
    # runs task 1 and leaves early; times in 100 MHz ticks
    rows = [(1, 0, 0 << 2, 0, 10, 90, 100), (1, 0, 2 << 2, 110, 120, 190, 200),
            (1, 0, -1, 210, 210, 210, 210),
            (1, 1, 1 << 2, 0, 10, 90, 100), (1, 1, -1, 105, 105, 105, 105)]
    raw = np.zeros(tr.HEADER_BYTES + len(rows) * tr.REC.itemsize, dtype=np.uint8)
    raw[:8] = np.frombuffer(np.uint64(len(rows)).tobytes(), dtype=np.uint8)
    raw[tr.HEADER_BYTES:] = _recs(rows).view(np.uint8)
    s = tr.summarize(tr.parse(raw))["up/gate"]
    assert s["tasks"] == 3 and s["workgroups"] == 2
    assert s["mean_us"]["claim_to_kloop"] == pytest.approx(0.1)
    assert s["mean_us"]["kloop"] == pytest.approx((80 + 70 + 80) / 3 * 0.01)
    assert s["mean_us"]["epilogue"] == pytest.approx(0.1)
    assert s["claim_gap_us"] == pytest.approx(0.1)
    assert s["tasks_per_workgroup"] == {"min": 1, "max": 2}
    # span 0 .. 210; wg 0 idle 10 ticks after its last task, wg 1 110
    assert s["idle_after_last_task"] == pytest.approx((10 + 110) / (2 * 210))


def test_attach_unsupported_without_trace_build():
    lib = moe.load_library()
    assert lib.moe_trace_attach(None, 0) == 2


@pytest.mark.skipif(not os.path.exists(buildlib.TRACE_LIB), reason="trace library not built")
def test_attach_validation_on_trace_build():
    import ctypes
    lib = ctypes.CDLL(buildlib.TRACE_LIB)
    lib.moe_trace_attach.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    assert lib.moe_trace_attach(None, 0) == 0
    assert lib.moe_trace_attach(0x100010, 4096) == 1     # not 64-byte aligned
    assert lib.moe_trace_attach(0x100000, 32) == 1       # smaller than the header


@pytest.mark.gpu
@pytest.mark.parametrize("name,S,launch", [("prefill_skew", 600, "two"),
                                           ("decode", 64, "two"),
                                           ("prefill_bal", 700, "one")])
def test_trace_records_on_gpu(name, S, launch):
    import torch

    from sparse_expert_ffn_amd import workloads as wk
    from tests.gpu_util import DeviceLayer, buffers, dev, host

    assert os.path.exists(buildlib.TRACE_LIB), "libmoe_trace.so must be built"
    wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    plain = moe.load_library()
    outs, recs = [], None
    for traced in (False, True):
        lib = moe.load_library(buildlib.TRACE_LIB) if traced else plain
        moe._LIB = lib
        try:
            buf = buffers(wl, out_f32=True, fused_launch=launch == "one")
            buf.route(L.A, L.Wr, L.bias)
            if traced:
                t = torch.zeros(tr.HEADER_BYTES + 8192 * tr.REC.itemsize, dtype=torch.uint8,
                                device="cuda")
                moe.moe_trace_attach(t)
            outs.append(host(L.forward(buf)).copy())
            torch.cuda.synchronize()
            if traced:
                moe.moe_trace_attach(None)
                recs = tr.parse(t.cpu().numpy())
        finally:
            moe._LIB = plain
    assert np.array_equal(outs[0], outs[1]), "timing records change no result"
    kinds = (1, 2) if launch == "two" else (3, 4)
    assert recs.size > 0 and set(np.unique(recs["kernel"])) <= set(kinds)
    tasks = recs[recs["task"] >= 0]
    assert np.all(tasks["t_claim"] <= tasks["t_rows"])
    assert np.all(tasks["t_rows"] <= tasks["t_kloop"])
    assert np.all(tasks["t_kloop"] <= tasks["t_end"])
    for k in ((1, 2) if launch == "two" else (4,)):
        ex = recs[(recs["kernel"] == k) & (recs["task"] < 0)]
        assert np.unique(ex["wg"]).size == ex.size, "one exit record per workgroup"
    for k in kinds:
        ids = tasks[tasks["kernel"] == k]["task"]
        whole = ids[(ids & 3) == 0] >> 2
        assert np.unique(whole).size == whole.size, "no task claimed twice"
    s = tr.summarize(recs)
    assert all(0.0 <= v["idle_after_last_task"] < 1.0 for v in s.values())
