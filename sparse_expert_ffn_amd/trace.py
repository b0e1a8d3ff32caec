"""Per-task timing of the persistent GEMM kernels, from the kernels' own
stamps (the library variant built with MOE_TRACE, libmoe_trace.so).

An external profiler sees one duration per launch; the persistent kernels'
balance lives inside the launch: how long each task's row metadata, K loop
and epilogue take, how long a claim takes, and how long each workgroup sits
idle after its last task while others finish (the tail the Weave review's
section 5.2 describes). The kernels stamp those moments themselves with the
GPU's 100 MHz constant clock (moe_trace_attach in include/moe.h), and this
module reads the records back and summarises them.

  python -m sparse_expert_ffn_amd.trace --workload prefill_bal [--launch one]

prints one JSON object per kernel. Nothing here touches the layer's
arithmetic; the records are timing only.
"""
from __future__ import annotations

import argparse
import json
import os

import numpy as np

TICK_US = 0.01  # 100 MHz constant clock
HEADER_BYTES = 64
REC = np.dtype([("kernel", "<u4"), ("wg", "<u4"), ("task", "<i8"), ("t_claim", "<u8"),
                ("t_rows", "<u8"), ("t_kloop", "<u8"), ("t_end", "<u8")])
KERNELS = {1: "up/gate", 2: "down", 3: "one launch: up/gate tasks", 4: "one launch: down tasks"}


def parse(raw: np.ndarray) -> np.ndarray:
    """Records from the bytes of a trace buffer (uint8 array)."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    n = int(raw[:8].view("<u8")[0])
    cap = (raw.size - HEADER_BYTES) // REC.itemsize
    recs = raw[HEADER_BYTES:HEADER_BYTES + min(n, cap) * REC.itemsize].view(REC)
    return recs


def summarize(recs: np.ndarray, kernels=(1, 2, 3, 4)) -> dict:
    """Per kernel id: task count, mean phase times (µs), claim gaps, tasks per
    workgroup, and the share of workgroup time spent idle after each
    workgroup's last task until the last one ends."""
    out = {}
    merged = {1: (1,), 2: (2,), 3: (3, 4), 4: (3, 4)}
    for k in kernels:
        r = recs[np.isin(recs["kernel"], merged[k])] if k in (3, 4) else recs[recs["kernel"] == k]
        tasks = r[(r["task"] >= 0) & (r["kernel"] == k)]
        if tasks.size == 0:
            continue
        exits = r[r["task"] < 0]
        t0 = int(r["t_claim"].min())
        t_last = int(max(r["t_end"].max(), exits["t_claim"].max() if exits.size else 0))
        span = max(t_last - t0, 1)
        wgs = np.unique(r["wg"])
        # a workgroup's finish: its exit stamp, else its last task's end
        finish = []
        for w in wgs:
            ex = exits[exits["wg"] == w]
            mine = r[(r["wg"] == w) & (r["task"] >= 0)]
            f = int(ex["t_claim"].max()) if ex.size else int(mine["t_end"].max())
            last_end = int(mine["t_end"].max()) if mine.size else f
            finish.append(last_end)
        finish = np.asarray(finish, dtype=np.float64)
        idle = float(np.sum(t_last - finish) / (wgs.size * span))
        per_wg = np.bincount(tasks["wg"].astype(np.int64))
        per_wg = per_wg[per_wg > 0]
        # gap between a workgroup's previous task end and its next claim result
        gaps = []
        for w in np.unique(tasks["wg"]):
            mine = np.sort(r[(r["wg"] == w) & (r["task"] >= 0)], order="t_claim")
            if mine.size > 1:
                gaps.extend((mine["t_claim"][1:].astype(np.int64) -
                             mine["t_end"][:-1].astype(np.int64)).tolist())
        ph = lambda a, b: float(np.mean(tasks[b].astype(np.int64) -
                                        tasks[a].astype(np.int64))) * TICK_US
        out[KERNELS[k]] = {
            "tasks": int(tasks.size), "workgroups": int(wgs.size),
            "split_parts": int(np.sum((tasks["task"] & 3) != 0)),
            "span_us": span * TICK_US,
            "mean_us": {"claim_to_kloop": ph("t_claim", "t_rows"),
                        "kloop": ph("t_rows", "t_kloop"),
                        "epilogue": ph("t_kloop", "t_end")},
            "claim_gap_us": float(np.mean(gaps)) * TICK_US if gaps else None,
            "tasks_per_workgroup": {"min": int(per_wg.min()), "max": int(per_wg.max())},
            "idle_after_last_task": idle,
        }
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="prefill_bal")
    ap.add_argument("--tokens", type=int, default=0)
    ap.add_argument("--block-size", type=int, default=0)
    ap.add_argument("--launch", choices=("two", "one"), default="two")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--records", type=int, default=1 << 16)
    a = ap.parse_args(argv)

    import torch

    import sparse_expert_ffn_amd as moe
    from sparse_expert_ffn_amd import buildlib
    from sparse_expert_ffn_amd import workloads as wk
    from sparse_expert_ffn_amd.layer import MoEBuffers, suggest_block_size

    if not os.path.exists(buildlib.TRACE_LIB):
        raise SystemExit(f"{buildlib.TRACE_LIB} is missing: build it first (buildlib.build_all)")
    moe.LIB_PATH = buildlib.TRACE_LIB
    moe.load_library()
    wl = wk.WORKLOADS[a.workload]
    if a.tokens:
        wl = wl.with_tokens(a.tokens)
    dtype = moe.MOE_MXFP8 if wl.mxfp8 else wl.dtype
    bm = a.block_size or suggest_block_size(wl.S, wl.k, wl.E, wl.capacity, dtype)
    li = wk.draw_layer(wl)

    def td(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    ins = [td(x) for x in (li.A, li.Wr, li.W_up, li.W_gate, li.W_down, li.Ws_up, li.Ws_gate,
                           li.Ws_down)]
    if wl.mxfp8:  # expert weights packed once for the MXFP8 GEMMs
        def pack(W):
            if W is None:
                return None
            E, K, N = (1,) + tuple(W.shape) if W.dim() == 2 else tuple(W.shape)
            out = torch.empty(moe.moe_mxfp8_weight_bytes(E, K, N), dtype=torch.uint8,
                              device="cuda")
            moe.moe_pack_mxfp8_weights(W, out)
            return out
        ins = ins[:2] + [pack(w) for w in ins[2:]]
    bias = td(li.bias)
    buf = MoEBuffers(wl.S, wl.H, wl.D, wl.E, wl.k, wl.D_shared, wl.capacity, bm,
                     wl.renormalize, dtype, fused_launch=a.launch == "one", device="cuda")
    trace = torch.zeros(HEADER_BYTES + a.records * REC.itemsize, dtype=torch.uint8,
                        device="cuda")
    for _ in range(a.warmup):
        buf.run(*ins, router_bias=bias)
    torch.cuda.synchronize()
    moe.moe_trace_attach(trace)
    buf.run(*ins, router_bias=bias)
    torch.cuda.synchronize()
    moe.moe_trace_attach(None)
    recs = parse(trace.cpu().numpy())
    res = {"workload": wl.name, "block_size": bm, "launch": a.launch,
           "records": int(recs.size), "kernels": summarize(recs)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
