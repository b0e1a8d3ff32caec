#!/usr/bin/env python3
"""Benchmark of the fused MoE layer forward pass on one MI355X.

One step = the whole hot path on one batch of resident synthetic input:
gate scores (GEMM) -> softmax top-k -> moe_align_block_size -> up/gate GEMM
with SwiGLU -> down GEMM with the router-weighted combine -> output cast,
all enqueued on one stream through the C ABI.

Default workload: the balanced prefill layer (S=16384 tokens, H=2048,
D=2048, E=64 experts, top-2, capacity factor 1.0, bf16 with fp32
accumulation), seeded synthetic inputs.

Prints one JSON line: whole-job tokens/s, the roofline of the dominant kernel
(the up/gate grouped GEMM, timed live with HIP events on its stream) and the
CPU oracle's tokens/s on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (MFMA / vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="prefill_bal")
    ap.add_argument("--block-size", type=int, default=0)
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count S (capacity recomputed)")
    ap.add_argument("--sched", choices=("queue", "batch", "quota"), default="queue",
                    help="grouped-GEMM scheduler: per-XCD atomic task queues (default), the "
                         "same queues claimed 4 tasks per atomic, or the static per-expert "
                         "workgroup quota (ablation baseline)")
    ap.add_argument("--combine", choices=("pass", "fused"), default="pass",
                    help="the router-weighted combine as a pass of its own after the down "
                         "GEMM (default) or inside its epilogue (last arrival per token)")
    ap.add_argument("--split-tail", action="store_true",
                    help="long-tail splitting: each up/gate queue's last tasks as two row halves")
    ap.add_argument("--launch", choices=("two", "one"), default="two",
                    help="the expert GEMMs as two persistent launches (up/gate, then down) "
                         "or as one (down tasks wait per m-block for its up/gate tasks)")
    ap.add_argument("--weight-copies", type=int, default=1,
                    help="rotate the steps over this many copies of the expert weights (a "
                         "cold-cache figure when one copy of the touched weights fits the "
                         "256 MB MALL)")
    ap.add_argument("--other", default="decode,prefill_skew",
                    help="comma-separated workloads timed after the headline one with the "
                         "same step loop (GPU timing only, in other_workloads); '' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU work of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def layer_counts(wl, counts_e, bm):
    """Algorithmic flops and bytes of one layer pass given the kept per-expert
    counts (routing-dependent)."""
    kept = int(counts_e.sum())
    touched = int((counts_e > 0).sum())
    # expert weights: bf16 / fp32 elements, or MXFP8 (a byte per element and a
    # scale byte per 32)
    b = 33.0 / 32.0 if wl.mxfp8 else wl.elem_bytes
    f_gate = 2.0 * wl.S * wl.H * wl.E
    f_up = 4.0 * wl.H * wl.D * kept + 4.0 * wl.H * wl.D_shared * wl.S
    f_down = 2.0 * wl.D * wl.H * kept + 2.0 * wl.D_shared * wl.H * wl.S
    w_expert = 3.0 * wl.H * wl.D * b
    bytes_w = touched * w_expert + 3.0 * wl.H * wl.D_shared * b
    bytes_up = touched * 2.0 * wl.H * wl.D * b + 2.0 * wl.H * wl.D_shared * b + \
        wl.S * wl.H * wl.elem_bytes
    bytes_io = 2.0 * wl.S * wl.H * wl.elem_bytes + wl.H * wl.E * wl.elem_bytes
    # both expert GEMMs in one kernel: the touched weights, A, and the fp32
    # slot rows it writes (h stays between its two halves)
    bytes_experts = bytes_w + wl.S * wl.H * wl.elem_bytes + \
        4.0 * wl.H * (kept + (wl.S if wl.D_shared else 0))
    return {"kept": kept, "touched": touched, "flops_gate": f_gate, "flops_up": f_up,
            "flops_down": f_down, "flops": f_gate + f_up + f_down,
            "bytes": bytes_w + bytes_io, "bytes_up": bytes_up, "bytes_experts": bytes_experts}


def measured_traffic(workload, block_size):
    """HBM bytes per launch of the up/gate kernel from the committed counter
    record (profiles/upgate_<workload>_traffic.json: FETCH_SIZE and
    WRITE_SIZE per dispatch, scaled by a plain device copy's readings), or
    None when there is no record for this workload and block size or the
    kernel sources have changed since it was taken."""
    from sparse_expert_ffn_amd import buildlib
    path = os.path.join(ROOT, "profiles", f"upgate_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("block_size") != block_size or rec.get("source_sha256") != buildlib.source_digest():
        return None
    return float(rec["hbm_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))


def host_info():
    """Host CPU as this process sees it: logical CPUs, the ones it may run
    on, and the model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def gpu_info(moe, torch):
    """The GPU as the HIP runtime reports it."""
    cus, mhz, name = moe.moe_device_query()
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    return {"name": name, "arch": getattr(props, "gcnArchName", None), "compute_units": cus,
            "peak_clock_mhz": mhz, "hbm_gib": round(props.total_memory / 2 ** 30, 1)}


def routing_stats(buf, wl):
    """Histogram figures of one step's routing: rows per expert before and
    after the capacity clip, empty experts, dropped assignments."""
    ids = buf.topk_ids.cpu().numpy().reshape(-1)
    routed = np.bincount(ids, minlength=wl.E)
    kept = buf.expert_counts.cpu().numpy()
    mean = wl.S * wl.k / wl.E
    return {"assignments": int(wl.S * wl.k), "kept": int(kept.sum()),
            "dropped": int(wl.S * wl.k - kept.sum()), "empty_experts": int((routed == 0).sum()),
            "max_rows_per_expert": int(routed.max()), "mean_rows_per_expert": mean,
            "max_over_mean": float(routed.max() / mean) if mean else None,
            "max_kept_rows": int(kept.max()), "capacity": wl.capacity}


def cpu_baseline(wl, target_s):
    """The oracle as it stands, on a bounded sample of the same workload
    (first S' tokens' worth: the same layer at S' tokens), whole layer."""
    import oracle
    from sparse_expert_ffn_amd import workloads as wk
    orc = oracle.default()

    def one(S):
        w = wl.with_tokens(S)
        li = wk.draw_layer(w)
        t0 = time.perf_counter()
        orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, w.k,
                  renormalize=w.renormalize, capacity=w.capacity, Ws_up=li.Ws_up,
                  Ws_gate=li.Ws_gate, Ws_down=li.Ws_down)
        return time.perf_counter() - t0

    S0 = min(wl.S, 64)
    t0 = one(S0)
    S1 = int(min(wl.S, max(S0, S0 * target_s / max(t0, 1e-3))))
    t1 = one(S1) if S1 != S0 else t0
    h = host_info()
    return {"value": S1 / t1, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{wl.name} layer at S={S1} tokens (same H, D, E, k, distributions; "
                      f"capacity recomputed for S), gate+top-k+capacity+experts+combine, "
                      f"{t1:.1f} s",
            "nproc": h["nproc"], "usable_cpus": h["usable_cpus"], "cpu_model": h["cpu_model"]}


def setup_workload(wl, args, torch, moe, dev="cuda"):
    """Resident device inputs and buffers of one workload; returns step()."""
    from sparse_expert_ffn_amd import workloads as wk
    from sparse_expert_ffn_amd.layer import MoEBuffers, suggest_block_size

    dtype = moe.MOE_MXFP8 if wl.mxfp8 else wl.dtype
    bm = args.block_size or suggest_block_size(wl.S, wl.k, wl.E, wl.capacity, dtype)

    def td(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    A, Wr, bias = wk.draw_routing_inputs(wl)
    su, sd, ssu, ssd = wk.expert_sigmas(wl)
    tdt = torch.bfloat16 if wl.dtype == wk.BF16 else torch.float32

    def experts(tid, shape, sigma):
        t = torch.empty((wl.E,) + shape, dtype=tdt, device=dev)

        def sink(e, slab):
            t[e].copy_(td(slab))
        wk.draw_experts(wl, tid, wl.E, shape, sigma, sink=sink)
        return t

    A_d, Wr_d, b_d = td(A), td(Wr), td(bias)
    Wu = experts(wk.T_WUP, (wl.H, wl.D), su)
    Wg = experts(wk.T_WGATE, (wl.H, wl.D), su)
    Wd = experts(wk.T_WDOWN, (wl.D, wl.H), sd)
    Wsu = Wsg = Wsd = None
    if wl.D_shared:
        Wsu = td(wk.draw_tensor(wl, wk.T_WSUP, (wl.H, wl.D_shared), ssu))
        Wsg = td(wk.draw_tensor(wl, wk.T_WSGATE, (wl.H, wl.D_shared), ssu))
        Wsd = td(wk.draw_tensor(wl, wk.T_WSDOWN, (wl.D_shared, wl.H), ssd))
    if wl.mxfp8:  # the expert weights packed once, as a weight load would
        def pack(W):
            if W is None:
                return None
            E, K, N = (1,) + tuple(W.shape) if W.dim() == 2 else tuple(W.shape)
            out = torch.empty(moe.moe_mxfp8_weight_bytes(E, K, N), dtype=torch.uint8, device=dev)
            moe.moe_pack_mxfp8_weights(W, out)
            return out
        Wu, Wg, Wd, Wsu, Wsg, Wsd = (pack(x) for x in (Wu, Wg, Wd, Wsu, Wsg, Wsd))
        torch.cuda.synchronize()
    n_copies = max(1, args.weight_copies)
    copies = [(Wu, Wg, Wd, Wsu, Wsg, Wsd)]
    for _ in range(n_copies - 1):  # same values, other addresses
        copies.append(tuple(None if x is None else x.clone() for x in copies[0]))
    buf = MoEBuffers(wl.S, wl.H, wl.D, wl.E, wl.k, wl.D_shared, wl.capacity, bm,
                     wl.renormalize, dtype, sched_quota=args.sched == "quota",
                     fused_launch=args.launch == "one", device=dev,
                     extra_flags=(moe.MOE_SCHED_BATCH if args.sched == "batch" else 0) |
                     (moe.MOE_COMBINE_FUSED if args.combine == "fused" else 0) |
                     (moe.MOE_SPLIT_TAIL if args.split_tail else 0))
    stream = torch.cuda.current_stream()
    n_step = [0]

    def step():
        w = copies[n_step[0] % n_copies]
        n_step[0] += 1
        buf.run(A_d, Wr_d, *w, router_bias=b_d, stream=stream)

    return step, buf, bm, stream, n_copies


def measure(wl, args, steps, warmup, torch, moe, full=True):
    """Time `steps` passes of the layer after `warmup` untimed ones; the
    roofline kernel (up/gate) is timed by HIP events on its own stream inside
    the timed region. Returns the record (the headline fields when full)."""
    from sparse_expert_ffn_amd import workloads as wk
    step, buf, bm, stream, n_copies = setup_workload(wl, args, torch, moe)
    one = args.launch == "one"
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    counts = buf.expert_counts.cpu().numpy()
    cnt = layer_counts(wl, counts, bm)
    routing = routing_stats(buf, wl)

    # HIP events around the up/gate kernel only (the roofline kernel), on the
    # stream it runs on: each bracketed kernel adds two marker packets, which
    # cost decode-sized steps about 1.5% each
    moe.moe_profile_enable(True, stages=(1,))
    moe.moe_profile_collect()  # drop anything recorded before the timed region
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    moe.moe_profile_enable(False)
    stage_ms, n_calls = moe.moe_profile_collect(5)
    ms = ev0.elapsed_time(ev1) / steps
    up_ms = stage_ms[1] / max(n_calls, 1)
    # setup, down and combine kernels, timed in a few extra steps after the
    # timed region
    moe.moe_profile_enable(True, stages=(0, 2, 3, 4))
    n_extra = min(steps, 10)
    for _ in range(n_extra):
        step()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    small_ms, n_small = moe.moe_profile_collect(5)
    down_ms = small_ms[2] / max(n_small, 1)
    # per-step times (an event pair per step), for the median; after the timed
    # region, which holds no per-step markers
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(steps, 16))]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    med_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) if evs else None
    status = moe.forward_status(buf.forward_ws)

    peak = PEAK_FP8_TFLOPS if wl.mxfp8 else (PEAK_BF16_TFLOPS if wl.dtype == wk.BF16
                                             else PEAK_F32_TFLOPS)
    # the roofline kernel: up/gate, or with one launch both expert GEMMs
    k_flops = cnt["flops_up"] + cnt["flops_down"] if one else cnt["flops_up"]
    k_bytes = cnt["bytes_experts"] if one else cnt["bytes_up"]
    up_tflops = k_flops / (up_ms * 1e-3) / 1e12
    up_gbs = k_bytes / (up_ms * 1e-3) / 1e9
    # the kernel's bound: its byte floor at the HBM peak vs its flop floor at
    # the MFMA peak (decode streams weights; prefill is MFMA work)
    hbm_bound = k_bytes / (PEAK_HBM_GBS * 1e9) > k_flops / (peak * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": up_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": up_gbs / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": up_tflops, "peak": peak, "unit": "TFLOP/s",
                "frac": up_tflops / peak}
    roof.update({"traffic": None if one else measured_traffic(wl.name, bm),
                 "traffic_unit": "HBM bytes per launch",
                 "kernel": ("up/gate + down grouped GEMMs, one launch" if one
                            else "up/gate grouped GEMM + SwiGLU"),
                 "avg_launch_ms": up_ms, "flops_per_launch": k_flops,
                 "bytes_per_launch": k_bytes})
    layer_tflops = cnt["flops"] / (ms * 1e-3) / 1e12
    floor_s = max(cnt["flops"] / (peak * 1e12), cnt["bytes"] / (PEAK_HBM_GBS * 1e9))
    layer_bound = "hbm" if cnt["bytes"] / (PEAK_HBM_GBS * 1e9) > cnt["flops"] / (peak * 1e12) \
        else "mfma"
    layer = {"tflops": layer_tflops, "mfma_frac": layer_tflops / peak,
             "bound": layer_bound, "floor_ms": floor_s * 1e3,
             "roofline_frac": floor_s / (ms * 1e-3),
             "gbs": cnt["bytes"] / (ms * 1e-3) / 1e9,
             "hbm_frac": cnt["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "kept": cnt["kept"],
             "touched_experts": cnt["touched"], "down_ms": None if one else down_ms,
             "down_tflops": None if one else cnt["flops_down"] / (down_ms * 1e-3) / 1e12,
             "setup_ms": small_ms[0] / max(n_small, 1),
             "combine_ms": small_ms[3] / max(n_small, 1),
             "median_ms_per_step": med_ms, "wall_s": wall, "status_word": status}
    config = {"workload": wl.name, "S": wl.S, "H": wl.H, "D": wl.D, "E": wl.E, "k": wl.k,
              "D_shared": wl.D_shared, "capacity": wl.capacity, "block_size": bm,
              "scheduler": args.sched, "launch": args.launch, "combine": args.combine,
              "split_tail": bool(args.split_tail),
              "weight_copies": n_copies,
              "parallelism": "single GPU"}
    if wl.mxfp8:
        layer["quantize_ms"] = small_ms[4] / max(n_small, 1)
    rec = {"ms_per_step": ms, "value": wl.S / (ms * 1e-3), "config": config, "roofline": roof,
           "layer": layer, "routing": routing, "steps": steps, "warmup": warmup,
           "dtype": "mxfp8" if wl.mxfp8 else ("bf16" if wl.dtype == wk.BF16 else "f32")}
    del buf
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU expert-parallel path is not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return

    import sparse_expert_ffn_amd as moe
    from sparse_expert_ffn_amd import workloads as wk

    moe.load_library()
    wl = wk.WORKLOADS[args.workload]
    if args.tokens > 0:
        wl = wl.with_tokens(args.tokens)
    head = measure(wl, args, args.steps, args.warmup, torch, moe)
    others = {}
    for name in [n for n in args.other.split(",") if n and n != wl.name]:
        o = measure(wk.WORKLOADS[name], args, min(args.steps, 20), min(args.warmup, 10), torch,
                    moe)
        others[name] = {"ms_per_step": o["ms_per_step"], "tokens_per_s": o["value"],
                        "steps": o["steps"], "warmup": o["warmup"], "config": o["config"],
                        "roofline": {k: o["roofline"][k] for k in
                                     ("bound", "achieved", "peak", "unit", "frac", "kernel",
                                      "avg_launch_ms")},
                        "layer": {k: o["layer"][k] for k in
                                  ("bound", "floor_ms", "roofline_frac", "tflops", "mfma_frac",
                                   "gbs", "hbm_frac", "down_ms", "combine_ms",
                                   "median_ms_per_step", "status_word")},
                        "routing": o["routing"]}
    out = {
        "metric": "MoE layer tokens/s + % bf16 MFMA peak (prefill) / % HBM BW (decode)",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded PCG64 normals, pages' distributions)",
        "config": head["config"],
        "roofline": head["roofline"],
        "layer": head["layer"],
        "routing": head["routing"],
        "gpu": gpu_info(moe, torch),
        "host": host_info(),
    }
    if others:
        out["other_workloads"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
