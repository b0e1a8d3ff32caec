"""GPU layer forward vs the CPU oracle, element by element, on one shared
routing (the GPU is fed the oracle's gate scores), at token counts the oracle
finishes in seconds: every workload, several block sizes, ragged tiles,
capacity drops, a hot expert, k = E, shared experts, fp32 and bf16, poisoned
workspaces and outputs."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, bf16_output_excess, buffers, dev, host, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def run_case(orc, wl, bm=None, li=None, logits=None, poison=True, atomic=False):
    """Oracle and GPU on one routing. bf16 layers run twice: with an fp32
    output (the parity bar applies to the fp32-accumulated result) and with a
    bf16 output (the bar plus that output's own rounding)."""
    li = li if li is not None else wk.draw_layer(wl)
    G_o = orc.gate_logits(li.A, li.Wr, li.bias) if logits is None else logits
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G_o)
    L = DeviceLayer(wl, li)
    outs = {}
    for out_f32 in ((False,) if wl.dtype == wk.F32 else (True, False)):
        buf = buffers(wl, bm, out_f32, atomic_combine=atomic)
        if poison:
            buf.forward_ws.fill_(0xFF)   # NaN patterns: any unwritten read shows up
            buf.align_ws.fill_(0xFF)
            buf.O.fill_(float("nan"))
        buf.route(logits_in=dev(G_o))
        O = L.forward(buf)
        torch.cuda.synchronize()
        assert moe.forward_status(buf.forward_ws) == 0, "status word set"
        assert np.array_equal(buf.topk_ids.cpu().numpy(), ref["ids"]), "routing differs"
        outs[out_f32] = host(O)
        assert np.all(np.isfinite(outs[out_f32])), "non-finite output"
    if wl.dtype == wk.F32:
        err, tol = parity(wl, outs[False], ref["O"])
        return err, tol, ref, outs[False]
    err, tol = parity(wl, outs[True], ref["O"])
    ex = bf16_output_excess(outs[False], ref["O"])
    assert ex <= 1.0, f"bf16 output beyond bar + own rounding: {ex:.3f}"
    return err, tol, ref, outs[True]


CASES = [("tiny_fp32", 64, 16), ("tiny_fp32", 64, 128), ("prefill_bal", 700, 128),
         ("prefill_bal", 700, 256), ("prefill_bal", 700, 16), ("prefill_bal", 333, 64),
         ("prefill_skew", 300, 128), ("prefill_skew", 300, 256), ("prefill_skew", 300, 32),
         ("decode", 64, 16), ("decode", 64, 128), ("decode", 1, 16), ("dsv3", 40, 128)]


@pytest.mark.parametrize("name,S,bm", CASES)
def test_layer_parity(orc, name, S, bm):
    wl = wk.WORKLOADS[name].with_tokens(S)
    err, tol, ref, _ = run_case(orc, wl, bm)
    print(f"{name} S={S} BM={bm}: err {err:.3e} (tol {tol:.0e})")
    assert err <= tol


def _small(dtype, **kw):
    base = dict(name="small", S=200, H=136, D=200, E=12, k=3, dtype=dtype,
                router_std=0.5)
    base.update(kw)
    return wk.Workload(**base)


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_ragged_tiles_and_shared(orc, dtype):
    """H, D, D_shared not multiples of the 128-wide tiles; K tails; shared expert."""
    wl = _small(dtype, D_shared=72)
    for bm in ((16, 64) if dtype == wk.F32 else (16, 64, 256)):
        err, tol, _, _ = run_case(orc, wl, bm)
        assert err <= tol, f"BM={bm}: {err:.3e}"


@pytest.mark.parametrize("dtype", [wk.F32, wk.BF16])
def test_capacity_drops(orc, dtype):
    wl = _small(dtype, capacity_factor=0.25)
    assert 0 < wl.capacity < 50
    err, tol, ref, _ = run_case(orc, wl, 32)
    assert ref["kept"] is not None and ref["kept"].sum() < wl.S * wl.k
    assert err <= tol


@pytest.mark.parametrize("bm", [128, 256])
def test_hot_expert_and_empty_experts(orc, bm):
    """Every token picks expert 5 first: one expert holds S rows (many m-blocks),
    most experts are empty."""
    wl = _small(wk.BF16, S=1500, E=40, k=2)
    li = wk.draw_layer(wl)
    rng = np.random.default_rng(0)
    G = rng.standard_normal((wl.S, wl.E)).astype(np.float32)
    G[:, 5] += 50.0
    G[:, 9] += 10.0 * (rng.random(wl.S) > 0.5)
    err, tol, ref, _ = run_case(orc, wl, bm, li=li, logits=G)
    assert err <= tol


def test_k_equals_E(orc):
    wl = _small(wk.BF16, S=130, E=4, k=4)
    err, tol, _, _ = run_case(orc, wl, 64)
    assert err <= tol


def test_all_dropped_but_shared(orc):
    """Capacity 1 on a tiny layer: most tokens get only the shared expert."""
    wl = _small(wk.F32, S=64, E=2, k=1, D_shared=16, capacity_factor=1.0 / 32)
    assert wl.capacity == 1
    err, tol, _, _ = run_case(orc, wl, 16)
    assert err <= tol


@pytest.mark.parametrize("atomic", [False, True])
def test_repeat_calls_same_buffers(orc, atomic):
    """Two forward passes on the same buffers: the default slot combine is
    bit-reproducible; the atomic combine may reorder its fp32 sums."""
    wl = wk.WORKLOADS["prefill_skew"].with_tokens(200)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    buf = buffers(wl, 64, atomic_combine=atomic)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    outs = []
    for _ in range(2):
        buf.route(logits_in=dev(G))
        outs.append(host(L.forward(buf)).copy())
    torch.cuda.synchronize()
    if atomic:
        assert np.max(np.abs(outs[0] - outs[1])) <= 1e-2 * np.sqrt(np.mean(outs[0] ** 2))
    else:
        assert np.array_equal(outs[0], outs[1])


ATOMIC_CASES = [("tiny_fp32", 64, 16), ("prefill_bal", 700, 256), ("prefill_skew", 300, 128),
                ("decode", 64, 16), ("dsv3", 40, 128)]


@pytest.mark.parametrize("name,S,bm", ATOMIC_CASES)
def test_layer_parity_atomic_combine(orc, name, S, bm):
    wl = wk.WORKLOADS[name].with_tokens(S)
    err, tol, _, _ = run_case(orc, wl, bm, atomic=True)
    assert err <= tol


def test_capacity_drops_atomic(orc):
    wl = _small(wk.BF16, capacity_factor=0.25)
    err, tol, _, _ = run_case(orc, wl, 32, atomic=True)
    assert err <= tol


QUOTA_CASES = [("prefill_skew", 300, 128), ("dsv3", 40, 256), ("decode", 64, 16),
               ("tiny_fp32", 64, 16), ("many_experts", 300, 32)]


@pytest.mark.parametrize("name,S,bm", QUOTA_CASES)
def test_quota_scheduler_same_output(orc, name, S, bm):
    """The static per-expert quota scheduler (ablation baseline) runs the same
    tiles as the queue scheduler: bit-identical output. many_experts has more
    experts (600) than workgroups, so each workgroup serves several; dsv3 adds
    the shared expert's tasks."""
    if name == "many_experts":
        wl = _small(wk.BF16, S=S, E=600, k=4)
    else:
        wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    outs = []
    for quota in (False, True):
        buf = buffers(wl, bm, out_f32=True, sched_quota=quota)
        buf.forward_ws.fill_(0xFF)
        buf.route(logits_in=dev(G))
        outs.append(host(L.forward(buf)).copy())
    torch.cuda.synchronize()
    assert np.all(np.isfinite(outs[1]))
    assert np.array_equal(outs[0], outs[1])
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
    err, tol = parity(wl, outs[1], ref["O"])
    assert err <= tol


FUSED_COMBINE_CASES = [("prefill_bal", 700, 128), ("prefill_bal", 700, 256),
                       ("prefill_skew", 300, 256), ("dsv3", 40, 256), ("decode", 64, 16),
                       ("tiny_fp32", 64, 16), ("drops", 200, 32), ("shared_drops", 64, 16)]


@pytest.mark.parametrize("name,S,bm", FUSED_COMBINE_CASES)
def test_fused_combine_same_output(orc, name, S, bm):
    """The combine inside the down epilogue (last arrival per token and tile
    adds the token's rows) gives the slot combine pass's output bit for bit:
    fp32 and bf16 outputs, the shared expert, decode sizes (queue kernel),
    capacity drops that leave tokens with no kept slot (zero rows), and every
    routed assignment dropped beside a shared expert."""
    if name == "drops":
        wl = _small(wk.BF16, S=S, capacity_factor=0.2)
    elif name == "shared_drops":
        wl = _small(wk.BF16, S=S, capacity_factor=0.05, D_shared=64)
    else:
        wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    if name in ("drops", "shared_drops"):
        kept = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                         renormalize=wl.renormalize, capacity=wl.capacity, logits=G)["kept"]
        assert (kept.reshape(wl.S, wl.k).sum(axis=1) == 0).any(), "no token lost every slot"
    f32_out = None
    for out_f32 in ((True,) if wl.dtype == wk.F32 else (True, False)):
        outs = []
        for flags in (0, moe.MOE_COMBINE_FUSED):
            buf = buffers(wl, bm, out_f32=out_f32, extra_flags=flags)
            buf.forward_ws.fill_(0xFF)
            buf.O.fill_(float("nan"))
            buf.route(logits_in=dev(G))
            outs.append(host(L.forward(buf)).copy())
            torch.cuda.synchronize()
            assert moe.forward_status(buf.forward_ws) == 0
        assert np.all(np.isfinite(outs[1])), "non-finite output (a row never written?)"
        assert np.array_equal(outs[0], outs[1]), f"out_f32={out_f32}: differs from the pass"
        if out_f32:
            f32_out = outs[1]
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
    err, tol = parity(wl, f32_out, ref["O"])
    assert err <= tol


def test_fused_combine_repeat_calls():
    """Repeated calls on the same buffers (arrival counters cleared by each
    call's setup kernel) give the same output bit for bit."""
    wl = wk.WORKLOADS["prefill_skew"].with_tokens(300)
    L = DeviceLayer(wl)
    buf = buffers(wl, 128, out_f32=True, extra_flags=moe.MOE_COMBINE_FUSED)
    outs = []
    for _ in range(3):
        buf.run(L.A, L.Wr, L.W_up, L.W_gate, L.W_down, router_bias=L.bias)
        torch.cuda.synchronize()
        outs.append(host(buf.O).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
