"""The task queues' options on the GPU: batched claims run the same tiles
(bit-identical output), and the end-of-kernel queue check reports tasks that
never ran (forced from the host by keeping the previous call's queue
counters; every kernel still ends normally: its claims simply fail)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, buffers, dev, host, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _run(L, buf, G):
    buf.route(logits_in=dev(G))
    O = host(L.forward(buf)).copy()
    torch.cuda.synchronize()
    return O, moe.forward_status(buf.forward_ws)


BATCH_CASES = [("prefill_skew", 300, 128), ("prefill_skew", 300, 256), ("dsv3", 40, 256),
               ("decode", 64, 16), ("tiny_fp32", 64, 16), ("prefill_bal_mxfp8", 300, 128)]


@pytest.mark.parametrize("split", [0, moe.MOE_SPLIT_TAIL])
@pytest.mark.parametrize("name,S,bm", BATCH_CASES)
def test_batched_claims_same_output(orc, name, S, bm, split):
    """Four tasks per queue atomic: the same tiles (with MOE_SPLIT_TAIL, half
    tiles at the queues' ends included) as one task per atomic, so the output
    is the same bit for bit, and the queue check passes."""
    wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    outs = []
    for flags in (0, moe.MOE_SCHED_BATCH):
        buf = buffers(wl, bm, out_f32=True)
        buf.shape.flags |= flags | split
        buf.forward_ws.fill_(0xFF)
        O, st = _run(L, buf, G)
        assert st == 0, f"status {st} with flags {flags}"
        outs.append(O)
    assert np.all(np.isfinite(outs[1]))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("name,S,bm", [("prefill_bal", 700, 128), ("dsv3", 40, 256),
                                       ("prefill_bal_mxfp8", 300, 128)])
def test_queue_check_reports_lost_tasks(orc, name, S, bm):
    """A call that keeps the previous call's queue counters hands out no
    tasks: the status word reports lost tasks and a wrong final count. The
    next ordinary call resets the counters and is right again."""
    wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    buf = buffers(wl, bm, out_f32=True)
    buf.forward_ws.zero_()
    good, st = _run(L, buf, G)
    assert st == 0
    buf.shape.flags |= moe.MOE_TEST_SKIP_QUEUE_RESET
    _, st = _run(L, buf, G)
    assert st & moe.MOE_STATUS_TASKS_LOST, f"status {st}"
    assert st & moe.MOE_STATUS_QUEUE_COUNT, f"status {st}"
    buf.shape.flags &= ~moe.MOE_TEST_SKIP_QUEUE_RESET
    again, st = _run(L, buf, G)
    assert st == 0
    assert np.array_equal(good, again)
    if not wl.mxfp8:
        ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                        renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                        Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
        err, tol = parity(wl, again, ref["O"])
        assert err <= tol


SPLIT_CASES = [("prefill_skew", 300, 128), ("prefill_skew", 700, 256), ("prefill_bal", 700, 128),
               ("prefill_bal", 3000, 256), ("dsv3", 100, 256), ("decode", 64, 16),
               ("tiny_fp32", 64, 16), ("prefill_bal_mxfp8", 300, 128)]


@pytest.mark.parametrize("name,S,bm", SPLIT_CASES)
def test_split_tail_same_output(orc, name, S, bm):
    """Long-tail splitting (MOE_SPLIT_TAIL): each up/gate queue's last tasks
    run as two row halves on the half-row core, which adds the same K chunks
    in the same order: the output equals the whole-tile run's bit for bit, and
    the queue check (which counts the half parts) passes. Where the flag has
    no effect (16-row tiles, fp32, MXFP8) the outputs are equal too."""
    wl = wk.WORKLOADS[name].with_tokens(S)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    outs = []
    for flags in (0, moe.MOE_SPLIT_TAIL):
        buf = buffers(wl, bm, out_f32=True)
        buf.shape.flags |= flags
        buf.forward_ws.fill_(0xFF)
        O, st = _run(L, buf, G)
        assert st == 0, f"status {st} with flags {flags}"
        outs.append(O)
    assert np.all(np.isfinite(outs[1]))
    assert np.array_equal(outs[0], outs[1])
