"""The layer's three calls enqueue only kernels (counters and flags are
cleared by a fill kernel, no memset node), so a caller can capture a whole
step in a HIP graph. A captured step, replayed several times with eager work
and synchronisations between the replays, gives the eager output bit for bit
every time."""
import numpy as np
import pytest
import torch

import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, buffers, host

pytestmark = pytest.mark.gpu

# decode: split gate, one-workgroup align, streaming down kernel; prefill_skew
# at 300 tokens: fused gate + top-k, queue kernels; dsv3: the shared expert
# (the last case with the combine inside the down epilogue: its arrival
# counters are cleared by the same fill kernel)
CASES = [("decode", 64, 16, 0), ("prefill_skew", 300, 128, 0), ("dsv3", 100, 256, 0),
         ("prefill_skew", 300, 128, moe.MOE_COMBINE_FUSED)]


@pytest.mark.parametrize("name,S,bm,flags", CASES)
def test_captured_step_replays_match_eager(name, S, bm, flags):
    wl = wk.WORKLOADS[name].with_tokens(S)
    L = DeviceLayer(wl)
    buf = buffers(wl, bm, out_f32=True, extra_flags=flags)

    def step():
        buf.run(L.A, L.Wr, L.W_up, L.W_gate, L.W_down, L.Ws_up, L.Ws_gate, L.Ws_down,
                router_bias=L.bias)

    step()
    torch.cuda.synchronize()
    eager = host(buf.O).copy()
    ids = buf.topk_ids.cpu().numpy().copy()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream once, outside the graph
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        buf.O.fill_(float("nan"))        # stale outputs must be overwritten by the replay
        buf.topk_ids.fill_(-1)
        buf.forward_ws.fill_(0xFF)       # counters, flags, slots: all re-initialised inside
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(buf.topk_ids.cpu().numpy(), ids), f"replay {rep}: routing"
        got = host(buf.O)
        assert np.array_equal(got, eager), f"replay {rep}: output differs from eager"
        step()                           # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(buf.O), eager)
