"""moe_forward_noalloc, the allocation-free variant of moe_forward (its
workspace is the library's own device array): the same kernels on the same
inputs, so its output equals moe_forward's bit for bit. Each case makes two
calls in a row on the one GPU array, the second with fewer tokens, so the
second call runs on what the first left behind."""
import numpy as np
import pytest
import torch

import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, buffers, host

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(name="small_shared", S=200, H=136, D=200, E=12, k=3, dtype=wk.BF16,
                router_std=0.5, D_shared=72)
    base.update(kw)
    return wk.Workload(**base)


CASES = [("decode", 64, 17, True), ("prefill_skew", 300, 120, True),
         ("small_shared", 200, 50, False), ("tiny_fp32", 64, 9, True)]


@pytest.mark.parametrize("name,S1,S2,out_f32", CASES)
def test_noalloc_matches_forward(name, S1, S2, out_f32):
    for S in (S1, S2):
        wl = (_small(S=S) if name == "small_shared" else wk.WORKLOADS[name].with_tokens(S))
        print(f"[noalloc {name} S={S}]", flush=True)
        L = DeviceLayer(wl)
        buf = buffers(wl, out_f32=out_f32)
        need = moe.moe_forward_workspace_bytes(buf.shape)
        assert 0 < need <= moe.MOE_NOALLOC_SCRATCH_BYTES
        buf.route(L.A, L.Wr, L.bias)
        ref = host(L.forward(buf)).copy()
        O = torch.full_like(buf.O, float("nan"))
        moe.moe_forward_noalloc(buf.shape, L.A, L.W_up, L.W_gate, L.W_down, L.Ws_up,
                                L.Ws_gate, L.Ws_down, buf.topk_weights, buf.sorted_ids,
                                buf.expert_ids, buf.ntpp, O)
        torch.cuda.synchronize()
        got = host(O)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), f"S={S}: differs from moe_forward"


def test_noalloc_rejects_oversize():
    wl = wk.WORKLOADS["prefill_bal"]
    shape = moe.make_shape(wl.S, wl.H, wl.D, wl.E, wl.k, capacity=wl.capacity, block_size=256)
    assert moe.moe_forward_workspace_bytes(shape) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    code = moe.moe_forward_noalloc(shape, x, x, x, x, None, None, None, x, x, x, x, x,
                                   check=False)
    assert code == 3  # MOE_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
