"""Full-size parity of the four bf16 workloads, in the configuration the
benchmark times (same shapes, block size and launch path):
  - gate scores of all S tokens from A and W_router vs the oracle's (tolerance);
  - routing and align of all tokens, fed the oracle's scores, bit-exact;
  - the layer output of all S tokens on the GPU; the oracle computes the rows
    of a sample of tokens (first, last and random ones) on the same routing,
    compared element by element (fp32 output: the bar; bf16 output: the bar
    plus its own rounding)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import (DeviceLayer, bf16_output_excess, buffers, dev, host, parity, rms)

pytestmark = pytest.mark.gpu

N_SAMPLE = 24


def log(msg):
    print(msg, flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["prefill_bal", "prefill_skew", "decode", "dsv3"])
def test_fullsize(name):
    wl = wk.WORKLOADS[name]
    orc = oracle.default()
    log(f"[{name}] drawing inputs")
    li = wk.draw_layer(wl)
    log(f"[{name}] oracle gate scores, routing, align")
    G_o = orc.gate_logits(li.A, li.Wr, li.bias)
    ids_o, w_o = orc.topk_softmax(G_o, wl.k, wl.renormalize)
    kept = orc.capacity_mask(ids_o, wl.E, wl.capacity) if wl.capacity else None
    log(f"[{name}] copying inputs to the device")
    L = DeviceLayer(wl, li)

    # gate scores from A, W_router on the GPU
    buf = buffers(wl, out_f32=True)
    log(f"[{name}] GPU gate scores, block size {buf.shape.block_size}")
    moe.moe_gate_topk(buf.shape, L.A, L.Wr, L.bias, None, buf.logits, buf.topk_ids,
                      buf.topk_weights, buf.gate_ws)
    torch.cuda.synchronize()
    G = buf.logits.cpu().numpy().astype(np.float64)
    gerr = float(np.max(np.abs(G - G_o)) / rms(G_o))
    assert gerr <= 1e-4, f"gate scores err {gerr:.3e}"

    # routing + align on the oracle's scores: bit-exact
    buf.route(logits_in=dev(G_o))
    torch.cuda.synchronize()
    assert np.array_equal(buf.topk_ids.cpu().numpy(), ids_o)
    assert np.array_equal(buf.topk_weights.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    si, ei, n, cnt = orc.align(ids_o, wl.E, buf.shape.block_size, wl.capacity)
    assert int(buf.ntpp.item()) == n
    assert np.array_equal(buf.sorted_ids.cpu().numpy()[:n], si[:n])
    assert np.array_equal(buf.expert_ids.cpu().numpy()[: n // buf.shape.block_size],
                          ei[: n // buf.shape.block_size])
    assert np.array_equal(buf.expert_counts.cpu().numpy(), cnt)

    # the layer on all tokens, fp32 and bf16 outputs
    log(f"[{name}] GPU layer forward")
    O32 = host(L.forward(buf)).copy()
    buf16 = buffers(wl, out_f32=False)
    buf16.route(logits_in=dev(G_o))
    O16 = host(L.forward(buf16)).copy()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(O32)) and np.all(np.isfinite(O16))

    rng = np.random.default_rng(7)
    tokens = np.unique(np.concatenate([[0, wl.S - 1],
                                       rng.choice(wl.S, min(N_SAMPLE, wl.S), replace=False)]))
    log(f"[{name}] oracle rows for {tokens.size} sampled tokens")
    ref = orc.layer_rows(li.A, li.W_up, li.W_gate, li.W_down, ids_o, w_o, kept, tokens,
                         li.Ws_up, li.Ws_gate, li.Ws_down)
    err, tol = parity(wl, O32[tokens], ref)
    ex = bf16_output_excess(O16[tokens], ref)
    log(f"[{name}] sampled rows: fp32-output err {err:.3e} (tol {tol:.0e}), "
        f"bf16 output / bound {ex:.3f}, gate err {gerr:.2e}")
    assert err <= tol
    assert ex <= 1.0
    del L
    torch.cuda.empty_cache()
