"""Up/gate and down GEMMs in one persistent launch (MOE_FUSED_LAUNCH): the
same tiles as the two-launch form, so the output is compared bit for bit with
it, and with the oracle to the parity bar. Cases cover routed-only and
shared-expert task spaces, every block size, ragged tiles and K tails,
capacity drops, one m-block per expert (decode), more experts than
workgroups, and repeated calls on one workspace (the per-m-block readiness
counters are cleared by every call). The full-size prefill workloads run too,
in the configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, buffers, dev, host, parity

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _small(**kw):
    base = dict(name="small", S=200, H=136, D=200, E=12, k=3, dtype=wk.BF16, router_std=0.5)
    base.update(kw)
    return wk.Workload(**base)


def _outputs(wl, li, G, bm, calls=1):
    """Output of the two-launch and the one-launch forward on one routing
    (fp32 output); the one-launch form runs `calls` times on one workspace."""
    L = DeviceLayer(wl, li)
    res = []
    for fused in (False, True):
        buf = buffers(wl, bm, out_f32=True, fused_launch=fused)
        buf.forward_ws.fill_(0xFF)
        buf.route(logits_in=dev(G))
        for _ in range(calls if fused else 1):
            buf.O.fill_(float("nan"))
            res.append(host(L.forward(buf)).copy())
            # no down task gave up its bounded wait for the SwiGLU rows
            assert moe.forward_status(buf.forward_ws) == 0
    torch.cuda.synchronize()
    return res[0], res[1:]


CASES = [
    ("prefill_skew", 300, 128), ("prefill_bal", 600, 256), ("dsv3", 40, 256),
    ("dsv3", 100, 128), ("decode", 64, 16), ("decode", 64, 32),
]


@pytest.mark.parametrize("name,S,bm", CASES)
def test_fused_same_output(orc, name, S, bm):
    wl = wk.WORKLOADS[name].with_tokens(S)
    log(f"[fused {name} S={S} bm={bm}]")
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    two, ones = _outputs(wl, li, G, bm, calls=2)
    for o in ones:
        assert np.all(np.isfinite(o))
        assert np.array_equal(two, o)
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
    err, tol = parity(wl, ones[-1], ref["O"])
    assert err <= tol


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
def test_fused_ragged_shared(orc, bm):
    """H, D, D_shared off the 128-wide tiles, K tails, a shared expert."""
    wl = _small(D_shared=72)
    log(f"[fused ragged bm={bm}]")
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    two, ones = _outputs(wl, li, G, bm)
    assert np.array_equal(two, ones[0])
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
    err, tol = parity(wl, ones[0], ref["O"])
    assert err <= tol


@pytest.mark.parametrize("kw,bm", [(dict(capacity_factor=0.25), 32),
                                   (dict(S=300, E=600, k=4), 32),
                                   (dict(S=1, k=2), 64)])
def test_fused_drops_many_experts_single_token(orc, kw, bm):
    wl = _small(**kw)
    log(f"[fused {kw} bm={bm}]")
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    two, ones = _outputs(wl, li, G, bm)
    assert np.array_equal(two, ones[0])
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, logits=G)
    err, tol = parity(wl, ones[0], ref["O"])
    assert err <= tol


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["prefill_bal", "prefill_skew"])
def test_fused_fullsize_same_output(name):
    """Full size, the benchmark's block size: the one-launch output equals the
    two-launch output (whose full-size parity with the oracle is tested on
    sampled tokens) bit for bit, over two calls."""
    wl = wk.WORKLOADS[name]
    orc = oracle.default()
    log(f"[fused fullsize {name}] inputs and oracle scores")
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    log(f"[fused fullsize {name}] GPU")
    two, ones = _outputs(wl, li, G, None, calls=2)
    for o in ones:
        assert np.all(np.isfinite(o))
        assert np.array_equal(two, o)


@pytest.mark.parametrize("name,S,bm", [("prefill_skew", 300, 128), ("dsv3", 40, 256)])
def test_fused_atomic_combine(orc, name, S, bm):
    """One launch with the atomic combine (fp32 accumulator, order not fixed):
    to the parity bar against the oracle."""
    wl = wk.WORKLOADS[name].with_tokens(S)
    log(f"[fused atomic {name} S={S} bm={bm}]")
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    L = DeviceLayer(wl, li)
    buf = buffers(wl, bm, out_f32=True, atomic_combine=True, fused_launch=True)
    buf.forward_ws.fill_(0xFF)
    buf.route(logits_in=dev(G))
    buf.O.fill_(float("nan"))
    out = host(L.forward(buf)).copy()
    torch.cuda.synchronize()
    assert moe.forward_status(buf.forward_ws) == 0
    assert np.all(np.isfinite(out))
    ref = orc.layer(li.A, li.Wr, li.bias, li.W_up, li.W_gate, li.W_down, wl.k,
                    renormalize=wl.renormalize, capacity=wl.capacity, Ws_up=li.Ws_up,
                    Ws_gate=li.Ws_gate, Ws_down=li.Ws_down, logits=G)
    err, tol = parity(wl, out, ref["O"])
    assert err <= tol
