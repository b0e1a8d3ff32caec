"""GPU parity of the routing steps: gate scores (tolerance), softmax top-k
(bit-exact when fed the oracle's scores) and their edge cases."""
import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DEV, buffers, dev, rms

pytestmark = pytest.mark.gpu

# each workload at a token count the oracle finishes in seconds (ragged sizes)
CASES = [("tiny_fp32", 64), ("prefill_bal", 700), ("prefill_skew", 300), ("decode", 64),
         ("dsv3", 100)]


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("name,S", CASES)
def test_gate_scores(orc, name, S):
    wl = wk.WORKLOADS[name].with_tokens(S)
    A, Wr, bias = wk.draw_routing_inputs(wl)
    G_o = orc.gate_logits(A, Wr, bias)
    buf = buffers(wl)
    moe.moe_gate_topk(buf.shape, dev(A), dev(Wr), dev(bias), None, buf.logits, buf.topk_ids,
                      buf.topk_weights, buf.gate_ws)
    torch.cuda.synchronize()
    G = buf.logits.cpu().numpy()
    err = float(np.max(np.abs(G.astype(np.float64) - G_o)) / rms(G_o))
    assert err <= 1e-4, f"{name}: gate scores max err / RMS = {err:.3e}"


def _topk_gpu(G, k, renormalize, dtype=wk.BF16):
    S, E = G.shape
    shape = moe.make_shape(S, 8, 8, E, k, renormalize=renormalize, block_size=16, dtype=dtype)
    ids = torch.empty((S, k), dtype=torch.int32, device=DEV)
    w = torch.empty((S, k), dtype=torch.float32, device=DEV)
    out = torch.empty((S, E), dtype=torch.float32, device=DEV)
    moe.moe_gate_topk(shape, None, None, None, dev(G), out, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), G), "logits_out must copy logits_in"
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name,S", CASES)
def test_topk_bitexact_on_oracle_scores(orc, name, S):
    wl = wk.WORKLOADS[name].with_tokens(S)
    A, Wr, bias = wk.draw_routing_inputs(wl)
    G_o = orc.gate_logits(A, Wr, bias)
    ids_o, w_o = orc.topk_softmax(G_o, wl.k, wl.renormalize)
    ids, w = _topk_gpu(G_o, wl.k, wl.renormalize)
    assert np.array_equal(ids, ids_o), f"{name}: top-k ids differ"
    assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32)), f"{name}: weights differ"


@pytest.mark.parametrize("E,k", [(1, 1), (3, 3), (8, 2), (100, 7), (256, 8), (1024, 32),
                                 (1000, 1), (65, 32)])
@pytest.mark.parametrize("renorm", [0, 1])
def test_topk_edge_shapes(orc, E, k, renorm):
    rng = np.random.default_rng(E * 100 + k)
    G = (rng.standard_normal((37, E)) * 2).astype(np.float32)
    ids_o, w_o = orc.topk_softmax(G, k, renorm)
    ids, w = _topk_gpu(G, k, renorm)
    assert np.array_equal(ids, ids_o)
    assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32))


def test_topk_ties(orc):
    rng = np.random.default_rng(5)
    G = rng.integers(-2, 3, size=(200, 64)).astype(np.float32)  # many exact ties
    G[:5] = 0.0                                                  # all equal
    G[5, :] = -0.0
    G[5, 7] = 0.0                                                # -0 and +0 compare equal
    for k in (1, 4, 17, 32):
        ids_o, w_o = orc.topk_softmax(G, k, 1)
        ids, w = _topk_gpu(G, k, 1)
        assert np.array_equal(ids, ids_o), f"k={k}"
        assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32))


def test_topk_fp32_mode_and_empty(orc):
    G = np.random.default_rng(1).standard_normal((5, 8)).astype(np.float32)
    ids_o, w_o = orc.topk_softmax(G, 2, 1)
    ids, w = _topk_gpu(G, 2, 1, dtype=wk.F32)
    assert np.array_equal(ids, ids_o)
    shape = moe.make_shape(0, 8, 8, 8, 2)
    assert moe.moe_gate_topk(shape, None, None, None, None, None, None, None) == 0


@pytest.mark.parametrize("name,S", CASES + [("prefill_bal", 16384), ("dsv3", 4096)])
def test_fused_gate_topk_consistent(orc, name, S):
    """Scores computed on the GPU (fused gate + top-k for bf16, E <= 256):
    the oracle's top-k of the GPU's own scores reproduces its ids and weights
    bit for bit."""
    wl = wk.WORKLOADS[name].with_tokens(S)
    A, Wr, bias = wk.draw_routing_inputs(wl)
    buf = buffers(wl)
    moe.moe_gate_topk(buf.shape, dev(A), dev(Wr), dev(bias), None, buf.logits, buf.topk_ids,
                      buf.topk_weights, buf.gate_ws)
    torch.cuda.synchronize()
    G = buf.logits.cpu().numpy()
    ids_o, w_o = orc.topk_softmax(G, wl.k, wl.renormalize)
    assert np.array_equal(buf.topk_ids.cpu().numpy(), ids_o)
    assert np.array_equal(buf.topk_weights.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


# Gate-score GEMM variants reached when the fused gate + top-k does not apply:
# bf16 with E > 256 (E % 8 == 0: the LDS-direct gate GEMM, three row-tile
# sizes by S), bf16 or fp32 with E % 8 != 0 (the register-staged GEMM with
# ragged columns), fp32 with E % 8 == 0; each followed by the separate top-k
# kernel. H = 200 leaves a K tail after three 64-wide stages.
GEMM_CASES = [(wk.BF16, 600, 8, 1), (wk.BF16, 600, 8, 300), (wk.BF16, 600, 8, 1500),
              (wk.BF16, 600, 8, 3300), (wk.BF16, 1000, 32, 77), (wk.BF16, 1020, 6, 150),
              (wk.BF16, 12, 3, 300), (wk.BF16, 12, 3, 1), (wk.F32, 12, 3, 300),
              (wk.F32, 5, 2, 77), (wk.F32, 64, 4, 200)]


@pytest.mark.parametrize("dtype,E,k,S", GEMM_CASES)
def test_gate_gemm_variants(orc, dtype, E, k, S):
    H = 200
    rng = np.random.default_rng([E, S, dtype])
    A = rng.standard_normal((S, H)).astype(np.float32)
    Wr = (rng.standard_normal((H, E)) / np.sqrt(H)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    if dtype == wk.BF16:
        A, Wr = wk.f32_to_bf16_bits(A), wk.f32_to_bf16_bits(Wr)
    G_o = orc.gate_logits(A, Wr, bias)
    shape = moe.make_shape(S, H, 8, E, k, block_size=16, dtype=dtype)
    ws_n = moe.moe_gate_workspace_bytes(shape)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=DEV) if ws_n else None
    G = torch.empty((S, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((S, k), dtype=torch.int32, device=DEV)
    w = torch.empty((S, k), dtype=torch.float32, device=DEV)
    moe.moe_gate_topk(shape, dev(A), dev(Wr), dev(bias), None, G, ids, w, ws)
    torch.cuda.synchronize()
    Gh = G.cpu().numpy()
    err = float(np.max(np.abs(Gh.astype(np.float64) - G_o)) / rms(G_o))
    assert err <= 1e-4, f"gate scores max err / RMS = {err:.3e}"
    # routing of the GPU's own scores: the oracle's top-k of them, bit for bit
    ids_o, w_o = orc.topk_softmax(Gh, k, 1)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
