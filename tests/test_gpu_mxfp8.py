"""GPU parity of the MXFP8 path against the oracle's MXFP8 layer:
  - the quantiser (moe_quantize_mxfp8) bit for bit against the oracle's on
    token rows and on edge values (ties, saturation, zero and tiny blocks,
    signed zeros), bf16 and fp32 inputs;
  - the weight packing bit for bit after unpacking its documented layout;
  - the SwiGLU rows the up/gate GEMM quantises (read from the workspace):
    against the exact SwiGLU values of the oracle's quantised operands,
    nearly every code equal and every other one a neighbouring E4M3 value
    (a value within the GEMM's rounding error of an E4M3 boundary may go
    either way);
  - the layer forward on one shared routing (the GPU is fed the oracle's
    gate scores) against oracle.layer_rows_mx on the oracle's own
    quantisation of the same bf16 inputs, to the MXFP8 bar: fp32 output
    mean |g - o| <= 2e-3 RMS(o) and max |g - o| <= (4 / sqrt(D)) RMS(o);
    bf16 output to the max bar plus its own rounding. The two sides quantise
    A and the weights bit for bit alike; they differ by the fp32
    accumulation and the matrix cores' own rounding of the block products,
    and by the SwiGLU codes those move across a rounding boundary: a flip
    moves one element of a row by one E4M3 step (at most 1/8 of its block's
    largest value), which moves the down projection's outputs by about
    1/sqrt(D) of their RMS;
  - full-size token samples, repeat calls bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from tests.gpu_util import DeviceLayer, buffers, dev, host, pack_mxfp8, rms

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def _quantize_gpu(X):
    Xd = dev(X)
    R, K = X.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(Xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _edge_rows():
    """fp32 rows of 32-value blocks built around the rule's decisions."""
    rng = np.random.default_rng(31)
    rows = []
    for k in (-130, -100, -20, -7, 0, 3, 8, 20, 100, 126):
        b = np.zeros(32, dtype=np.float64)
        b[0] = 2.0 ** k                         # amax exactly a power of two
        b[1] = 1.9375 * 2.0 ** k                # saturates at 448
        grid = 2.0 ** (k - 8 - 3)               # E4M3 spacing of the top binade / 2^8
        b[2:10] = (np.arange(8) + 8.5) * grid * 2 ** 4   # half-way points (ties)
        b[10:20] = rng.standard_normal(10) * 2.0 ** k
        b[20] = -0.0
        b[21] = -(2.0 ** (k - 20))              # a tiny negative: rounds to -0
        b[22:] = rng.standard_normal(10) * 2.0 ** (k - 12)
        b[22:26] = (np.arange(4) + 0.5) * 2.0 ** (k - 8 - 9)  # ties in the subnormal range
        b[26] = 464 * 2.0 ** (k - 8)            # half-way to 480: saturates to 448
        b[27] = -447.9 * 2.0 ** (k - 8)         # just inside the top code
        rows.append(b)
    rows.append(np.zeros(32))
    X = np.concatenate(rows).reshape(-1, 64) if len(rows) % 2 == 0 else \
        np.concatenate(rows + [np.zeros(32)]).reshape(-1, 64)
    return X.astype(np.float32)


def test_quantize_rows_bitexact(orc):
    wl = wk.WORKLOADS["prefill_bal"].with_tokens(300)
    A, _, _ = wk.draw_routing_inputs(wl)          # bf16 token rows
    for X in (A, _edge_rows(), (np.random.default_rng(3).standard_normal((64, 512)) *
                                np.ldexp(1.0, np.random.default_rng(4).integers(
                                    -40, 40, (64, 1)))).astype(np.float32)):
        c, s = _quantize_gpu(X)
        rc, rs = orc.mx_quantize_rows(X)
        assert np.array_equal(s, rs), "scales differ"
        bad = np.argwhere(c != rc)
        assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: {c[tuple(bad[0])]} vs " \
                              f"{rc[tuple(bad[0])]}"


@pytest.mark.parametrize("E,K,N", [(3, 256, 384), (1, 2048, 128)])
def test_pack_weights_bitexact(orc, E, K, N):
    W = wk.f32_to_bf16_bits((np.random.default_rng(E * K).standard_normal((E, K, N)) /
                             np.sqrt(K)).astype(np.float32))
    W[0, :32, 5] = 0                                   # an all-zero block
    packed = pack_mxfp8(dev(W)).cpu().numpy()
    assert packed.size == moe.moe_mxfp8_weight_bytes(E, K, N) == E * (N // 128) * (K // 64) * 8448
    blk = packed.reshape(E, N // 128, K // 64, 8448)
    codes = blk[..., :8192].reshape(E, N // 128, K // 64, 128, 64)
    scales = blk[..., 8192:].reshape(E, N // 128, K // 64, 128, 2)
    # codes[e, j, s, c, kk] = code of W[e][64 s + kk][128 j + c]
    c_kn = codes.transpose(0, 2, 4, 1, 3).reshape(E, K, N)
    s_kn = scales.transpose(0, 2, 4, 1, 3).reshape(E, K // 32, N)
    rc, rs = orc.mx_quantize_cols(W)
    assert np.array_equal(s_kn, rs), "packed scales"
    assert np.array_equal(c_kn, rc), "packed codes"


def _oracle_mx(orc, li, ids, w, kept, tokens=None):
    q = orc.mx_quantize_cols
    sh = {}
    if li.Ws_up is not None:
        sh = dict(Wsu=q(li.Ws_up), Wsg=q(li.Ws_gate), Wsd=q(li.Ws_down))
    Aq, As = orc.mx_quantize_rows(li.A)
    return orc.layer_rows_mx(Aq, As, q(li.W_up), q(li.W_gate), q(li.W_down), ids, w, kept,
                             tokens, **sh)


# The MXFP8 bar (fp32 output; the bf16 output adds its own rounding to the max).
TOL_MX_MEAN = 2e-3


def tol_mx_max(wl):
    """The reach of a few flipped SwiGLU codes: 4 / sqrt(D) of the RMS (the
    narrower of the routed and shared intermediate sizes)."""
    d = min(wl.D, wl.D_shared) if wl.D_shared else wl.D
    return 4.0 / np.sqrt(d)


def mx_errors(g, o):
    """(max |g - o|, mean |g - o|) / RMS(o)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    r = max(rms(o), 1e-30)
    return float(np.max(np.abs(g - o))) / r, float(np.mean(np.abs(g - o))) / r


def mx_bf16_excess(g16, o, tol_max):
    g16 = np.asarray(g16, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    bound = tol_max * max(rms(o), 1e-30) + 2.0 ** -8 * np.abs(o)
    return float(np.max(np.abs(g16 - o) / bound))


def run_mx_case(orc, wl, bm=None, li=None, logits=None):
    li = li if li is not None else wk.draw_layer(wl)
    G_o = orc.gate_logits(li.A, li.Wr, li.bias) if logits is None else logits
    ids, w = orc.topk_softmax(G_o, wl.k, wl.renormalize)
    kept = orc.capacity_mask(ids, wl.E, wl.capacity) if wl.capacity else None
    L = DeviceLayer(wl, li)
    outs = {}
    for out_f32 in (True, False):
        buf = buffers(wl, bm, out_f32)
        buf.forward_ws.fill_(0xFF)
        buf.O.fill_(float("nan"))
        buf.route(logits_in=dev(G_o))
        outs[out_f32] = host(L.forward(buf)).copy()
        torch.cuda.synchronize()
        assert np.array_equal(buf.topk_ids.cpu().numpy(), ids), "routing differs"
        assert np.all(np.isfinite(outs[out_f32])), "non-finite output"
    ref = _oracle_mx(orc, li, ids, w, kept)
    emax, emean = mx_errors(outs[True], ref)
    tmax = tol_mx_max(wl)
    ex = mx_bf16_excess(outs[False], ref, tmax)
    log(f"  max err {emax:.3e} (bar {tmax:.3e}) mean err {emean:.3e} (of RMS), "
        f"bf16 output / bound {ex:.3f}")
    assert emax <= tmax and emean <= TOL_MX_MEAN
    assert ex <= 1.0, f"bf16 output beyond bar + own rounding: {ex:.3f}"
    return emax, tmax, ref, outs[True]


def _small(**kw):
    base = dict(name="small_mx", S=200, H=256, D=384, E=12, k=3, dtype=wk.BF16,
                router_std=0.5, mxfp8=True)
    base.update(kw)
    return wk.Workload(**base)


CASES = [("prefill_bal_mxfp8", 700, 256), ("prefill_bal_mxfp8", 333, 128),
         ("prefill_skew_mxfp8", 300, 128), ("prefill_skew_mxfp8", 300, 256),
         ("decode_mxfp8", 64, 64), ("decode_mxfp8", 1, 64)]


@pytest.mark.parametrize("name,S,bm", CASES)
def test_mx_layer_parity(orc, name, S, bm):
    wl = wk.WORKLOADS[name].with_tokens(S)
    log(f"[mxfp8 {name} S={S} BM={bm}]")
    err, tol, _, _ = run_mx_case(orc, wl, bm)
    log(f"  err {err:.3e} (tol {tol:.0e})")
    assert err <= tol


@pytest.mark.parametrize("bm", [64, 128, 256])
def test_mx_shared_expert_and_drops(orc, bm):
    """A shared expert, capacity drops, N and K over several tiles."""
    wl = _small(D_shared=256, capacity_factor=0.5)
    log(f"[mxfp8 shared+drops bm={bm}]")
    err, tol, _, _ = run_mx_case(orc, wl, bm)
    assert err <= tol


@pytest.mark.parametrize("bm", [128, 256])
def test_mx_hot_expert(orc, bm):
    """Every token picks expert 5 first: one expert over many m-blocks, most
    experts empty."""
    wl = _small(S=1500, E=40, k=2)
    li = wk.draw_layer(wl)
    rng = np.random.default_rng(0)
    G = rng.standard_normal((wl.S, wl.E)).astype(np.float32)
    G[:, 5] += 50.0
    log(f"[mxfp8 hot expert bm={bm}]")
    err, tol, _, _ = run_mx_case(orc, wl, bm, li=li, logits=G)
    assert err <= tol


def test_mx_repeat_calls_same_buffers(orc):
    wl = wk.WORKLOADS["prefill_skew_mxfp8"].with_tokens(200)
    li = wk.draw_layer(wl)
    L = DeviceLayer(wl, li)
    buf = buffers(wl, 128)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    outs = []
    for _ in range(2):
        buf.route(logits_in=dev(G))
        outs.append(host(L.forward(buf)).copy())
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["prefill_bal_mxfp8", "decode_mxfp8"])
def test_mx_fullsize_sampled(orc, name):
    """Full size, the benchmark's block size: all tokens on the GPU, the
    oracle's rows for a sample of tokens on the same routing."""
    wl = wk.WORKLOADS[name]
    log(f"[mxfp8 fullsize {name}] inputs, oracle scores")
    li = wk.draw_layer(wl)
    G_o = orc.gate_logits(li.A, li.Wr, li.bias)
    ids, w = orc.topk_softmax(G_o, wl.k, wl.renormalize)
    kept = orc.capacity_mask(ids, wl.E, wl.capacity) if wl.capacity else None
    L = DeviceLayer(wl, li)
    buf = buffers(wl, out_f32=True)
    buf.route(logits_in=dev(G_o))
    log(f"[mxfp8 fullsize {name}] GPU forward, block size {buf.shape.block_size}")
    O = host(L.forward(buf)).copy()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(O))
    rng = np.random.default_rng(7)
    tokens = np.unique(np.concatenate([[0, wl.S - 1], rng.choice(wl.S, min(12, wl.S),
                                                                 replace=False)]))
    log(f"[mxfp8 fullsize {name}] oracle rows for {tokens.size} tokens")
    ref = _oracle_mx(orc, li, ids, w, kept, tokens)
    emax, emean = mx_errors(O[tokens], ref)
    log(f"[mxfp8 fullsize {name}] max err {emax:.3e} mean err {emean:.3e} (of RMS)")
    assert emax <= tol_mx_max(wl) and emean <= TOL_MX_MEAN


def _ws_offsets(shape, cap_rows):
    """Byte offsets of the SwiGLU rows in an MXFP8 forward workspace (the
    section order the library lays out: counters, slots, kept flags, h)."""
    ru = lambda x: (x + 255) // 256 * 256
    F = shape.S * shape.k
    y = ru(2144 * 4)
    ys = y + ru(F * shape.H * 4)
    kept = ys + ru(shape.S * shape.H * 4 if shape.D_shared else 0)
    return kept + ru(F)


def test_mx_swiglu_codes(orc):
    """The quantised SwiGLU rows in the workspace against the exact SwiGLU
    of the oracle's quantised operands: each value within one E4M3 step of
    the oracle's code, or of the exact h once the GEMM's own rounding of u
    and g is allowed for; at least 98% of the codes equal."""
    wl = wk.WORKLOADS["prefill_skew_mxfp8"].with_tokens(300)
    li = wk.draw_layer(wl)
    G = orc.gate_logits(li.A, li.Wr, li.bias)
    ids, _ = orc.topk_softmax(G, wl.k, wl.renormalize)
    L = DeviceLayer(wl, li)
    buf = buffers(wl, 128, out_f32=True)
    buf.route(logits_in=dev(G))
    L.forward(buf)
    torch.cuda.synchronize()
    BM, D, H = 128, wl.D, wl.H
    ntpp = int(buf.ntpp.item())
    si = buf.sorted_ids.cpu().numpy()[:ntpp]
    cap = (wl.S * wl.k + wl.E * (BM - 1) + BM - 1) // BM * BM
    h0 = _ws_offsets(buf.shape, cap)
    ws = buf.forward_ws.cpu().numpy()
    hb = ws[h0:h0 + ntpp * (D // 64) * 66].reshape(ntpp // BM, D // 64, BM * 66)
    e4 = orc.e4m3_values(np.arange(256, dtype=np.uint8))
    Aq, As = orc.mx_quantize_rows(li.A)
    deq = lambda c, s, ax: e4[c] * np.ldexp(1.0, np.repeat(s.astype(int) - 127, 32, axis=ax))
    Ad = deq(Aq, As, -1)
    Wq = {n: orc.mx_quantize_cols(getattr(li, n)) for n in ("W_up", "W_gate")}
    same = total = 0
    for p in np.flatnonzero(si < wl.S * wl.k)[::7]:  # a sample of the kept rows
        f = si[p]
        t, j = divmod(int(f), wl.k)
        e = ids[t, j]
        b, r = divmod(int(p), BM)
        Wu = deq(Wq["W_up"][0][e], Wq["W_up"][1][e], 0)
        Wg = deq(Wq["W_gate"][0][e], Wq["W_gate"][1][e], 0)
        u64, g64 = Ad[t] @ Wu, Ad[t] @ Wg
        sig = 1 / (1 + np.exp(-u64))
        h64 = u64 * sig * g64
        h = h64.astype(np.float32)
        ref = deq(*orc.mx_quantize_rows(h[None, :]), -1)[0]
        # what the GPU's u and g may differ by: the matrix cores round each
        # block product and the fp32 sums (measured: 6e-5 of the largest
        # output on a one-tile test); bounded here by 2^-10 of the sum of
        # the terms' magnitudes, and carried through h = SiLU(u)·g
        du = np.abs(Ad[t]) @ np.abs(Wu) * 2.0 ** -10
        dg = np.abs(Ad[t]) @ np.abs(Wg) * 2.0 ** -10
        dh = np.abs(sig * (1 + u64 * (1 - sig)) * g64) * du + np.abs(u64 * sig) * dg
        codes = np.concatenate([hb[b, s][r * 64:(r + 1) * 64] for s in range(D // 64)])
        scl = np.concatenate([hb[b, s][BM * 64 + 2 * r:BM * 64 + 2 * r + 2]
                              for s in range(D // 64)])
        got = e4[codes] * np.ldexp(1.0, np.repeat(scl.astype(int) - 127, 32))
        rs = orc.mx_quantize_rows(h[None, :])[1][0]
        total += D
        same += int(np.sum(got == ref))
        # each value within one E4M3 step of the exact one's code: 1/8 of the
        # larger of the two, or one subnormal step of the coarser scale (a
        # block maximum within the GEMM's rounding of a power of two may have
        # moved the block's scale by one)
        sc = np.repeat(np.maximum(scl, rs).astype(int) - 127, 32)
        step = np.maximum(np.maximum(np.abs(ref), np.abs(got)) / 8, np.ldexp(1.0, sc - 9))
        bad = (np.abs(got - ref) > step) & (np.abs(got - h64) > step + dh)
        i = int(np.argmax(np.where(bad, np.abs(got - h64) - step - dh, -np.inf)))
        assert not bad.any(), (f"row {p} col {i}: code value {got[i]!r}, exact h {h64[i]!r}, "
                               f"oracle code value {ref[i]!r}, step {step[i]!r}, GEMM bound "
                               f"{dh[i]!r}")
        assert np.all(np.abs(scl.astype(int) - rs.astype(int)) <= 1), "a scale off by more than 1"
    log(f"  SwiGLU codes equal: {same} of {total}")
    assert same >= 0.98 * total
