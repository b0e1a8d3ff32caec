"""Pins of the CPU oracle against things other than itself.

Each ``check_*`` takes a loaded oracle and raises AssertionError when the
oracle disagrees with what the MoE pages and the mathematics fix:
hand-worked examples (tests/golden), textbook library routines on the same
inputs (numpy / torch float64 matmul, softmax, stable argsort, SiLU), closed
forms and invariants of the layer. ``CHECKS`` lists them all; the pin tests
run every check against the oracle, and the planted-mistake test runs them
against deliberately wrong builds of the oracle, each of which must fail at
least one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from sparse_expert_ffn_amd import workloads as wk

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f64(x):
    """Exact float64 view of an fp32 array or bf16 bit patterns."""
    if x.dtype == np.uint16:
        return wk.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _rand(shape, sigma, dtype, seed):
    x = (np.random.default_rng(seed).standard_normal(shape) * sigma).astype(np.float32)
    return wk.f32_to_bf16_bits(x) if dtype == wk.BF16 else x


def _tiny_layer(dtype, S=24, H=16, D=12, E=6, k=2, Ds=0, seed=1):
    r = lambda shape, s, i: _rand(shape, s, dtype, [seed, i])
    L = dict(A=r((S, H), 1.0, 0), Wr=r((H, E), 0.5, 1),
             W_up=r((E, H, D), 1 / math.sqrt(H), 2), W_gate=r((E, H, D), 1 / math.sqrt(H), 3),
             W_down=r((E, D, H), 1 / math.sqrt(D), 4))
    if Ds:
        L.update(Ws_up=r((H, Ds), 1 / math.sqrt(H), 5), Ws_gate=r((H, Ds), 1 / math.sqrt(H), 6),
                 Ws_down=r((Ds, H), 1 / math.sqrt(Ds), 7))
    return L


def _dense_reference(L, ids, w, kept=None):
    """Dense brute force: every expert on every token, masked by the routing
    (torch float64). O_s = sum_e mask[s,e] w[s,e] W_down^e SwiGLU(...) + shared."""
    A = torch.from_numpy(_f64(L["A"]))
    Wu = torch.from_numpy(_f64(L["W_up"]))
    Wg = torch.from_numpy(_f64(L["W_gate"]))
    Wd = torch.from_numpy(_f64(L["W_down"]))
    S, k = ids.shape
    E = Wu.shape[0]
    M = torch.zeros(S, E, dtype=torch.float64)
    for s in range(S):
        for j in range(k):
            if kept is None or kept[s, j]:
                M[s, int(ids[s, j])] += float(w[s, j])
    U = torch.einsum("sh,ehd->esd", A, Wu)
    G = torch.einsum("sh,ehd->esd", A, Wg)
    Y = torch.einsum("esd,edn->esn", torch.nn.functional.silu(U) * G, Wd)
    O = torch.einsum("se,esn->sn", M, Y)
    if L.get("Ws_up") is not None:
        su = A @ torch.from_numpy(_f64(L["Ws_up"]))
        sg = A @ torch.from_numpy(_f64(L["Ws_gate"]))
        O = O + (torch.nn.functional.silu(su) * sg) @ torch.from_numpy(_f64(L["Ws_down"]))
    return O.numpy()


def _layer(orc, L, k, capacity=0, renormalize=1, bias=None, logits=None):
    return orc.layer(L["A"], L["Wr"], bias, L["W_up"], L["W_gate"], L["W_down"], k,
                     renormalize=renormalize, capacity=capacity, Ws_up=L.get("Ws_up"),
                     Ws_gate=L.get("Ws_gate"), Ws_down=L.get("Ws_down"), logits=logits)


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1e-300, float(np.abs(b).max()))
    err = float(np.abs(a - b).max()) / scale
    assert err <= rtol, f"{what}: max error {err:.3e} (relative to max |ref|) > {rtol:.1e}"


# ------------------------------------------------------------ golden examples

def check_golden_layer(orc):
    fx = _golden("worked_layer.json")
    f32 = lambda x: np.asarray(x, dtype=np.float32)
    A, Wr = f32(fx["A"]), f32(fx["W_router"])
    Wu, Wg, Wd = f32(fx["W_up"]), f32(fx["W_gate"]), f32(fx["W_down"])
    out = orc.layer(A, Wr, None, Wu, Wg, Wd, fx["k"], renormalize=fx["renormalize"])
    ex = fx["expected"]
    assert np.array_equal(out["G"], f32(ex["G"])), "worked example: gate scores"
    assert np.array_equal(out["ids"], np.asarray(ex["ids"])), f"worked example: ids {out['ids']}"
    _close(out["w"], ex["weights"], 1e-7, "worked example: router weights")
    assert np.array_equal(out["w"], f32(ex["weights_fp32"])), "router weights rounded once to fp32"
    _close(out["O"], ex["O"], 1e-12, "worked example: layer output")


def check_golden_align(orc):
    for c in _golden("worked_align.json")["cases"]:
        ids = np.asarray(c["ids"], dtype=np.int32)
        si, ei, ntpp, counts = orc.align(ids, c["E"], c["BM"], c["C"])
        assert ntpp == c["ntpp"], f"{c['note']}: ntpp {ntpp}"
        assert si[:ntpp].tolist() == c["sorted_ids"], f"{c['note']}: sorted_ids {si[:ntpp]}"
        assert ei[: ntpp // c["BM"]].tolist() == c["expert_ids"], f"{c['note']}: expert_ids"
        assert counts.tolist() == c["counts"], f"{c['note']}: counts"


def check_golden_topk(orc):
    for c in _golden("worked_topk.json")["cases"]:
        G = np.asarray(c["G"], dtype=np.float32)
        ids, w = orc.topk_softmax(G, c["k"], 1)
        assert ids.tolist() == c["ids"], f"ties: {ids.tolist()} != {c['ids']}"
        if "weights" in c:
            assert w.tolist() == c["weights"], f"tie weights {w.tolist()}"


# ------------------------------------------------------------ library routines

def check_logits_matmul(orc):
    for dtype in (wk.F32, wk.BF16):
        A = _rand((37, 96), 1.0, dtype, [2, 0])
        Wr = _rand((96, 24), 0.1, dtype, [2, 1])
        bias = np.linspace(-1, 1, 24).astype(np.float32)
        G = orc.gate_logits(A, Wr)
        ref = (_f64(A) @ _f64(Wr)).astype(np.float32)
        _close(G, ref, 2e-7, "gate scores vs numpy float64 matmul")
        Gb = orc.gate_logits(A, Wr, bias)
        assert np.array_equal(Gb, G + bias), "router bias must be an fp32 add to the scores"


def check_router_bias(orc):
    """The router bias is added to the fp32 scores before ranking. Two closed
    forms of that reading: a bias equal for every expert shifts all scores
    alike, so the choice and the renormalised weights stay those of the
    softmax of the unbiased scores; a bias far above the score spread on one
    expert puts that expert in every token's first slot, and the remaining
    slots follow the unbiased ranking (stable argsort) of the other experts."""
    A = _rand((64, 32), 1.0, wk.F32, [5, 0])
    Wr = _rand((32, 16), 0.05, wk.F32, [5, 1])
    G = orc.gate_logits(A, Wr)
    k = 4
    ids, w = orc.topk_softmax(G, k, 1)
    # 0.25 is exact in fp32 and small next to the scores' ulp range: the
    # shifted scores are exact, so the ranking is unchanged
    Gc = orc.gate_logits(A, Wr, np.full(16, 0.25, dtype=np.float32))
    assert np.array_equal(Gc, (G.astype(np.float64) + 0.25).astype(np.float32))
    ids_c, w_c = orc.topk_softmax(Gc, k, 1)
    assert np.array_equal(ids_c, ids), "an equal bias on every expert changes no choice"
    sel = np.take_along_axis(G.astype(np.float64), ids, axis=1)
    ref = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    _close(w_c, ref, 1.2e-7, "renormalised weights under an equal bias")
    hot = 11
    b = np.zeros(16, dtype=np.float32)
    b[hot] = 1000.0
    ids_h, _ = orc.topk_softmax(orc.gate_logits(A, Wr, b), k, 1)
    assert np.all(ids_h[:, 0] == hot), "a dominant bias puts its expert in slot 0"
    rest = np.delete(G.astype(np.float64), hot, axis=1)
    order = np.argsort(-rest, axis=1, kind="stable")[:, : k - 1]
    order = order + (order >= hot)
    assert np.array_equal(ids_h[:, 1:], order), "other slots follow the unbiased ranking"


def check_topk_library(orc):
    rng = np.random.default_rng(3)
    for E, k in ((8, 2), (24, 5), (64, 8), (5, 5)):
        G = rng.standard_normal((50, E)).astype(np.float32)
        ids, w = orc.topk_softmax(G, k, 1)
        ref_ids = np.argsort(-G.astype(np.float64), axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref_ids), f"top-{k} of {E} vs stable argsort"
        full = torch.softmax(torch.from_numpy(G.astype(np.float64)), dim=1).numpy()
        sel = np.take_along_axis(full, ref_ids, axis=1)
        # renormalised weights = full softmax at the chosen ids, rescaled to sum 1
        _close(w, sel / sel.sum(axis=1, keepdims=True), 1.2e-7, "renormalised softmax")
        ids0, w0 = orc.topk_softmax(G, k, 0)
        assert np.array_equal(ids0, ids)
        _close(w0, sel, 1.2e-7, "plain softmax weights at the chosen ids")
        if k == E:  # k = E with renormalisation is the full softmax
            _close(np.take_along_axis(w, np.argsort(ids, axis=1), axis=1), full, 1.2e-7,
                   "k=E softmax")


def check_topk_invariants(orc):
    rng = np.random.default_rng(4)
    G = (rng.standard_normal((200, 64)) * 0.9).astype(np.float32)
    ids, w = orc.topk_softmax(G, 8, 1)
    assert ids.min() >= 0 and ids.max() < 64
    assert all(len(set(r)) == 8 for r in ids.tolist()), "ids must be distinct"
    g = np.take_along_axis(G, ids, axis=1)
    assert np.all(np.diff(g, axis=1) <= 0), "slots ordered by descending score"
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1) <= 8 * 2 ** -24), "sum to 1"


# ---------------------------------------------------------------------- align

def _align_bruteforce(ids, E, BM, C):
    flat = ids.reshape(-1)
    F = flat.size
    order = np.argsort(flat, kind="stable")  # by expert, ascending f inside
    counts = np.bincount(flat, minlength=E)
    kept = np.minimum(counts, C) if C else counts
    pad = -(-kept // BM) * BM
    off = np.concatenate([[0], np.cumsum(pad)])
    si = np.full(int(off[-1]), F, dtype=np.int64)
    start = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        mine = order[start[e]: start[e + 1]][: kept[e]]
        si[off[e]: off[e] + kept[e]] = mine
    ei = np.repeat(np.arange(E), pad // BM)
    return si, ei, int(off[-1]), kept


def check_align_bruteforce(orc):
    for dist in ("random", "alternating_empty", "skewed", "mostly_empty", "all_to_one"):
        for (S, k, E, BM, C) in ((300, 2, 24, 16, 0), (257, 4, 64, 48, 0), (500, 2, 8, 1, 0),
                                 (256, 2, 64, 32, 6), (129, 8, 100, 128, 0)):
            ids = wk.draw_topk_ids(S, k, E, dist, seed=S)
            si, ei, ntpp, counts = orc.align(ids, E, BM, C)
            rsi, rei, rntpp, rcounts = _align_bruteforce(ids, E, BM, C)
            tag = f"{dist} S={S} k={k} E={E} BM={BM} C={C}"
            assert ntpp == rntpp, f"{tag}: ntpp"
            assert np.array_equal(si[:ntpp], rsi), f"{tag}: sorted_ids"
            assert np.array_equal(ei[: ntpp // BM], rei), f"{tag}: expert_ids"
            assert np.array_equal(counts, rcounts), f"{tag}: counts"
            # invariants the pages fix: counts sum to S*k (dropless); every block
            # holds one expert's entries then sentinels S*k
            if not C:
                assert counts.sum() == S * k
            blk = si[:ntpp].reshape(-1, BM)
            for b in range(blk.shape[0]):
                real = blk[b][blk[b] != S * k]
                assert np.all(ids.reshape(-1)[real] == ei[b])
                assert np.all(blk[b][: real.size] == real), "sentinels trail the block"


def check_capacity_mask(orc):
    ids = wk.draw_topk_ids(400, 2, 16, "skewed", seed=9)
    for C in (1, 7, 50, 800):
        kept = orc.capacity_mask(ids, 16, C)
        flat = ids.reshape(-1)
        ref = np.zeros(flat.size, dtype=np.uint8)
        for e in range(16):
            where = np.nonzero(flat == e)[0]  # ascending token order
            ref[where[:C]] = 1
        assert np.array_equal(kept.reshape(-1), ref), f"capacity C={C}"
        si, ei, ntpp, counts = orc.align(ids, 16, 4, C)
        kept_f = set(np.nonzero(ref)[0].tolist())
        in_sorted = set(x for x in si[:ntpp].tolist() if x != flat.size)
        assert in_sorted == kept_f, "align keeps exactly the capacity mask's assignments"


# ---------------------------------------------------------------------- layer

def check_layer_dense(orc):
    for dtype in (wk.F32, wk.BF16):
        for (S, H, D, E, k, C, Ds) in ((24, 16, 12, 6, 2, 0, 0), (40, 8, 20, 5, 3, 9, 0),
                                       (17, 12, 8, 4, 2, 0, 10)):
            L = _tiny_layer(dtype, S, H, D, E, k, Ds, seed=S)
            out = _layer(orc, L, k, capacity=C)
            ref = _dense_reference(L, out["ids"], out["w"], out["kept"])
            _close(out["O"], ref, 1e-12, f"dense brute force dtype={dtype} E={E} k={k} C={C}")


def check_plain_ffn(orc):
    """E = k = 1: the layer is a plain SwiGLU FFN (weight 1)."""
    L = _tiny_layer(wk.F32, S=9, H=10, D=7, E=1, k=1, seed=5)
    out = _layer(orc, L, 1)
    assert np.all(out["w"] == 1.0)
    A = torch.from_numpy(_f64(L["A"]))
    u = A @ torch.from_numpy(_f64(L["W_up"][0]))
    g = A @ torch.from_numpy(_f64(L["W_gate"][0]))
    ref = (torch.nn.functional.silu(u) * g) @ torch.from_numpy(_f64(L["W_down"][0]))
    _close(out["O"], ref.numpy(), 1e-12, "E=k=1 plain FFN")


def check_down_scaling(orc):
    L = _tiny_layer(wk.BF16, seed=6)
    base = _layer(orc, L, 2)["O"]
    L2 = dict(L)
    L2["W_down"] = wk.f32_to_bf16_bits(wk.bf16_bits_to_f32(L["W_down"]) * 2)
    assert np.array_equal(_layer(orc, L2, 2)["O"], 2 * base), "W_down -> 2 W_down gives O -> 2 O"


def check_expert_permutation(orc):
    L = _tiny_layer(wk.F32, S=30, E=7, k=3, seed=7)
    base = _layer(orc, L, 3)["O"]
    p = np.array([3, 6, 0, 5, 1, 4, 2])
    Lp = dict(L, Wr=np.ascontiguousarray(L["Wr"][:, p]),
              W_up=np.ascontiguousarray(L["W_up"][p]), W_gate=np.ascontiguousarray(L["W_gate"][p]),
              W_down=np.ascontiguousarray(L["W_down"][p]))
    _close(_layer(orc, Lp, 3)["O"], base, 1e-13, "expert relabelling leaves O unchanged")


def check_token_permutation(orc):
    L = _tiny_layer(wk.F32, S=25, seed=8)
    base = _layer(orc, L, 2)["O"]
    p = np.random.default_rng(0).permutation(25)
    Lp = dict(L, A=np.ascontiguousarray(L["A"][p]))
    _close(_layer(orc, Lp, 2)["O"], base[p], 1e-13, "token permutation permutes O rows")


def check_capacity_limits(orc):
    L = _tiny_layer(wk.F32, S=20, E=4, k=2, seed=10)
    dropless = _layer(orc, L, 2)["O"]
    assert np.array_equal(_layer(orc, L, 2, capacity=20)["O"], dropless), "C >= S is dropless"
    out1 = _layer(orc, L, 2, capacity=1)
    assert int(out1["kept"].sum()) == sum(1 for e in range(4) if (out1["ids"] == e).any())


def check_zero_expert(orc):
    L = _tiny_layer(wk.F32, S=30, E=5, k=2, seed=11)
    out = _layer(orc, L, 2)
    Lz = dict(L, W_down=L["W_down"].copy())
    Lz["W_down"][2] = 0
    kept = (out["ids"] != 2).astype(np.uint8)
    ref = orc.layer_rows(L["A"], L["W_up"], L["W_gate"], L["W_down"], out["ids"], out["w"], kept)
    _close(_layer(orc, Lz, 2)["O"], ref, 1e-13, "an all-zero expert contributes 0")


def check_shared_only(orc):
    L = _tiny_layer(wk.F32, S=15, H=12, D=8, E=4, k=2, Ds=6, seed=12)
    L["W_down"] = np.zeros_like(L["W_down"])
    O = _layer(orc, L, 2)["O"]
    A = torch.from_numpy(_f64(L["A"]))
    u = A @ torch.from_numpy(_f64(L["Ws_up"]))
    g = A @ torch.from_numpy(_f64(L["Ws_gate"]))
    ref = (torch.nn.functional.silu(u) * g) @ torch.from_numpy(_f64(L["Ws_down"]))
    _close(O, ref.numpy(), 1e-12, "shared expert alone is a plain FFN with weight 1")


def check_layer_rows_subset(orc):
    """Rows of a listed token subset, in a shuffled order with repeats: row i
    of the result is token tokens[i]'s output, with its own routing, capacity
    flags and shared expert (dense brute force, and the full run's rows)."""
    for dtype in (wk.F32, wk.BF16):
        L = _tiny_layer(dtype, S=31, H=12, D=10, E=5, k=2, Ds=6, seed=14)
        out = _layer(orc, L, 2, capacity=9)
        assert out["kept"] is not None and out["kept"].sum() < 31 * 2
        p = np.array([30, 3, 17, 3, 0, 22, 9], dtype=np.int64)
        rows = orc.layer_rows(L["A"], L["W_up"], L["W_gate"], L["W_down"], out["ids"],
                              out["w"], out["kept"], p, L["Ws_up"], L["Ws_gate"], L["Ws_down"])
        ref = _dense_reference(L, out["ids"], out["w"], out["kept"])
        _close(rows, ref[p], 1e-12, f"token subset rows vs dense brute force dtype={dtype}")
        assert np.array_equal(rows, out["O"][p]), "token subset rows vs the full run"


def check_weights_sum_one_layer(orc):
    """Identical experts: with weights summing to 1, O equals one expert's FFN."""
    L = _tiny_layer(wk.F32, S=12, H=8, D=6, E=4, k=3, seed=13)
    for key in ("W_up", "W_gate", "W_down"):
        L[key] = np.ascontiguousarray(np.repeat(L[key][:1], 4, axis=0))
    O = _layer(orc, L, 3)["O"]
    one = orc.layer_rows(L["A"], L["W_up"][:1].copy(), L["W_gate"][:1].copy(),
                         L["W_down"][:1].copy(), np.zeros((12, 1), np.int32),
                         np.ones((12, 1), np.float32))
    _close(O, one, 1e-6, "identical experts with weights summing to 1")


# ---------------------------------------------------------------------- MXFP8

def _e4m3_table():
    """Every finite non-negative E4M3 value, from torch's float8_e4m3fn
    (a library's decoding of the format), indexed by code 0x00 .. 0x7E."""
    codes = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return codes.to(torch.float64).numpy()


def check_e4m3_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2, "NaN codes 0x7F, 0xFF"
    assert np.array_equal(got[~nan], ref[~nan]), "E4M3 values vs torch float8_e4m3fn"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signed zero"


def check_e4m3_encode(orc):
    """Nearest E4M3 value by brute force over the 127 magnitudes, ties to the
    even code; |x| >= 448 saturates; zero results keep the sign. Inputs: every
    value, every midpoint between neighbours (the ties), random values over
    all binades and the subnormal range, values past 448."""
    table = _e4m3_table()
    mids = (table[1:] + table[:-1]) / 2
    rng = np.random.default_rng(21)
    rand = np.ldexp(rng.random(3000) + 0.5, rng.integers(-14, 10, 3000))
    x = np.concatenate([table, mids, rand, [448.0, 449.0, 463.9, 464.0, 500.0, 1e30,
                                            2.0 ** -10, 2.0 ** -11]])
    x = np.concatenate([x, -x, [0.0, -0.0]])
    got = orc.e4m3_encode(x)
    a = np.abs(x)
    ref = np.empty(x.size, dtype=np.uint8)
    for i, v in enumerate(a):
        if v >= 448.0:
            c = 0x7E
        else:
            d = np.abs(table - v)
            best = np.flatnonzero(d == d.min())
            c = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        ref[i] = c | (0x80 if np.signbit(x[i]) else 0)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"E4M3 rounding: {x[bad[:5]]} -> {got[bad[:5]]}, expected {ref[bad[:5]]}"
    # a library's rounding of the same values inside the finite range
    inr = a < 464.0
    lib = torch.from_numpy(x[inr]).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(got[inr], lib.numpy()), "E4M3 rounding vs torch float8_e4m3fn"


def check_mx_golden(orc):
    for b in _golden("worked_mxfp8.json")["blocks"]:
        v = np.asarray(b["values"], dtype=np.float32)[None, :]
        c, s = orc.mx_quantize_rows(v)
        assert int(s[0, 0]) == b["scale_code"], f"scale of {b['values'][:4]}: {s[0, 0]}"
        assert c[0].tolist() == b["codes"], f"codes of {b['values'][:4]}: {c[0][:6]}"
        # the same block along a column of a [32][N] matrix
        cc, sc = orc.mx_quantize_cols(np.ascontiguousarray(np.repeat(v.T, 3, axis=1)))
        assert np.all(sc == b["scale_code"]) and np.all(cc[:, 1] == c[0])


def _mx_reference(x64, axis):
    """The MX rule written with numpy / torch pieces: scale exponent from the
    block maximum's binary exponent, elements by torch's E4M3 rounding after
    the saturation at 448 (torch has no saturation of its own)."""
    x = np.moveaxis(np.asarray(x64, dtype=np.float64), axis, -1)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e2 = np.frexp(amax)
    se = np.where(amax > 0, np.clip(e2 - 1 - 8, -127, 127), -127)
    y = np.clip(blocks / np.ldexp(1.0, se)[..., None], -448.0, 448.0)
    q = torch.from_numpy(y).to(torch.float32).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).numpy().reshape(x.shape)
    vals = q.to(torch.float64).numpy() * np.ldexp(1.0, se)[..., None]
    return (np.moveaxis(codes, -1, axis), np.moveaxis((se + 127).astype(np.uint8), -1, axis),
            np.moveaxis(vals.reshape(x.shape), -1, axis))


def check_mx_quantize_reference(orc):
    rng = np.random.default_rng(22)
    for dtype in (wk.F32, wk.BF16):
        X = _rand((7, 96), 1.0, dtype, [22, 0])
        X64 = _f64(X).copy()
        X64[0, :32] = 0.0                     # an all-zero block
        X64[1, 32:64] *= 2.0 ** -120          # a block near the bottom of the scale range
        X64[2, 64:] = np.ldexp(1.0, rng.integers(-6, 6, 32))  # exact after scaling
        Xq = X64.astype(np.float32)
        c, s = orc.mx_quantize_rows(Xq)
        rc, rs, _ = _mx_reference(Xq, -1)
        assert np.array_equal(s, rs), "MX scales vs the reference rule"
        assert np.array_equal(c, rc), "MX codes vs the reference rule"
        back = orc.e4m3_values(c[2, 64:]) * np.ldexp(1.0, int(s[2, 2]) - 127)
        assert np.array_equal(back, X64[2, 64:]), "powers of two survive quantisation"
        cc, sc = orc.mx_quantize_cols(np.ascontiguousarray(Xq.T))
        assert np.array_equal(cc, c.T) and np.array_equal(sc, s.T), "rows vs columns"
    # scaling a block by 2^j moves its scale by j and keeps its codes
    X = _rand((4, 64), 1.0, wk.F32, [22, 1])
    c0, s0 = orc.mx_quantize_rows(X)
    c1, s1 = orc.mx_quantize_rows((X.astype(np.float64) * 2.0 ** 5).astype(np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 5)


def _mx_layer_reference(orc_q, L, ids, w, kept):
    """Dense brute force of the MXFP8 layer (torch float64): every expert on
    every token masked by the routing; operands dequantised with the reference
    rule; u, g and the SwiGLU value rounded to fp32, the SwiGLU rows
    requantised along D before the down projection."""
    A = _mx_reference(_f64(L["A"]), -1)[2]
    deq = lambda W: _mx_reference(_f64(W), -2)[2]
    Wu, Wg, Wd = deq(L["W_up"]), deq(L["W_gate"]), deq(L["W_down"])
    S, k = ids.shape
    E = Wu.shape[0]
    M = np.zeros((S, E))
    for s in range(S):
        for j in range(k):
            if kept is None or kept[s, j]:
                M[s, int(ids[s, j])] += float(w[s, j])

    def ffn(a, wu, wg, wd):
        u = (a @ wu).astype(np.float32).astype(np.float64)
        g = (a @ wg).astype(np.float32).astype(np.float64)
        h = (torch.nn.functional.silu(torch.from_numpy(u)).numpy() * g).astype(np.float32)
        return _mx_reference(h.astype(np.float64), -1)[2] @ wd

    O = sum(M[:, e:e + 1] * ffn(A, Wu[e], Wg[e], Wd[e]) for e in range(E))
    if L.get("Ws_up") is not None:
        O = O + ffn(A, deq(L["Ws_up"]), deq(L["Ws_gate"]), deq(L["Ws_down"]))
    return O


def _mx_layer(orc, L, ids, w, kept=None, tokens=None):
    q = orc.mx_quantize_cols
    sh = {}
    if L.get("Ws_up") is not None:
        sh = dict(Wsu=q(L["Ws_up"]), Wsg=q(L["Ws_gate"]), Wsd=q(L["Ws_down"]))
    Aq, As = orc.mx_quantize_rows(L["A"])
    return orc.layer_rows_mx(Aq, As, q(L["W_up"]), q(L["W_gate"]), q(L["W_down"]), ids, w,
                             kept, tokens, **sh)


def check_layer_mx_dense(orc):
    for dtype in (wk.F32, wk.BF16):
        for (S, H, D, E, k, C, Ds) in ((20, 64, 32, 4, 2, 0, 0), (17, 32, 64, 5, 3, 6, 32)):
            L = _tiny_layer(dtype, S, H, D, E, k, Ds, seed=S + H)
            out = _layer(orc, L, k, capacity=C)  # the routing
            got = _mx_layer(orc, L, out["ids"], out["w"], out["kept"])
            ref = _mx_layer_reference(orc, L, out["ids"], out["w"], out["kept"])
            _close(got, ref, 1e-12, f"MXFP8 layer vs dense brute force dtype={dtype} Ds={Ds}")
            # against the unquantised layer: the format's own error, a few % of RMS
            rms = float(np.sqrt(np.mean(out["O"] ** 2)))
            err = float(np.max(np.abs(got - out["O"]))) / rms
            assert 0.0 < err < 0.5, f"MXFP8 layer vs unquantised: {err:.3f} of RMS"


CHECKS = [check_golden_layer, check_golden_align, check_golden_topk, check_logits_matmul,
          check_topk_library, check_topk_invariants, check_align_bruteforce,
          check_capacity_mask, check_layer_dense, check_plain_ffn, check_down_scaling,
          check_expert_permutation, check_token_permutation, check_capacity_limits,
          check_zero_expert, check_shared_only, check_weights_sum_one_layer,
          check_router_bias, check_layer_rows_subset, check_e4m3_decode, check_e4m3_encode,
          check_mx_golden, check_mx_quantize_reference, check_layer_mx_dense]
