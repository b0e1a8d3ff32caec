"""Seeded input generator: determinism, shapes, distributions, bf16 rounding."""
import math

import numpy as np

from sparse_expert_ffn_amd import workloads as wk


def test_same_seed_same_bytes():
    wl = wk.WORKLOADS["tiny_fp32"]
    a = wk.draw_layer(wl)
    b = wk.draw_layer(wl)
    for key in ("A", "Wr", "W_up", "W_gate", "W_down"):
        assert getattr(a, key).tobytes() == getattr(b, key).tobytes(), key


def test_per_expert_streams_independent_of_subset():
    wl = wk.WORKLOADS["decode"].with_tokens(4)
    full = wk.draw_experts(wl, wk.T_WUP, 6, (8, 4), 0.5)
    part = wk.draw_experts(wl, wk.T_WUP, 6, (8, 4), 0.5, experts=[5, 2])
    assert np.array_equal(part[0], full[5]) and np.array_equal(part[1], full[2])


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e-3], dtype=np.float32)
    b = wk.f32_to_bf16_bits(x)
    back = wk.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to even (1.0)
    assert back[1] == 1.0
    assert back[2] == 1.0078125
    assert back[0] == 1.0 and back[4] == -2.5
    assert abs(back[5] - x[5]) <= abs(x[5]) * 2 ** -8


def test_distributions():
    wl = wk.WORKLOADS["prefill_bal"].with_tokens(256)
    A, Wr, b = wk.draw_routing_inputs(wl)
    assert A.dtype == np.uint16 and A.shape == (256, 2048) and Wr.shape == (2048, 64)
    assert b is None
    a = wk.bf16_bits_to_f32(A)
    assert abs(a.std() - 1.0) < 0.02
    assert abs(wk.bf16_bits_to_f32(Wr).std() - 0.02) < 0.001
    assert wl.capacity == math.ceil(256 * 2 / 64)
    assert wk.WORKLOADS["prefill_bal"].capacity == 512


def test_zipf_bias():
    wl = wk.WORKLOADS["prefill_skew"]
    b = wk.router_bias(wl)
    r = np.arange(1, 65, dtype=np.float64)
    p = r ** -1.2 / (r ** -1.2).sum()
    assert np.allclose(b, 3 * np.log(p), rtol=1e-6)
    assert np.all(np.diff(b) < 0)


def test_topk_id_distributions():
    for dist in wk.ID_DISTS:
        ids = wk.draw_topk_ids(100, 4, 24, dist, seed=1)
        assert ids.shape == (100, 4) and ids.dtype == np.int32
        assert all(len(set(r)) == 4 for r in ids.tolist())
        assert ids.min() >= 0 and ids.max() < 24
    ids = wk.draw_topk_ids(100, 2, 24, "alternating_empty")
    assert np.all(ids % 2 == 0)
