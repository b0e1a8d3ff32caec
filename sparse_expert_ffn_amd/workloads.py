"""Seeded synthetic workloads for the fused MoE layer.

This module only draws inputs. It holds none of the layer's arithmetic, and it
serves both the CPU oracle (``oracle/``) and the HIP library alike: tests and
the benchmark draw tensors here and hand the same bytes to each side.

Workloads (shapes and value distributions as the MoE pages state them):

* ``tiny_fp32``      S=64, H=128, D=256, E=8, top-2, fp32, no shared expert.
* ``prefill_bal``    S=16384, H=2048, D=2048, E=64, top-2, bf16, capacity factor
                     1.0 (FlashMoE evaluation setup: H=2048, FFN=2048, top-2,
                     CF 1.0, 16K tokens).
* ``prefill_skew``   S=8192, H=2048, D=1024, E=64, top-4, bf16, router bias
                     b_e = 3 ln(Zipf_1.2 rank weight of expert e).
* ``decode``         S=64, H=2048, D=768, E=256, top-8, bf16.
* ``dsv3``           S=4096, H=7168, D=2048, E=256, top-8 + one shared expert of
                     the same intermediate size, bf16 (DeepSeek-V3-style layer,
                     Mixture-of-Kittens page, "Overlapping compute and
                     communication in MoE").

Generator recipe: every tensor t (and every expert e of a per-expert weight)
has its own numpy PCG64 stream ``default_rng([seed, t, e])``; values are
``standard_normal`` float32 draws times sigma (float32 multiply). bf16 tensors
are the round-to-nearest-even bf16 of those float32 values, stored as uint16
bit patterns. The second parameter of N(0, s) is a standard deviation.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = 0
BF16 = 1

# tensor ids of the per-tensor random streams
T_A, T_WR, T_WUP, T_WGATE, T_WDOWN, T_WSUP, T_WSGATE, T_WSDOWN = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    S: int
    H: int
    D: int
    E: int
    k: int
    dtype: int                  # F32 or BF16
    D_shared: int = 0           # 0: no shared expert
    capacity_factor: float = 0.0  # 0: dropless
    router_std: float = 0.02    # std of W_router
    zipf_bias: float = 0.0      # b_e = zipf_bias * ln p_{e+1}; 0 = no bias
    zipf_s: float = 1.2
    renormalize: int = 1
    seed: int = 0
    mxfp8: bool = False         # expert GEMMs in MXFP8 (inputs still drawn in bf16)

    @property
    def capacity(self) -> int:
        """Slots per expert, C = ceil(CF * S * k / E); 0 means dropless."""
        if self.capacity_factor <= 0:
            return 0
        return int(math.ceil(self.capacity_factor * self.S * self.k / self.E))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def with_tokens(self, S: int, name: str | None = None) -> "Workload":
        """Same layer and distributions with a different token count."""
        return dataclasses.replace(self, S=S, name=name or f"{self.name}_S{S}")

    def describe(self) -> dict:
        return {"workload": self.name, "S": self.S, "H": self.H, "D": self.D,
                "E": self.E, "k": self.k, "D_shared": self.D_shared,
                "capacity": self.capacity,
                "dtype": "f32" if self.dtype == F32 else ("mxfp8" if self.mxfp8 else "bf16")}


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", S=64, H=128, D=256, E=8, k=2, dtype=F32,
                          router_std=0.02),
    "prefill_bal": Workload("prefill_bal", S=16384, H=2048, D=2048, E=64, k=2,
                            dtype=BF16, capacity_factor=1.0, router_std=0.02),
    "prefill_skew": Workload("prefill_skew", S=8192, H=2048, D=1024, E=64, k=4,
                             dtype=BF16, router_std=0.02, zipf_bias=3.0),
    "decode": Workload("decode", S=64, H=2048, D=768, E=256, k=8, dtype=BF16,
                       router_std=1.0 / math.sqrt(2048)),
    "dsv3": Workload("dsv3", S=4096, H=7168, D=2048, E=256, k=8, dtype=BF16,
                     D_shared=2048, router_std=1.0 / math.sqrt(7168)),
}
# The same layers with MXFP8 expert GEMMs (the Mixture-of-Kittens page's
# low-precision format): identical inputs, the expert weights and the GEMM
# operands quantised to MXFP8.
for _n in ("prefill_bal", "prefill_skew", "decode", "dsv3"):
    WORKLOADS[_n + "_mxfp8"] = dataclasses.replace(WORKLOADS[_n], name=_n + "_mxfp8", mxfp8=True)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(seed: int, tid: int, sub: int, n: int, sigma: float, dtype: int) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, sub])
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    return x


def _nthreads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw_tensor(wl: Workload, tid: int, shape, sigma: float, sub: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    return _draw(wl.seed, tid, sub, n, sigma, wl.dtype).reshape(shape)


def draw_experts(wl: Workload, tid: int, n_exp: int, shape, sigma: float,
                 experts=None, sink=None) -> np.ndarray | None:
    """Per-expert stream e of tensor tid, shape [n_exp, *shape].

    With ``sink`` given, each expert slab is passed to ``sink(e, slab)`` as
    soon as it is drawn and nothing is kept (lets callers stream 20+ GB of
    weights straight to device memory).
    """
    n = int(np.prod(shape))
    ids = list(range(n_exp)) if experts is None else list(experts)

    def one(e):
        return e, _draw(wl.seed, tid, e, n, sigma, wl.dtype).reshape(shape)

    out = None
    if sink is None:
        out = np.empty((len(ids),) + tuple(shape),
                       dtype=np.uint16 if wl.dtype == BF16 else np.float32)
    with ThreadPoolExecutor(_nthreads()) as ex:
        for i, (e, slab) in enumerate(ex.map(one, ids)):
            if sink is not None:
                sink(e, slab)
            else:
                out[i] = slab
    return out


def router_bias(wl: Workload) -> np.ndarray | None:
    """Per-expert router bias b_e = c * ln p_{r(e)}, p = Zipf(s) rank weights
    over the E experts, rank r(e) = e + 1 (float32). None when unbiased."""
    if wl.zipf_bias == 0.0:
        return None
    r = np.arange(1, wl.E + 1, dtype=np.float64)
    p = r ** (-wl.zipf_s)
    p /= p.sum()
    return (wl.zipf_bias * np.log(p)).astype(np.float32)


@dataclasses.dataclass
class LayerInputs:
    A: np.ndarray          # [S][H]
    Wr: np.ndarray         # [H][E]
    bias: np.ndarray | None
    W_up: np.ndarray | None    # [E][H][D]
    W_gate: np.ndarray | None  # [E][H][D]
    W_down: np.ndarray | None  # [E][D][H]
    Ws_up: np.ndarray | None = None    # [H][Ds]
    Ws_gate: np.ndarray | None = None  # [H][Ds]
    Ws_down: np.ndarray | None = None  # [Ds][H]


def expert_sigmas(wl: Workload):
    """(up/gate std, down std, shared up/gate std, shared down std)."""
    su = 1.0 / math.sqrt(wl.H)
    sd = 1.0 / math.sqrt(wl.D)
    ssd = 1.0 / math.sqrt(wl.D_shared) if wl.D_shared else 0.0
    return su, sd, su, ssd


def draw_routing_inputs(wl: Workload):
    """A [S][H], W_router [H][E], bias [E] or None."""
    A = draw_tensor(wl, T_A, (wl.S, wl.H), 1.0)
    Wr = draw_tensor(wl, T_WR, (wl.H, wl.E), wl.router_std)
    return A, Wr, router_bias(wl)


def draw_layer(wl: Workload, experts: bool = True) -> LayerInputs:
    """Every input of the layer, held in host memory (small/medium layers)."""
    A, Wr, b = draw_routing_inputs(wl)
    li = LayerInputs(A=A, Wr=Wr, bias=b, W_up=None, W_gate=None, W_down=None)
    if experts:
        su, sd, ssu, ssd = expert_sigmas(wl)
        li.W_up = draw_experts(wl, T_WUP, wl.E, (wl.H, wl.D), su)
        li.W_gate = draw_experts(wl, T_WGATE, wl.E, (wl.H, wl.D), su)
        li.W_down = draw_experts(wl, T_WDOWN, wl.E, (wl.D, wl.H), sd)
        if wl.D_shared:
            li.Ws_up = draw_tensor(wl, T_WSUP, (wl.H, wl.D_shared), ssu)
            li.Ws_gate = draw_tensor(wl, T_WSGATE, (wl.H, wl.D_shared), ssu)
            li.Ws_down = draw_tensor(wl, T_WSDOWN, (wl.D_shared, wl.H), ssd)
    return li


# ---------------------------------------------------------------- routing ids
# Synthetic top-k id tensors for the align step alone (distributions of the
# vLLM align-kernel PR's tests and benchmark: random / alternating_empty /
# skewed / mostly_empty, plus all-to-one).

ID_DISTS = ("random", "alternating_empty", "skewed", "mostly_empty", "all_to_one")


def draw_topk_ids(S: int, k: int, E: int, dist: str, seed: int = 0) -> np.ndarray:
    """[S][k] int32, each row k distinct experts in [0, E)."""
    rng = np.random.default_rng([seed, 100, ID_DISTS.index(dist)])
    if k > E:
        raise ValueError("k > E")
    if dist == "all_to_one":
        base = np.zeros(S, dtype=np.int64)
        ids = (base[:, None] + np.arange(k)[None, :]) % E
        return ids.astype(np.int32)
    if dist == "random":
        w = np.ones(E)
    elif dist == "alternating_empty":
        w = np.where(np.arange(E) % 2 == 0, 1.0, 0.0)
        if (w > 0).sum() < k:
            w = np.ones(E)
    elif dist == "skewed":
        w = (np.arange(1, E + 1, dtype=np.float64)) ** -1.2
    elif dist == "mostly_empty":
        w = np.zeros(E)
        w[: max(k, min(E, 3))] = 1.0
    else:
        raise ValueError(dist)
    p = w / w.sum()
    # Gumbel top-k: k distinct experts per row drawn without replacement
    g = np.log(np.where(p > 0, p, 1e-300))[None, :] - np.log(-np.log(rng.random((S, E))))
    g[:, p == 0] = -np.inf
    ids = np.argsort(-g, axis=1, kind="stable")[:, :k]
    return ids.astype(np.int32)
