"""Helpers shared by the GPU tests: host -> device copies of the seeded
inputs, the error metrics of the parity bar, and per-workload settings."""
from __future__ import annotations

import numpy as np
import torch

import sparse_expert_ffn_amd as moe
from sparse_expert_ffn_amd import workloads as wk
from sparse_expert_ffn_amd.layer import MoEBuffers, suggest_block_size

DEV = "cuda:0"

# Parity bar: fp32 max |g - o| / max(|o|, RMS(o)) <= 1e-4 over every element,
#               and the plain max |g - o| / |o| <= 1e-4 over the elements with
#               |o| >= RMS(o) / 10 (below that the plain ratio measures the
#               cancellation in o, not the kernels: an element 1e6 times
#               smaller than its neighbours has no meaningful relative error);
#             bf16 max |g - o| / RMS(o) <= 2e-2 (fp32 accumulation).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
PLAIN_FLOOR = 0.1


def dev(a, device=DEV):
    """numpy (fp32 / bf16 bit patterns as uint16 / int32) -> device tensor."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t):
    if t.dtype == torch.bfloat16:
        return wk.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def rms(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def err_f32(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    r = max(rms(o), 1e-30)
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), r)))


def err_f32_plain(g, o, floor=PLAIN_FLOOR):
    """max |g - o| / |o| over the elements with |o| >= floor * RMS(o)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    sel = np.abs(o) >= floor * rms(o)
    if not np.any(sel):
        return 0.0
    return float(np.max(np.abs(g[sel] - o[sel]) / np.abs(o[sel])))


def err_bf16(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    return float(np.max(np.abs(g - o)) / max(rms(o), 1e-30))


def parity(wl, g, o):
    """(error, tolerance) of the parity bar for this workload's dtype. In bf16
    mode ``g`` is the fp32-accumulated output (written as fp32)."""
    if wl.dtype == wk.F32:
        return max(err_f32(g, o), err_f32_plain(g, o)), TOL_F32
    return err_bf16(g, o), TOL_BF16


def bf16_output_excess(g16, o):
    """A bf16 output is the fp32 result rounded once more: each element may
    sit up to half a bf16 ulp (<= 2^-8 |o|) beyond the bar. Returns the worst
    ratio |g - o| / (TOL_BF16 RMS(o) + 2^-8 |o|); <= 1 passes."""
    g16 = np.asarray(g16, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if o.size == 0:
        return 0.0
    bound = TOL_BF16 * max(rms(o), 1e-30) + 2.0 ** -8 * np.abs(o)
    return float(np.max(np.abs(g16 - o) / bound))


def lib_dtype(wl):
    """The C-ABI dtype of a workload: MOE_MXFP8 for its MXFP8 form."""
    return moe.MOE_MXFP8 if wl.mxfp8 else wl.dtype


def block_size_for(wl):
    return suggest_block_size(wl.S, wl.k, wl.E, wl.capacity, lib_dtype(wl))


def buffers(wl, block_size=None, out_f32=False, atomic_combine=False, sched_quota=False,
            fused_launch=False, extra_flags=0):
    bm = block_size or block_size_for(wl)
    return MoEBuffers(wl.S, wl.H, wl.D, wl.E, wl.k, wl.D_shared, wl.capacity, bm,
                      wl.renormalize, lib_dtype(wl), out_f32=out_f32,
                      atomic_combine=atomic_combine, sched_quota=sched_quota,
                      fused_launch=fused_launch, device=DEV, extra_flags=extra_flags)


def pack_mxfp8(W):
    """A bf16 device weight tensor [E][K][N] (or [K][N]) packed for the
    MXFP8 GEMMs by the library."""
    if W is None:
        return None
    E, K, N = (1,) + tuple(W.shape) if W.dim() == 2 else tuple(W.shape)
    packed = torch.empty(moe.moe_mxfp8_weight_bytes(E, K, N), dtype=torch.uint8,
                         device=W.device)
    moe.moe_pack_mxfp8_weights(W, packed)
    return packed


class DeviceLayer:
    """Every input of a layer on the device (weights streamed per expert).
    For an MXFP8 workload the expert weights are packed on the device."""

    def __init__(self, wl, li=None):
        self.wl = wl
        if li is None:
            li = wk.draw_layer(wl)
        self.li = li
        self.A = dev(li.A)
        self.Wr = dev(li.Wr)
        self.bias = dev(li.bias)
        ws = [dev(x) for x in (li.W_up, li.W_gate, li.W_down, li.Ws_up, li.Ws_gate, li.Ws_down)]
        if wl.mxfp8:
            ws = [pack_mxfp8(w) for w in ws]
        (self.W_up, self.W_gate, self.W_down, self.Ws_up, self.Ws_gate,
         self.Ws_down) = ws

    def forward(self, buf):
        return buf.forward(self.A, self.W_up, self.W_gate, self.W_down, self.Ws_up,
                           self.Ws_gate, self.Ws_down)
