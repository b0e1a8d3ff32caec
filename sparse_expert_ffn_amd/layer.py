"""Device buffers for one MoE layer shape, and the three C-ABI calls in order.

Allocation (torch, device memory) happens once in the constructor; ``run``
only enqueues moe_gate_topk, moe_align_block_size and moe_forward on the
stream, so repeated calls allocate nothing.
"""
from __future__ import annotations

import torch

from . import (MOE_BF16, MOE_F32, MOE_MXFP8, make_shape, moe_align_block_size, moe_align_workspace_bytes,
               moe_forward, moe_forward_workspace_bytes, moe_gate_topk, moe_gate_workspace_bytes)


class MoEBuffers:
    def __init__(self, S, H, D, E, k, D_shared=0, capacity=0, block_size=128, renormalize=1,
                 dtype=MOE_BF16, out_f32=False, atomic_combine=False, sched_quota=False,
                 fused_launch=False, device="cuda", extra_flags=0):
        self.shape = make_shape(S, H, D, E, k, D_shared, capacity, block_size, renormalize,
                                dtype, out_f32, atomic_combine, sched_quota, fused_launch,
                                extra_flags)
        self.tdtype = torch.bfloat16 if dtype != MOE_F32 and not out_f32 else torch.float32
        dev = torch.device(device)
        cap = S * k + E * (block_size - 1)
        i32, f32 = torch.int32, torch.float32
        self.logits = torch.empty((S, E), dtype=f32, device=dev)
        self.topk_ids = torch.empty((S, k), dtype=i32, device=dev)
        self.topk_weights = torch.empty((S, k), dtype=f32, device=dev)
        self.sorted_ids = torch.empty(max(cap, 1), dtype=i32, device=dev)
        self.expert_ids = torch.empty(max(cap // block_size, 1), dtype=i32, device=dev)
        self.ntpp = torch.empty(1, dtype=i32, device=dev)
        self.expert_counts = torch.empty(E, dtype=i32, device=dev)
        gate_ws = moe_gate_workspace_bytes(self.shape)
        self.gate_ws = torch.empty(gate_ws, dtype=torch.uint8, device=dev) if gate_ws else None
        self.align_ws = torch.empty(max(moe_align_workspace_bytes(self.shape), 1),
                                    dtype=torch.uint8, device=dev)
        self.forward_ws = torch.empty(max(moe_forward_workspace_bytes(self.shape), 1),
                                      dtype=torch.uint8, device=dev)
        self.O = torch.empty((S, H), dtype=self.tdtype, device=dev)

    def route(self, A=None, W_router=None, router_bias=None, logits_in=None, stream=None):
        moe_gate_topk(self.shape, A, W_router, router_bias, logits_in, self.logits,
                      self.topk_ids, self.topk_weights, self.gate_ws, stream)
        moe_align_block_size(self.shape, self.topk_ids, self.sorted_ids, self.expert_ids,
                             self.ntpp, self.expert_counts, self.align_ws, stream)

    def forward(self, A, W_up, W_gate, W_down, Ws_up=None, Ws_gate=None, Ws_down=None,
                stream=None):
        moe_forward(self.shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down,
                    self.topk_weights, self.sorted_ids, self.expert_ids, self.ntpp, self.O,
                    self.forward_ws, stream)
        return self.O

    def run(self, A, W_router, W_up, W_gate, W_down, Ws_up=None, Ws_gate=None, Ws_down=None,
            router_bias=None, logits_in=None, stream=None):
        """One pass of the whole layer: gate, top-k, align, experts, combine."""
        self.route(A, W_router, router_bias, logits_in, stream)
        return self.forward(A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, stream)


def suggest_block_size(S: int, k: int, E: int, capacity: int = 0, dtype: int = 1) -> int:
    """Rows per sorted block (vLLM's fused_moe note grows the block with the
    token count: 16 / 32 / 64, larger for prefill). The GEMM kernels skip
    16-row groups that hold only padding, so a block large enough for one
    expert's rows costs little more than their own work and streams that
    expert's weights once: pick the smallest block that holds the expected
    largest expert, taken as 1.25x the mean rows per expert, or the
    capacity when that is smaller (no expert keeps more). 256 for bf16 and
    MXFP8 only; MXFP8 takes 64 at least."""
    mean = S * k / max(E, 1)
    want = 1.25 * mean
    if capacity > 0:
        want = min(want, capacity)
    top = 256 if dtype != MOE_F32 else 128
    # the MXFP8 tiles come in 64, 128 and 256 rows
    for bm in ((64, 128, 256) if dtype == MOE_MXFP8 else (16, 32, 64, 128, 256)):
        if bm >= want or bm == top:
            return bm
    return top
