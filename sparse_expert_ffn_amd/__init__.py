"""Fused Mixture-of-Experts layer forward pass on one MI355X (gfx950).

Thin ctypes binding of the C ABI in include/moe.h, with the same names.
It only marshals arguments: every step of the layer runs in the HIP kernels
of libmoe.so. Array arguments are device tensors (torch, on the GPU) or raw
device addresses (int); ``stream`` is a torch stream, a raw hipStream_t
(int), or None for torch's current stream.

Loading fails loudly when libmoe.so has not been built (``build()``); there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["MOE_F32", "MOE_BF16", "MOE_MXFP8", "moe_mxfp8_weight_bytes", "moe_pack_mxfp8_weights",
           "moe_quantize_mxfp8", "MoeError", "moe_shape", "make_shape", "load_library",
           "moe_gate_workspace_bytes", "moe_gate_topk", "moe_align_workspace_bytes",
           "moe_align_block_size",
           "moe_forward_workspace_bytes", "moe_forward", "moe_status_string",
           "moe_profile_enable", "moe_profile_collect", "moe_device_query", "moe_trace_attach",
           "moe_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES", "forward_status",
           "build",
           "LIB_PATH", "STATUS", "MOE_FORWARD_STATUS_OFFSET", "MOE_STATUS_READY_TIMEOUT",
           "MOE_STATUS_TASKS_LOST", "MOE_STATUS_QUEUE_COUNT", "MOE_SCHED_BATCH",
           "MOE_TEST_SKIP_QUEUE_RESET", "MOE_COMBINE_FUSED", "MOE_SPLIT_TAIL"]

# SPARSE_EXPERT_FFN_LIB: load the library from another path (e.g. a build
# with different compile-time tile settings)
LIB_PATH = os.environ.get("SPARSE_EXPERT_FFN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1
MOE_MXFP8 = 2  # MXFP8 expert GEMMs (bf16 activations, packed MXFP8 expert weights)
MOE_OUTPUT_F32 = 1
MOE_COMBINE_ATOMIC = 2
MOE_SCHED_QUOTA = 4  # ablation baseline: static per-expert workgroup quota
MOE_FUSED_LAUNCH = 8  # up/gate and down GEMMs in one persistent launch (bf16)
MOE_SCHED_BATCH = 16  # batched claims: 4 tasks per queue atomic
MOE_TEST_SKIP_QUEUE_RESET = 32  # testing the status word: keep the previous call's queue counters
MOE_COMBINE_FUSED = 64  # the deterministic combine inside the down GEMM's epilogue
MOE_SPLIT_TAIL = 128  # long-tail splitting: the up/gate queues' last tasks as two row halves
# byte offset of the int32 status word in the moe_forward workspace, and its bits
MOE_FORWARD_STATUS_OFFSET = 128
MOE_STATUS_READY_TIMEOUT = 1
MOE_STATUS_TASKS_LOST = 2
MOE_STATUS_QUEUE_COUNT = 4
# device array behind moe_forward_noalloc, per GPU
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_HIP"}

# names of the entry points declared in include/moe.h
EXPORTS = ("moe_gate_workspace_bytes", "moe_gate_topk", "moe_align_workspace_bytes",
           "moe_align_block_size",
           "moe_forward_workspace_bytes", "moe_forward", "moe_status_string",
           "moe_profile_enable", "moe_profile_collect", "moe_device_query", "moe_trace_attach",
           "moe_forward_noalloc", "moe_mxfp8_weight_bytes", "moe_pack_mxfp8_weights",
           "moe_quantize_mxfp8")


class MoeError(RuntimeError):
    def __init__(self, call: str, code: int):
        self.code = code
        super().__init__(f"{call} failed: {STATUS.get(code, code)}")


class moe_shape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64), ("D_shared", ctypes.c_int64),
                ("capacity", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]

    def __repr__(self):
        return ("moe_shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_)
                + ")")


def make_shape(S, H, D, E, k, D_shared=0, capacity=0, block_size=128, renormalize=1,
               dtype=MOE_BF16, out_f32=False, atomic_combine=False,
               sched_quota=False, fused_launch=False, extra_flags=0) -> moe_shape:
    flags = ((MOE_OUTPUT_F32 if out_f32 else 0) | (MOE_COMBINE_ATOMIC if atomic_combine else 0)
             | (MOE_SCHED_QUOTA if sched_quota else 0)
             | (MOE_FUSED_LAUNCH if fused_launch else 0) | extra_flags)
    return moe_shape(S, H, D, E, k, D_shared, capacity, block_size, renormalize, dtype, flags)


_LIB = None


def build(verbose: bool = False) -> list:
    """Compile libmoe.so and its timing-record variant libmoe_trace.so for
    gfx950 in-tree (hipcc)."""
    from . import buildlib as _b
    global _LIB
    _LIB = None
    return _b.build_all(verbose=verbose)


def load_library(path: str | None = None) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: the HIP library must be built first "
                          "(sparse_expert_ffn_amd.build())")
    lib = ctypes.CDLL(p)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    sp = ctypes.POINTER(moe_shape)
    lib.moe_gate_workspace_bytes.argtypes = [sp]
    lib.moe_gate_workspace_bytes.restype = sz
    lib.moe_gate_topk.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_align_workspace_bytes.argtypes = [sp]
    lib.moe_align_workspace_bytes.restype = sz
    lib.moe_align_block_size.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_forward_workspace_bytes.argtypes = [sp]
    lib.moe_forward_workspace_bytes.restype = sz
    lib.moe_forward.argtypes = [sp] + [vp] * 13 + [sz, vp]
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_profile_enable.argtypes = [ctypes.c_int]
    lib.moe_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]
    lib.moe_device_query.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                     ctypes.c_char_p, sz]
    lib.moe_trace_attach.argtypes = [vp, sz]
    lib.moe_forward_noalloc.argtypes = [sp] + [vp] * 13
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_mxfp8_weight_bytes.argtypes = [i64, i64, i64]
    lib.moe_mxfp8_weight_bytes.restype = sz
    lib.moe_pack_mxfp8_weights.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.moe_pack_mxfp8_weights.restype = ctypes.c_int
    lib.moe_quantize_mxfp8.argtypes = [vp, i64, i64, ctypes.c_int32, vp, vp, vp]
    lib.moe_quantize_mxfp8.restype = ctypes.c_int
    for name in ("moe_gate_topk", "moe_align_block_size", "moe_forward", "moe_profile_enable",
                 "moe_profile_collect", "moe_device_query", "moe_trace_attach"):
        getattr(lib, name).restype = ctypes.c_int
    del i64
    if path is None:
        _LIB = lib
    return lib


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        if getattr(x, "device", None) is not None and x.device.type != "cuda":
            raise ValueError(f"tensor on {x.device}: the library takes device memory")
        return x.data_ptr() if x.numel() else None
    raise TypeError(f"cannot pass {type(x)} as a device pointer")


def _nbytes(x):
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass the workspace as a tensor, or (address, nbytes)")
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(workspace):
    if isinstance(workspace, tuple):
        return workspace[0], workspace[1]
    return _addr(workspace), _nbytes(workspace)


def _check(call, code):
    if code != 0:
        raise MoeError(call, code)


def moe_status_string(code: int) -> str:
    return load_library().moe_status_string(code).decode()


def moe_gate_workspace_bytes(shape) -> int:
    return int(load_library().moe_gate_workspace_bytes(ctypes.byref(shape)))


def moe_gate_topk(shape, A, W_router, router_bias, logits_in, logits_out, topk_ids,
                  topk_weights, workspace=None, stream=None, check=True) -> int:
    wa, wn = _ws(workspace)
    code = load_library().moe_gate_topk(
        ctypes.byref(shape), _addr(A), _addr(W_router), _addr(router_bias), _addr(logits_in),
        _addr(logits_out), _addr(topk_ids), _addr(topk_weights), wa, wn, _stream(stream))
    if check:
        _check("moe_gate_topk", code)
    return code


def moe_align_workspace_bytes(shape) -> int:
    return int(load_library().moe_align_workspace_bytes(ctypes.byref(shape)))


def moe_align_block_size(shape, topk_ids, sorted_ids, expert_ids, num_tokens_post_padded,
                         expert_counts, workspace, stream=None, check=True) -> int:
    wa, wn = _ws(workspace)
    code = load_library().moe_align_block_size(
        ctypes.byref(shape), _addr(topk_ids), _addr(sorted_ids), _addr(expert_ids),
        _addr(num_tokens_post_padded), _addr(expert_counts), wa, wn, _stream(stream))
    if check:
        _check("moe_align_block_size", code)
    return code


def moe_forward_workspace_bytes(shape) -> int:
    return int(load_library().moe_forward_workspace_bytes(ctypes.byref(shape)))


def moe_forward(shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, topk_weights,
                sorted_ids, expert_ids, num_tokens_post_padded, O, workspace, stream=None,
                check=True) -> int:
    wa, wn = _ws(workspace)
    code = load_library().moe_forward(
        ctypes.byref(shape), _addr(A), _addr(W_up), _addr(W_gate), _addr(W_down), _addr(Ws_up),
        _addr(Ws_gate), _addr(Ws_down), _addr(topk_weights), _addr(sorted_ids),
        _addr(expert_ids), _addr(num_tokens_post_padded), _addr(O), wa, wn, _stream(stream))
    if check:
        _check("moe_forward", code)
    return code


def moe_forward_noalloc(shape, A, W_up, W_gate, W_down, Ws_up, Ws_gate, Ws_down, topk_weights,
                        sorted_ids, expert_ids, num_tokens_post_padded, O, stream=None,
                        check=True) -> int:
    """moe_forward with the library's own device array as the workspace (at
    most MOE_NOALLOC_SCRATCH_BYTES): the call allocates nothing."""
    code = load_library().moe_forward_noalloc(
        ctypes.byref(shape), _addr(A), _addr(W_up), _addr(W_gate), _addr(W_down), _addr(Ws_up),
        _addr(Ws_gate), _addr(Ws_down), _addr(topk_weights), _addr(sorted_ids),
        _addr(expert_ids), _addr(num_tokens_post_padded), _addr(O), _stream(stream))
    if check:
        _check("moe_forward_noalloc", code)
    return code


def moe_mxfp8_weight_bytes(E: int, K: int, N: int) -> int:
    """Bytes of a weight tensor [E][K][N] packed for the MXFP8 GEMMs."""
    return int(load_library().moe_mxfp8_weight_bytes(E, K, N))


def moe_pack_mxfp8_weights(W, packed, stream=None, check=True) -> int:
    """Quantise a bf16 weight tensor W [E][K][N] (device) along K to MXFP8
    into ``packed`` (moe_mxfp8_weight_bytes(E, K, N) device bytes)."""
    E, K, N = (1,) + tuple(W.shape) if W.dim() == 2 else tuple(W.shape)
    code = load_library().moe_pack_mxfp8_weights(_addr(W), E, K, N, _addr(packed),
                                                 _stream(stream))
    if check:
        _check("moe_pack_mxfp8_weights", code)
    return code


def moe_quantize_mxfp8(X, codes, scales, stream=None, check=True) -> int:
    """MXFP8 codes [R][K] and scales [R][K/32] of the rows of X [R][K]
    (bf16 or fp32 device tensor)."""
    import torch
    R, K = X.shape
    dt = MOE_BF16 if X.dtype == torch.bfloat16 else MOE_F32
    code = load_library().moe_quantize_mxfp8(_addr(X), R, K, dt, _addr(codes), _addr(scales),
                                             _stream(stream))
    if check:
        _check("moe_quantize_mxfp8", code)
    return code


def moe_profile_enable(enable: bool, stages=(0, 1, 2, 3, 4)) -> None:
    """Time the given moe_forward stages (0 setup, 1 up/gate, 2 down, 3
    combine, 4 MXFP8 token-row quantisation) with HIP events on the call's
    stream, or stop timing."""
    mask = sum(1 << s for s in set(stages)) if enable else 0
    _check("moe_profile_enable", load_library().moe_profile_enable(mask))


def moe_profile_collect(n_stages: int = 5):
    """(per-stage milliseconds summed over recorded calls, number of calls)."""
    buf = (ctypes.c_float * n_stages)()
    n = ctypes.c_int(0)
    _check("moe_profile_collect", load_library().moe_profile_collect(buf, n_stages,
                                                                     ctypes.byref(n)))
    return [float(x) for x in buf], int(n.value)


def forward_status(workspace) -> int:
    """The status word moe_forward left in ``workspace`` (a device uint8
    tensor; read after the stream has finished the call): 0, or
    MOE_STATUS_* bits."""
    w = workspace[MOE_FORWARD_STATUS_OFFSET:MOE_FORWARD_STATUS_OFFSET + 4]
    return int(w.cpu().view(dtype=__import__("torch").int32).item())


def moe_device_query():
    """(compute units, peak engine clock in MHz, device name) of the current
    HIP device, as the runtime reports them."""
    cus = ctypes.c_int(0)
    khz = ctypes.c_int(0)
    name = ctypes.create_string_buffer(256)
    _check("moe_device_query", load_library().moe_device_query(
        ctypes.byref(cus), ctypes.byref(khz), name, 256))
    return int(cus.value), khz.value / 1000.0, name.value.decode(errors="replace")


def moe_trace_attach(buffer, check=True) -> int:
    """Record per-task timing into ``buffer`` (a 64-byte aligned device uint8
    tensor; None stops). MOE_ERR_UNSUPPORTED unless the loaded library was
    built with MOE_TRACE (``buildlib.build_trace()``)."""
    a, n = (None, 0) if buffer is None else _ws(buffer)
    code = load_library().moe_trace_attach(a, n)
    if check:
        _check("moe_trace_attach", code)
    return code
