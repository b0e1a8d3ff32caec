"""The C-ABI library: it loads, exports every entry point include/moe.h
declares, and rejects bad arguments on the host (no GPU needed: each call
here returns from argument validation before anything is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_expert_ffn_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 0x100000  # 16-byte aligned address, never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        moe.build()
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    for n in names:
        assert n in exported, f"{n} not exported"
        assert hasattr(lib, n)


def test_shape_struct_layout():
    # int64 x 7, int32 x 4 -> 72 bytes, no padding surprises
    assert ctypes.sizeof(moe.moe_shape) == 72


def test_status_strings(lib):
    for code, name in moe.STATUS.items():
        assert moe.moe_status_string(code) == name
    assert moe.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def shape(**kw):
    base = dict(S=64, H=128, D=256, E=8, k=2, D_shared=0, capacity=0, block_size=16,
                renormalize=1, dtype=moe.MOE_BF16)
    base.update(kw)
    return moe.make_shape(**base)


def gate(lib, s, **kw):
    args = dict(A=FAKE, Wr=FAKE, bias=None, lin=None, lout=FAKE, ids=FAKE, w=FAKE, ws=None,
                wsn=0)
    args.update(kw)
    return lib.moe_gate_topk(ctypes.byref(s) if s is not None else None, args["A"], args["Wr"],
                             args["bias"], args["lin"], args["lout"], args["ids"], args["w"],
                             args["ws"], args["wsn"], None)


def test_gate_topk_validation(lib):
    assert gate(lib, None) == 1
    assert gate(lib, shape(k=9)) == 1                   # k > E
    assert gate(lib, shape(k=0)) == 1
    assert gate(lib, shape(E=2000, k=2)) == 2           # E > 1024
    assert gate(lib, shape(E=64, k=33)) == 2            # k > 32
    assert gate(lib, shape(dtype=7)) == 1
    assert gate(lib, shape(renormalize=2)) == 1
    assert gate(lib, shape(), ids=None) == 1
    assert gate(lib, shape(), lout=None) == 1           # scores need a buffer
    assert gate(lib, shape(H=100)) == 2                 # H not a multiple of 8
    assert gate(lib, shape(), A=FAKE + 4) == 2          # misaligned
    assert gate(lib, shape(S=0), ids=None, w=None) == 0  # empty call
    # few tokens and a long H: the GEMM is split along H and needs a workspace
    dec = shape(S=64, H=2048, E=256, k=8)
    need = moe.moe_gate_workspace_bytes(dec)
    assert need > 0
    assert gate(lib, dec) == 3                          # no workspace
    assert gate(lib, dec, ws=FAKE, wsn=need - 1) == 3   # too small
    assert gate(lib, dec, ws=FAKE + 4, wsn=need) == 2   # misaligned
    s = shape()
    s.flags = 256                                       # undefined flag bit
    assert gate(lib, s) == 1


def align(lib, s, ws_bytes=1 << 20, **kw):
    args = dict(ids=FAKE, si=FAKE, ei=FAKE, n=FAKE, c=FAKE, ws=FAKE)
    args.update(kw)
    return lib.moe_align_block_size(ctypes.byref(s), args["ids"], args["si"], args["ei"],
                                    args["n"], args["c"], args["ws"], ws_bytes, None)


def test_align_validation(lib):
    assert align(lib, shape(block_size=0)) == 1
    assert align(lib, shape(capacity=-1)) == 1
    assert align(lib, shape(), si=None) == 1
    assert align(lib, shape(), ws=None) == 1
    assert align(lib, shape(), ws_bytes=8) == 3
    big = shape(S=2**30, k=8, E=256)
    assert align(lib, big) == 2                         # indices would overflow int32


def test_workspace_sizes(lib):
    # gate: split only for few row tiles or a long H (bf16, E <= 256); the
    # partial scores of every split, fp32
    assert moe.moe_gate_workspace_bytes(shape(S=16384, H=2048, E=64)) == 0
    assert moe.moe_gate_workspace_bytes(shape(S=64, H=2048, E=256, dtype=moe.MOE_F32)) == 0
    assert moe.moe_gate_workspace_bytes(shape(S=64, H=2048, E=1024, k=8)) == 0
    d = moe.moe_gate_workspace_bytes(shape(S=64, H=2048, E=256, k=8))
    assert d >= 2 * 64 * 256 * 4 and d % (64 * 256 * 4) == 0
    v3 = moe.moe_gate_workspace_bytes(shape(S=4096, H=7168, E=256, k=8))
    assert v3 >= 2 * 4096 * 256 * 4 and v3 % (4096 * 256 * 4) == 0
    assert moe.moe_gate_workspace_bytes(shape(k=9)) == 0
    for bm in (1, 16, 48, 128):
        s = shape(block_size=bm)
        assert moe.moe_align_workspace_bytes(s) > 0
    assert moe.moe_align_workspace_bytes(shape(k=9)) == 0
    s = shape(block_size=128, S=16384, H=2048, D=2048, E=64, k=2)
    f = moe.moe_forward_workspace_bytes(s)
    # O_acc (fp32) + h rows (bf16), at least
    assert f >= 16384 * 2048 * 4 + (16384 * 2 + 64 * 127) * 2048 * 2
    assert moe.moe_forward_workspace_bytes(shape(block_size=48)) == 0  # forward BM set
    sh = moe.moe_forward_workspace_bytes(shape(D_shared=64))
    assert sh > moe.moe_forward_workspace_bytes(shape())


def fwd(lib, s, ws_bytes=1 << 30, **kw):
    a = dict(A=FAKE, Wu=FAKE, Wg=FAKE, Wd=FAKE, Su=None, Sg=None, Sd=None, w=FAKE, si=FAKE,
             ei=FAKE, n=FAKE, O=FAKE, ws=FAKE)
    a.update(kw)
    return lib.moe_forward(ctypes.byref(s), a["A"], a["Wu"], a["Wg"], a["Wd"], a["Su"], a["Sg"],
                           a["Sd"], a["w"], a["si"], a["ei"], a["n"], a["O"], a["ws"], ws_bytes,
                           None)


def test_forward_validation(lib):
    assert fwd(lib, shape(block_size=48)) == 2
    assert fwd(lib, shape(D=100)) == 2
    assert fwd(lib, shape(H=0)) == 1
    assert fwd(lib, shape(D_shared=64)) == 1            # shared weights missing
    assert fwd(lib, shape(), Su=FAKE, Sg=FAKE, Sd=FAKE) == 1  # shared weights without D_shared
    assert fwd(lib, shape(), O=None) == 1
    assert fwd(lib, shape(), A=FAKE + 2) == 2
    assert fwd(lib, shape(), ws_bytes=100) == 3
    assert fwd(lib, shape(S=0), A=None, O=None) == 0    # empty call, nothing enqueued
    # one-launch form: bf16 only, not with the quota scheduler
    assert fwd(lib, shape(dtype=moe.MOE_F32, fused_launch=True)) == 2
    assert fwd(lib, shape(fused_launch=True, sched_quota=True)) == 2
    s = shape()
    s.flags = 256                                       # undefined flag bit
    assert fwd(lib, s) == 1
    # the fused combine: not with the atomic combine, one launch, or MXFP8
    assert fwd(lib, shape(atomic_combine=True, extra_flags=moe.MOE_COMBINE_FUSED)) == 2
    assert fwd(lib, shape(fused_launch=True, extra_flags=moe.MOE_COMBINE_FUSED)) == 2
    assert fwd(lib, shape(dtype=moe.MOE_MXFP8, H=256, D=256, block_size=64,
                          extra_flags=moe.MOE_COMBINE_FUSED)) == 2
    # its arrival counters take workspace
    assert (moe.moe_forward_workspace_bytes(shape(extra_flags=moe.MOE_COMBINE_FUSED))
            > moe.moe_forward_workspace_bytes(shape()))
    # batched claims and the queue-reset test hook: the two-launch queues only
    for f in (moe.MOE_SCHED_BATCH, moe.MOE_TEST_SKIP_QUEUE_RESET):
        assert fwd(lib, shape(fused_launch=True, extra_flags=f)) == 2
        assert fwd(lib, shape(sched_quota=True, extra_flags=f)) == 2
    # long-tail splitting: a kernel choice, with or without the other options
    assert (moe.moe_forward_workspace_bytes(shape(extra_flags=moe.MOE_SPLIT_TAIL))
            == moe.moe_forward_workspace_bytes(shape()) > 0)
    assert moe.moe_forward_workspace_bytes(shape(sched_quota=True,
                                                 extra_flags=moe.MOE_SPLIT_TAIL)) > 0
    assert moe.moe_forward_workspace_bytes(shape(dtype=moe.MOE_F32, fused_launch=True)) == 0
    # readiness counters: one per routed and per shared m-block, more workspace
    assert (moe.moe_forward_workspace_bytes(shape(D_shared=64, fused_launch=True))
            >= moe.moe_forward_workspace_bytes(shape(D_shared=64)))


def _header_macros():
    text = open(HEADER).read()
    return {m: int(v) for m, v in re.findall(r"#define\s+(MOE_\w+)\s+(\d+)", text)}


def test_forward_status_word_layout(lib):
    """The status word's offset and bits in include/moe.h match the binding and
    the library's counter block (cleared by every call), and every valid
    shape's workspace covers it."""
    macros = _header_macros()
    off = macros["MOE_FORWARD_STATUS_OFFSET"]
    assert off == moe.MOE_FORWARD_STATUS_OFFSET and off % 4 == 0
    assert macros["MOE_STATUS_READY_TIMEOUT"] == moe.MOE_STATUS_READY_TIMEOUT
    common = open(os.path.join(ROOT, "sparse_expert_ffn_amd", "csrc", "moe_common.h")).read()
    word = int(re.search(r"kStatusWord\s*=\s*(\d+)", common).group(1))
    timeout = int(re.search(r"kStatusReadyTimeout\s*=\s*(\d+)", common).group(1))
    queues = int(re.search(r"kQuotaBase\s*=\s*(\d+)", common).group(1))
    assert word * 4 == off and timeout == moe.MOE_STATUS_READY_TIMEOUT
    assert 16 <= word < queues, "inside the counter block, clear of the task queues"
    lost = int(re.search(r"kStatusTasksLost\s*=\s*(\d+)", common).group(1))
    count = int(re.search(r"kStatusQueueCount\s*=\s*(\d+)", common).group(1))
    assert macros["MOE_STATUS_TASKS_LOST"] == moe.MOE_STATUS_TASKS_LOST == lost
    assert macros["MOE_STATUS_QUEUE_COUNT"] == moe.MOE_STATUS_QUEUE_COUNT == count
    bits = [timeout, lost, count]
    assert all(b & (b - 1) == 0 for b in bits) and len(set(bits)) == 3, "distinct single bits"
    # the per-GEMM done / exit counters: after both GEMMs' queues, before the status word
    done = int(re.search(r"kDoneBase\s*=\s*(\d+)", common).group(1))
    assert 16 <= done and done + 4 <= word
    for f in ("MOE_SCHED_BATCH", "MOE_TEST_SKIP_QUEUE_RESET", "MOE_COMBINE_FUSED"):
        assert macros[f] == getattr(moe, f)
    for kw in (dict(), dict(S=1, E=1, k=1), dict(dtype=moe.MOE_F32, block_size=128),
               dict(fused_launch=True), dict(atomic_combine=True)):
        assert moe.moe_forward_workspace_bytes(shape(**kw)) >= off + 4, kw


def test_noalloc_validation(lib):
    """The allocation-free forward rejects shapes whose workspace exceeds its
    device array, and bad arguments, before touching the device."""
    macros = _header_macros()
    assert "MOE_NOALLOC_SCRATCH_BYTES" in open(HEADER).read()
    assert moe.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20
    big = shape(S=16384, H=2048, D=2048, E=64, k=2, capacity=512, block_size=256)
    assert moe.moe_forward_workspace_bytes(big) > moe.MOE_NOALLOC_SCRATCH_BYTES
    f = lambda s: lib.moe_forward_noalloc(ctypes.byref(s) if s is not None else None,
                                          *([FAKE] * 4), None, None, None, *([FAKE] * 5), None)
    assert f(big) == 3                       # MOE_ERR_WORKSPACE_TOO_SMALL
    assert f(None) == 1
    assert f(shape(k=9)) == 1
    assert f(shape(block_size=48)) == 2
    assert macros  # header parsed


def test_mxfp8_validation(lib):
    """MXFP8 entry points reject bad arguments before touching the device."""
    assert moe.moe_mxfp8_weight_bytes(64, 2048, 2048) == 64 * 16 * 32 * 8448
    assert moe.moe_mxfp8_weight_bytes(1, 96, 128) == 0       # K not a multiple of 64
    assert moe.moe_mxfp8_weight_bytes(1, 128, 96) == 0       # N not a multiple of 128
    pack = lambda W, E, K, N, out: lib.moe_pack_mxfp8_weights(W, E, K, N, out, None)
    assert pack(None, 1, 128, 128, FAKE) == 1
    assert pack(FAKE, 0, 128, 128, FAKE) == 1
    assert pack(FAKE, 1, 96, 128, FAKE) == 2
    assert pack(FAKE, 1, 128, 128, FAKE + 8) == 2             # misaligned
    q = lambda X, R, K, dt, c, s: lib.moe_quantize_mxfp8(X, R, K, dt, c, s, None)
    assert q(FAKE, 4, 64, 7, FAKE, FAKE) == 1                 # dtype
    assert q(FAKE, 4, 48, moe.MOE_BF16, FAKE, FAKE) == 2      # K % 32
    assert q(None, 4, 64, moe.MOE_BF16, FAKE, FAKE) == 1
    assert q(None, 0, 64, moe.MOE_BF16, None, None) == 0      # empty
    # the MXFP8 forward's shape rules
    ok = shape(S=64, H=256, D=384, E=8, k=2, block_size=64, dtype=moe.MOE_MXFP8)
    assert moe.moe_forward_workspace_bytes(ok) > 0
    for bad in (dict(H=200), dict(D=200), dict(block_size=32), dict(block_size=16)):
        s = shape(**dict(dict(S=64, H=256, D=384, E=8, k=2, block_size=64,
                              dtype=moe.MOE_MXFP8), **bad))
        assert moe.moe_forward_workspace_bytes(s) == 0, bad
    for flag in ("atomic_combine", "sched_quota", "fused_launch"):
        s = moe.make_shape(64, 256, 384, 8, 2, block_size=64, dtype=moe.MOE_MXFP8,
                           **{flag: True})
        assert moe.moe_forward_workspace_bytes(s) == 0, flag
