"""CPU oracle of the fused MoE layer forward pass (ctypes wrapper of moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it to check and time the HIP library. The library never
imports it, and it never imports the library.

Functions take numpy arrays (fp32 arrays, or uint16 bf16 bit patterns for
bf16 layers) and return numpy arrays. See moe_oracle.c for what each step
computes and which passage of the MoE pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_PLANT_DIR = os.path.join(_HERE, "_build")

# Deliberately wrong variants used only by the pin self-test.
PLANTS = ("TIE_HIGH", "WEIGHT_NO_EXP", "CAP_OFF_BY_ONE", "ALIGN_REVERSED",
          "SILU_ON_GATE", "DOWN_TRANSPOSED", "WEIGHT_SLOT0", "DROP_SHARED", "ROW_INDEX",
          "E4M3_TIES_AWAY", "E4M3_NO_SATURATE", "MX_EMAX7", "MX_WEIGHT_UNSCALED",
          "MX_NO_H_QUANT")

F32 = 0
BF16 = 1


def lib_path(plant: str | None = None) -> str:
    if plant is None:
        return _LIB
    return os.path.join(_PLANT_DIR, f"liboracle_{plant.lower()}.so")


def build(plant: str | None = None) -> str:
    """Compile moe_oracle.c with gcc (-O2, OpenMP, IEEE semantics kept)."""
    out = lib_path(plant)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-o", out + ".tmp", _SRC, "-lm"]
    if plant is not None:
        if plant not in PLANTS:
            raise ValueError(plant)
        cmd.insert(1, f"-DORACLE_PLANT_{plant}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class Oracle:
    """One loaded build of the oracle (the real one, or a planted variant)."""

    def __init__(self, plant: str | None = None):
        path = lib_path(plant)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(plant)
        self.plant = plant
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_gate_logits.argtypes = [_i64, _i64, _i64, ctypes.c_int, _p, _p, _p, _p]
        L.oracle_topk_softmax.argtypes = [_i64, _i64, _i64, ctypes.c_int, _p, _p, _p]
        L.oracle_capacity_mask.argtypes = [_i64, _i64, _i64, _i64, _p, _p]
        L.oracle_align.argtypes = [_i64, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.oracle_layer_rows.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                        _p, _p, _p, _p, _p, _p, _p,
                                        _p, _p, _p, _i64, _p, _p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_e4m3_values.argtypes = [_i64, _p, _p]
        L.oracle_e4m3_encode_array.argtypes = [_i64, _p, _p]
        L.oracle_mx_quantize_rows.argtypes = [_i64, _i64, ctypes.c_int, _p, _p, _p]
        L.oracle_mx_quantize_cols.argtypes = [_i64, _i64, ctypes.c_int, _p, _p, _p]
        L.oracle_layer_rows_mx.argtypes = [_i64] * 5 + [_p] * 14 + [_p, _p, _p, _i64, _p, _p]
        for f in (L.oracle_e4m3_values, L.oracle_e4m3_encode_array, L.oracle_mx_quantize_rows,
                  L.oracle_mx_quantize_cols, L.oracle_layer_rows_mx):
            f.restype = None
        for f in (L.oracle_gate_logits, L.oracle_topk_softmax, L.oracle_capacity_mask,
                  L.oracle_align, L.oracle_layer_rows):
            f.restype = None

    # ------------------------------------------------------------ helpers
    @staticmethod
    def _dtype_of(x: np.ndarray) -> int:
        if x.dtype == np.float32:
            return F32
        if x.dtype == np.uint16:
            return BF16
        raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {x.dtype}")

    @staticmethod
    def _ptr(x):
        if x is None:
            return None
        assert x.flags["C_CONTIGUOUS"]
        return x.ctypes.data_as(ctypes.c_void_p)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # ------------------------------------------------------------- steps
    def gate_logits(self, A, Wr, bias=None) -> np.ndarray:
        """G [S][E] fp32 = A [S][H] . Wr [H][E] (+ bias [E])."""
        S, H = A.shape
        H2, E = Wr.shape
        assert H == H2 and A.dtype == Wr.dtype
        A = np.ascontiguousarray(A)
        Wr = np.ascontiguousarray(Wr)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        G = np.empty((S, E), dtype=np.float32)
        self.lib.oracle_gate_logits(S, H, E, self._dtype_of(A), self._ptr(A), self._ptr(Wr),
                                    self._ptr(b), self._ptr(G))
        return G

    def topk_softmax(self, G, k: int, renormalize: int = 1):
        """(ids [S][k] int32, weights [S][k] fp32)."""
        G = np.ascontiguousarray(G, dtype=np.float32)
        S, E = G.shape
        ids = np.empty((S, k), dtype=np.int32)
        w = np.empty((S, k), dtype=np.float32)
        self.lib.oracle_topk_softmax(S, E, k, int(renormalize), self._ptr(G), self._ptr(ids),
                                     self._ptr(w))
        return ids, w

    def capacity_mask(self, ids, E: int, C: int) -> np.ndarray:
        """kept [S][k] uint8 (1 = assignment gets a slot below C)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        S, k = ids.shape
        kept = np.empty((S, k), dtype=np.uint8)
        self.lib.oracle_capacity_mask(S, k, E, C, self._ptr(ids), self._ptr(kept))
        return kept

    @staticmethod
    def align_capacity(S: int, k: int, E: int, BM: int) -> int:
        return S * k + E * (BM - 1)

    def align(self, ids, E: int, BM: int, C: int = 0):
        """(sorted_ids, expert_ids, ntpp, counts); buffers sized for the worst
        case, entries past ntpp (and past ntpp/BM blocks) are unspecified."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        S, k = ids.shape
        cap = self.align_capacity(S, k, E, BM)
        sorted_ids = np.full(cap, -1, dtype=np.int32)
        expert_ids = np.full(max(1, cap // BM), -1, dtype=np.int32)
        ntpp = np.zeros(1, dtype=np.int32)
        counts = np.zeros(E, dtype=np.int32)
        self.lib.oracle_align(S, k, E, BM, C, self._ptr(ids), self._ptr(sorted_ids),
                              self._ptr(expert_ids), self._ptr(ntpp), self._ptr(counts))
        return sorted_ids, expert_ids, int(ntpp[0]), counts

    def layer_rows(self, A, W_up, W_gate, W_down, ids, w, kept=None, tokens=None,
                   Ws_up=None, Ws_gate=None, Ws_down=None) -> np.ndarray:
        """O rows [n][H] (float64) for the listed tokens (default: all)."""
        S, H = A.shape
        E, H2, D = W_up.shape
        assert H2 == H and W_down.shape == (E, D, H)
        k = ids.shape[1]
        Ds = 0 if Ws_up is None else Ws_up.shape[1]
        if tokens is None:
            tokens = np.arange(S, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        if tokens.size and (tokens.min() < 0 or tokens.max() >= S):
            raise IndexError("token out of range")
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        if kept is not None:
            kept = np.ascontiguousarray(kept, dtype=np.uint8)
        O = np.empty((tokens.size, H), dtype=np.float64)
        P = self._ptr
        self.lib.oracle_layer_rows(H, D, E, k, Ds, self._dtype_of(A), P(A), P(W_up), P(W_gate),
                                   P(W_down), P(Ws_up), P(Ws_gate), P(Ws_down), P(ids), P(w),
                                   P(kept), tokens.size, P(tokens), P(O))
        return O

    # ------------------------------------------------------------- MXFP8
    def e4m3_values(self, codes) -> np.ndarray:
        """float64 values of E4M3 codes (uint8 array)."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e4m3_values(c.size, self._ptr(c), self._ptr(out))
        return out

    def e4m3_encode(self, x) -> np.ndarray:
        """Nearest E4M3 codes of float64 values (ties to even, saturating)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_e4m3_encode_array(x.size, self._ptr(x), self._ptr(out))
        return out

    def mx_quantize_rows(self, X):
        """MX blocks along the last axis of X [..][K]: (codes [..][K] uint8,
        scales [..][K/32] uint8)."""
        X = np.ascontiguousarray(X)
        K = X.shape[-1]
        assert K % 32 == 0
        R = X.size // K
        codes = np.empty(X.shape, dtype=np.uint8)
        scales = np.empty(X.shape[:-1] + (K // 32,), dtype=np.uint8)
        self.lib.oracle_mx_quantize_rows(R, K, self._dtype_of(X), self._ptr(X),
                                         self._ptr(codes), self._ptr(scales))
        return codes, scales

    def mx_quantize_cols(self, W):
        """MX blocks along axis -2 of W [..][K][N] (each column's K values in
        blocks of 32): (codes [..][K][N], scales [..][K/32][N])."""
        W = np.ascontiguousarray(W)
        K, N = W.shape[-2:]
        assert K % 32 == 0
        lead = W.shape[:-2]
        codes = np.empty(W.shape, dtype=np.uint8)
        scales = np.empty(lead + (K // 32, N), dtype=np.uint8)
        Wf = W.reshape((-1, K, N))
        cf = codes.reshape((-1, K, N))
        sf = scales.reshape((-1, K // 32, N))
        for i in range(Wf.shape[0]):
            wi = np.ascontiguousarray(Wf[i])
            ci = np.empty((K, N), dtype=np.uint8)
            si = np.empty((K // 32, N), dtype=np.uint8)
            self.lib.oracle_mx_quantize_cols(K, N, self._dtype_of(wi), self._ptr(wi),
                                             self._ptr(ci), self._ptr(si))
            cf[i] = ci
            sf[i] = si
        return codes, scales

    def layer_rows_mx(self, Aq, As, Wu, Wg, Wd, ids, w, kept=None, tokens=None,
                      Wsu=None, Wsg=None, Wsd=None) -> np.ndarray:
        """O rows [n][H] (float64) of the MXFP8 layer. Aq/As: the token rows'
        codes and scales; Wu, Wg, Wd, Wsu, Wsg, Wsd: (codes, scales) pairs in
        the layouts of mx_quantize_cols applied to W_up, W_gate [E][H][D],
        W_down [E][D][H] and the shared [H][Ds], [H][Ds], [Ds][H]."""
        S, H = Aq.shape
        E, _, D = Wu[0].shape
        k = ids.shape[1]
        Ds = 0 if Wsu is None else Wsu[0].shape[1]
        if tokens is None:
            tokens = np.arange(S, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        if kept is not None:
            kept = np.ascontiguousarray(kept, dtype=np.uint8)
        c = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.uint8)
        arrs = [c(Aq), c(As), c(Wu[0]), c(Wu[1]), c(Wg[0]), c(Wg[1]), c(Wd[0]), c(Wd[1])]
        sh = [None] * 6 if Wsu is None else [c(Wsu[0]), c(Wsu[1]), c(Wsg[0]), c(Wsg[1]),
                                             c(Wsd[0]), c(Wsd[1])]
        O = np.empty((tokens.size, H), dtype=np.float64)
        P = self._ptr
        self.lib.oracle_layer_rows_mx(H, D, E, k, Ds, *[P(a) for a in arrs + sh], P(ids), P(w),
                                      P(kept), tokens.size, P(tokens), P(O))
        return O

    # ---------------------------------------------------------- whole layer
    def layer(self, A, Wr, bias, W_up, W_gate, W_down, k, renormalize=1, capacity=0,
              Ws_up=None, Ws_gate=None, Ws_down=None, logits=None, tokens=None):
        """Full forward: logits -> top-k -> capacity -> expert FFNs -> combine.
        Returns a dict with G, ids, w, kept and O (rows of ``tokens``)."""
        G = self.gate_logits(A, Wr, bias) if logits is None else np.ascontiguousarray(logits)
        ids, w = self.topk_softmax(G, k, renormalize)
        kept = self.capacity_mask(ids, W_up.shape[0], capacity) if capacity else None
        O = self.layer_rows(A, W_up, W_gate, W_down, ids, w, kept, tokens, Ws_up, Ws_gate,
                            Ws_down)
        return {"G": G, "ids": ids, "w": w, "kept": kept, "O": O}


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
