"""ctypes wrapper of the fp64 CPU oracle (``liboracle.so``).

TEST INFRASTRUCTURE ONLY. This module and the C library under ``oracle/`` are
the independent reference that the GPU path is checked against. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
product package never does, and this module imports nothing from it.

Each method works on numpy arrays for one (batch, head) unit, mirroring the C
functions in ``eta_oracle.c`` (which cite the passages of the pages they
follow). bfloat16 data is passed as its raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "eta_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

KV_F32 = 0
KV_BF16 = 1
BOUND_COMBINED = 0
BOUND_GEO = 1

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


def compile_oracle(src: str = SRC, out: str = LIB_PATH, extra=()) -> str:
    """Compile an oracle C source into a shared library with gcc (plain -O2; `extra`
    flags are appended, e.g. sanitizers)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
           "-I", HERE, *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _kv(a: np.ndarray):
    """Return (contiguous array, kv_dtype code) for a key/value slab."""
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), KV_BF16
    return _c(a, np.float32), KV_F32


class OracleLib:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str = LIB_PATH):
        L = ctypes.CDLL(path)
        L.eta_oracle_bf16_to_f64.restype = ctypes.c_double
        L.eta_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.eta_oracle_predict_tau.restype = None
        L.eta_oracle_predict_tau.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             _fp, _fp, _fp, _dp]
        L.eta_oracle_block_meta.restype = ctypes.c_int
        L.eta_oracle_block_meta.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, _vp, _dp, _dp, _dp]
        L.eta_oracle_bounds.restype = None
        L.eta_oracle_bounds.argtypes = [ctypes.c_int, ctypes.c_int, _fp, _dp, _dp, _dp,
                                        ctypes.c_double, ctypes.c_int, _dp]
        L.eta_oracle_block_maxdev.restype = ctypes.c_int
        L.eta_oracle_block_maxdev.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _vp, _dp]
        L.eta_oracle_bounds_centered.restype = None
        L.eta_oracle_bounds_centered.argtypes = [ctypes.c_int, ctypes.c_int, _fp, _dp, _dp, _dp,
                                                 _dp]
        L.eta_oracle_screen.restype = ctypes.c_int
        L.eta_oracle_screen.argtypes = [ctypes.c_int, _dp, ctypes.c_double, _ip]
        L.eta_oracle_union.restype = ctypes.c_int
        L.eta_oracle_union.argtypes = [ctypes.c_int, _ip, _ip, ctypes.c_int, ctypes.c_int, _ip]
        L.eta_oracle_gate.restype = ctypes.c_double
        L.eta_oracle_gate.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_int]
        L.eta_oracle_attend.restype = None
        L.eta_oracle_attend.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _fp, _vp, _vp, ctypes.c_double, _ip, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_int, _dp, _dp]
        L.eta_oracle_prefill.restype = ctypes.c_int
        L.eta_oracle_prefill.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _fp, _vp, _vp, _dp, ctypes.c_double, ctypes.c_int,
                                         _dp, _dp, _dp]
        self.L = L
        self.path = path

    def bf16_to_f64(self, bits: int) -> float:
        return self.L.eta_oracle_bf16_to_f64(int(bits))

    def predict_tau(self, q, W, bias) -> np.ndarray:
        """q float32 [B,H,d]; W float32 [H*d,H] or None; bias [H] -> tau fp64 [B,H]."""
        q = _c(q, np.float32)
        B, H, d = q.shape
        bias = _c(bias, np.float32)
        tau = np.empty((B, H), dtype=np.float64)
        Wp = None
        if W is not None:
            W = _c(W, np.float32)
            assert W.shape == (H * d, H)
            Wp = W.ctypes.data_as(_fp)
        self.L.eta_oracle_predict_tau(B, H, d, q.ctypes.data_as(_fp), Wp,
                                      bias.ctypes.data_as(_fp), tau.ctypes.data_as(_dp))
        return tau

    def block_meta(self, K, T: int, bs: int = 64):
        """K [T_cap,d] (float32, or uint16 bf16 bits) -> (centroid [nblk,d], var, maxnorm)."""
        K, kvd = _kv(K)
        d = K.shape[1]
        assert 0 <= T <= K.shape[0]
        nblk = (T + bs - 1) // bs
        c = np.empty((max(nblk, 1), d), dtype=np.float64)
        v = np.empty(max(nblk, 1), dtype=np.float64)
        m = np.empty(max(nblk, 1), dtype=np.float64)
        self.L.eta_oracle_block_meta(T, d, bs, kvd, K.ctypes.data, c.ctypes.data_as(_dp),
                                     v.ctypes.data_as(_dp), m.ctypes.data_as(_dp))
        return c[:nblk], v[:nblk], m[:nblk]

    def bounds(self, q, centroid, var, maxnorm, z: float = 4.0,
               mode: int = BOUND_COMBINED) -> np.ndarray:
        """The combined (mode 0) or max-norm (mode 1) bound per block; the centered
        bound has its own call (bounds_centered)."""
        if mode not in (BOUND_COMBINED, BOUND_GEO):
            raise ValueError(f"bound mode {mode}: use bounds_centered for the centered bound")
        q = _c(q, np.float32)
        centroid = _c(centroid, np.float64)
        var = _c(var, np.float64)
        maxnorm = _c(maxnorm, np.float64)
        nblk, d = centroid.shape
        U = np.empty(max(nblk, 1), dtype=np.float64)
        self.L.eta_oracle_bounds(nblk, d, q.ctypes.data_as(_fp), centroid.ctypes.data_as(_dp),
                                 var.ctypes.data_as(_dp), maxnorm.ctypes.data_as(_dp),
                                 float(z), int(mode), U.ctypes.data_as(_dp))
        return U[:nblk]

    def block_maxdev(self, K, T: int, bs: int = 64) -> np.ndarray:
        """K [T_cap,d] (float32, or uint16 bf16 bits) -> per block, the largest
        distance of a key from the block's centroid [nblk]."""
        K, kvd = _kv(K)
        d = K.shape[1]
        assert 0 <= T <= K.shape[0]
        nblk = (T + bs - 1) // bs
        out = np.empty(max(nblk, 1), dtype=np.float64)
        self.L.eta_oracle_block_maxdev(T, d, bs, kvd, K.ctypes.data, out.ctypes.data_as(_dp))
        return out[:nblk]

    def bounds_centered(self, q, centroid, maxnorm, maxdev) -> np.ndarray:
        """min(s|q|maxnorm, s(q.c + |q| maxdev)) per block."""
        q = _c(q, np.float32)
        centroid = _c(centroid, np.float64)
        maxnorm = _c(maxnorm, np.float64)
        maxdev = _c(maxdev, np.float64)
        nblk, d = centroid.shape
        U = np.empty(max(nblk, 1), dtype=np.float64)
        self.L.eta_oracle_bounds_centered(nblk, d, q.ctypes.data_as(_fp),
                                          centroid.ctypes.data_as(_dp),
                                          maxnorm.ctypes.data_as(_dp),
                                          maxdev.ctypes.data_as(_dp), U.ctypes.data_as(_dp))
        return U[:nblk]

    def screen(self, U, tau: float) -> np.ndarray:
        U = _c(U, np.float64)
        idx = np.empty(max(len(U), 1), dtype=np.int32)
        cnt = self.L.eta_oracle_screen(len(U), U.ctypes.data_as(_dp), float(tau),
                                       idx.ctypes.data_as(_ip))
        return idx[:cnt].copy()

    def union(self, lists, nblk: int) -> np.ndarray:
        """Ascending union of a group's admitted lists (a list of int arrays)."""
        g = len(lists)
        stride = max([len(x) for x in lists] + [1])
        buf = np.zeros((g, stride), dtype=np.int32)
        cnts = np.zeros(g, dtype=np.int32)
        for j, x in enumerate(lists):
            buf[j, :len(x)] = x
            cnts[j] = len(x)
        out = np.empty(max(nblk, 1), dtype=np.int32)
        n = self.L.eta_oracle_union(g, buf.ctypes.data_as(_ip), cnts.ctypes.data_as(_ip), stride,
                                    nblk, out.ctypes.data_as(_ip))
        return out[:n].copy()

    def gate(self, S: float, tau: float, beta: float = 5.0, hard: bool = False) -> float:
        return self.L.eta_oracle_gate(float(S), float(tau), float(beta), int(bool(hard)))

    def attend(self, q, K, V, T: int, tau: float, idx, beta: float = 5.0,
               hard: bool = False, bs: int = 64):
        """Gated softmax attention of one unit over the admitted blocks idx.

        Returns (out fp64 [d], lse float)."""
        q = _c(q, np.float32)
        K, kvd = _kv(K)
        V, kvd_v = _kv(V)
        assert kvd == kvd_v and K.shape == V.shape
        d = K.shape[1]
        idx = _c(idx, np.int32)
        idx_buf = idx if len(idx) else np.zeros(1, dtype=np.int32)
        out = np.empty(d, dtype=np.float64)
        lse = np.empty(1, dtype=np.float64)
        self.L.eta_oracle_attend(T, d, bs, kvd, q.ctypes.data_as(_fp), K.ctypes.data,
                                 V.ctypes.data, float(tau), idx_buf.ctypes.data_as(_ip),
                                 len(idx), float(beta), int(bool(hard)),
                                 out.ctypes.data_as(_dp), lse.ctypes.data_as(_dp))
        return out, float(lse[0])

    def prefill(self, Q, K, V, T_k: int, tau, beta: float = 5.0, hard: bool = False):
        """Training-time forward of one (row, head): Q [T_q, d] (float32, or uint16
        bf16 bit patterns, widened exactly), K, V [>= T_k, d], tau [T_q]; query t sits
        at position T_k - T_q + t. Returns (out fp64 [T_q, d], lse [T_q],
        gate_sum [T_q])."""
        if Q.dtype == np.uint16:
            Q = (np.ascontiguousarray(Q).astype(np.uint32) << 16).view(np.float32)
        Q = _c(Q, np.float32)
        T_q, d = Q.shape
        K, kvd = _kv(K)
        V, kvd_v = _kv(V)
        assert kvd == kvd_v and K.shape == V.shape and K.shape[1] == d
        assert 0 <= T_q <= T_k <= K.shape[0]
        tau = _c(tau, np.float64)
        out = np.empty((max(T_q, 1), d), dtype=np.float64)
        lse = np.empty(max(T_q, 1), dtype=np.float64)
        gs = np.empty(max(T_q, 1), dtype=np.float64)
        tau_buf = tau if T_q else np.zeros(1)
        rc = self.L.eta_oracle_prefill(T_q, T_k, d, kvd, Q.ctypes.data_as(_fp), K.ctypes.data,
                                       V.ctypes.data, tau_buf.ctypes.data_as(_dp), float(beta),
                                       int(bool(hard)), out.ctypes.data_as(_dp),
                                       lse.ctypes.data_as(_dp), gs.ctypes.data_as(_dp))
        assert rc == 0
        return out[:T_q], lse[:T_q], gs[:T_q]

    def unit_step(self, q_unit, K, V, T, tau, meta, z=4.0, mode=BOUND_COMBINED, beta=5.0,
                  hard=False, bs=64):
        """Bound + screen + attend for one unit, given its metadata (c, var, maxnorm).

        Returns dict(U, idx, out, lse)."""
        c, v, m = meta
        U = self.bounds(q_unit, c, v, m, z=z, mode=mode)
        idx = self.screen(U, tau)
        out, lse = self.attend(q_unit, K, V, T, tau, idx, beta=beta, hard=hard, bs=bs)
        return {"U": U, "idx": idx, "out": out, "lse": lse}


_default = None


def default() -> OracleLib:
    """The oracle built from ``eta_oracle.c`` (compiled on first use if absent), or the
    build of it that ETA_ORACLE_LIB names (a sanitizer-instrumented one, for instance)."""
    global _default
    if _default is None:
        path = os.environ.get("ETA_ORACLE_LIB")
        if not path:
            path = LIB_PATH
            if not os.path.exists(path):
                compile_oracle()
        _default = OracleLib(path)
    return _default
