"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The GPU product path never calls it, and it shares
no code with the GPU kernels.  The arithmetic lives in ``oracle.c`` (plain C,
fp64, libm); this module only marshals numpy arrays.

Functions and the passages they follow (Lecture 11, "Kernel Optimization
Techniques: FlashAttention, flash-decoding and megakernel"):
  attention     standard attention, Algorithm 0 (section 2), safe softmax
                (section 3.4), LSE = m + ln l (section 5.1); with a key range
                it is flash-decoding's per-segment output (section 6.2).
  online_row    one-pass online softmax times V (section 3.1).
  merge         merge of partial states (m, l, o) (section 3.2).
  lse_combine   flash-decoding combine in LSE form (section 6.2).
  attention_bwd gradients of sum(dO * O) w.r.t. Q, K, V from the full P
                (section 5.1, the standard backward).

Parity pins: every function above is pinned by tests against facts the pages
or the mathematics fix (worked Exercise 1, closed forms, brute force in
high-precision decimals, an independent library routine).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_DTYPES = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}


def compile_library(src: str, out: str) -> str:
    """gcc -O2 (IEEE arithmetic: no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", tmp, src,
                           "-lm", "-lpthread"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_library(SOURCE, LIBRARY)
    return LIBRARY


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


class Oracle:
    """ctypes front end over one build of oracle.c."""

    def __init__(self, path: str | None = None):
        if path is None:
            if not os.path.exists(LIBRARY):
                build(force=True)
            path = LIBRARY
        lib = ctypes.CDLL(path)
        i64, d64, vp, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.oracle_attention.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, i32, d64,
                                         i64, i64, vp, i64, vp, vp, vp, i32]
        lib.oracle_attention.restype = i32
        lib.oracle_online_row.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_online_row.restype = None
        lib.oracle_merge.argtypes = [d64, d64, vp, d64, d64, vp, i64, vp, vp, vp]
        lib.oracle_merge.restype = None
        lib.oracle_lse_combine.argtypes = [vp, vp, i64, i64, vp, vp]
        lib.oracle_lse_combine.restype = None
        lib.oracle_attention_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, i32, d64,
                                             vp, vp, vp, vp, i32]
        lib.oracle_attention_bwd.restype = i32
        u64, f32 = ctypes.c_uint64, ctypes.c_float
        lib.oracle_fp8_quantize.argtypes = [vp, i64, i64, i64, i64, i32, u64, u64, f32, vp, vp]
        lib.oracle_fp8_quantize.restype = i32
        lib.oracle_e4m3_encode_n.argtypes = [vp, i64, vp]
        lib.oracle_e4m3_encode_n.restype = None
        lib.oracle_e4m3_decode_n.argtypes = [vp, i64, vp]
        lib.oracle_e4m3_decode_n.restype = None
        lib.oracle_fwht_rows.argtypes = [vp, i64, i64]
        lib.oracle_fwht_rows.restype = None
        self.lib = lib

    # ------------------------------------------------------------------ Algorithm 0
    def attention(self, Q, K, V, causal=False, scale=None, rows=None, k_range=None,
                  return_p=False, nthreads=None):
        """Exact attention.  Q [B,H,N_q,d], K/V [B,H_kv,N_k,d]; uint16 (bf16 bits), float32 or float64.

        rows: optional flat row ids (b*H + h)*N_q + i.  k_range: optional (k_lo, k_hi).
        Returns (O [n_rows, d] or [B,H,N_q,d], LSE [n_rows] or [B,H,N_q][, P]).
        """
        Q, K, V = (np.ascontiguousarray(x) for x in (Q, K, V))
        if not (Q.dtype == K.dtype == V.dtype) or Q.dtype not in _DTYPES:
            raise TypeError("Q, K, V must share one of uint16 (bf16), float32, float64")
        B, H, N_q, d = Q.shape
        Bk, H_kv, N_k, dk = K.shape
        if V.shape != K.shape or Bk != B or dk != d:
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        k_lo, k_hi = (0, N_k) if k_range is None else (int(k_range[0]), int(k_range[1]))
        if rows is None:
            n_rows, rows_arr, rows_ptr = B * H * N_q, None, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64).ravel()
            n_rows, rows_ptr = rows_arr.size, rows_arr.ctypes.data
        O = np.empty((n_rows, d), dtype=np.float64)
        LSE = np.empty(n_rows, dtype=np.float64)
        P = np.empty((n_rows, N_k), dtype=np.float64) if return_p else None
        rc = self.lib.oracle_attention(Q.ctypes.data, K.ctypes.data, V.ctypes.data, _DTYPES[Q.dtype],
                                       B, H, H_kv, N_q, N_k, d, int(bool(causal)), float(scale),
                                       k_lo, k_hi, rows_ptr, n_rows, O.ctypes.data, LSE.ctypes.data,
                                       P.ctypes.data if P is not None else None,
                                       host_threads() if nthreads is None else int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention failed with code %d" % rc)
        if rows is None:
            O = O.reshape(B, H, N_q, d)
            LSE = LSE.reshape(B, H, N_q)
            if P is not None:
                P = P.reshape(B, H, N_q, N_k)
        return (O, LSE, P) if return_p else (O, LSE)

    # ------------------------------------------------------------------ online softmax
    def online_row(self, s, Vr, block):
        """One pass over scores s [n] and value rows Vr [n, d] in blocks; returns dict."""
        s = np.ascontiguousarray(s, dtype=np.float64)
        Vr = np.ascontiguousarray(Vr, dtype=np.float64)
        n = s.size
        d = Vr.shape[1] if Vr.ndim == 2 else 0
        nb = -(-n // block) if n else 0
        o = np.empty(max(d, 1))
        m, l = ctypes.c_double(), ctypes.c_double()
        mt, lt, at = np.empty(max(nb, 1)), np.empty(max(nb, 1)), np.empty(max(nb, 1))
        self.lib.oracle_online_row(s.ctypes.data, Vr.ctypes.data, n, d, int(block), o.ctypes.data,
                                   ctypes.byref(m), ctypes.byref(l), mt.ctypes.data, lt.ctypes.data,
                                   at.ctypes.data)
        return {"o": o[:d], "m": m.value, "l": l.value, "m_trace": mt[:nb], "l_trace": lt[:nb],
                "alpha_trace": at[:nb]}

    # ------------------------------------------------------------------ merges
    def merge(self, a, b):
        """a, b: (m, l, o) states; returns the merged (m, l, o)."""
        m_a, l_a, o_a = a
        m_b, l_b, o_b = b
        o_a = np.ascontiguousarray(o_a, dtype=np.float64)
        o_b = np.ascontiguousarray(o_b, dtype=np.float64)
        d = o_a.size
        out = np.empty(max(d, 1))
        m, l = ctypes.c_double(), ctypes.c_double()
        self.lib.oracle_merge(float(m_a), float(l_a), o_a.ctypes.data, float(m_b), float(l_b),
                              o_b.ctypes.data, d, ctypes.byref(m), ctypes.byref(l), out.ctypes.data)
        return m.value, l.value, out[:d]

    def lse_combine(self, lse_s, o_s):
        """lse_s [S], o_s [S, d] -> (lse, o [d])."""
        lse_s = np.ascontiguousarray(lse_s, dtype=np.float64)
        o_s = np.ascontiguousarray(o_s, dtype=np.float64)
        S, d = o_s.shape
        out = np.empty(max(d, 1))
        lse = ctypes.c_double()
        self.lib.oracle_lse_combine(lse_s.ctypes.data, o_s.ctypes.data, S, d, ctypes.byref(lse),
                                    out.ctypes.data)
        return lse.value, out[:d]


    # ------------------------------------------------------------------ backward
    def attention_bwd(self, Q, K, V, dO, causal=False, scale=None, nthreads=None):
        """Gradients of sum(dO * O).  Q, dO [B,H,N_q,d], K/V [B,H_kv,N_k,d] (one shared dtype).

        Returns (dQ [B,H,N_q,d], dK [B,H_kv,N_k,d], dV [B,H_kv,N_k,d], D [B,H,N_q]) in fp64.
        """
        Q, K, V, dO = (np.ascontiguousarray(x) for x in (Q, K, V, dO))
        if not (Q.dtype == K.dtype == V.dtype == dO.dtype) or Q.dtype not in _DTYPES:
            raise TypeError("Q, K, V, dO must share one of uint16 (bf16), float32, float64")
        B, H, N_q, d = Q.shape
        Bk, H_kv, N_k, dk = K.shape
        if V.shape != K.shape or Bk != B or dk != d or dO.shape != Q.shape:
            raise ValueError("shape mismatch")
        if scale is None:
            scale = 1.0 / np.sqrt(d)
        dQ = np.empty((B, H, N_q, d))
        dK = np.empty((B, H_kv, N_k, d))
        dV = np.empty((B, H_kv, N_k, d))
        D = np.empty((B, H, N_q))
        rc = self.lib.oracle_attention_bwd(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dO.ctypes.data,
                                           _DTYPES[Q.dtype], B, H, H_kv, N_q, N_k, d, int(bool(causal)),
                                           float(scale), dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data,
                                           D.ctypes.data, host_threads() if nthreads is None else int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_bwd failed with code %d" % rc)
        return dQ, dK, dV, D


    # ------------------------------------------------------------------ FP8 quantisation
    def e4m3_encode(self, x):
        """float32 array -> uint8 OCP e4m3fn codes (nearest-even)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_e4m3_encode_n(x.ctypes.data, x.size, out.ctypes.data)
        return out

    def e4m3_decode(self, c):
        """uint8 e4m3fn codes -> float64 values (NaN for the NaN codes)."""
        c = np.ascontiguousarray(c, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e4m3_decode_n(c.ctypes.data, c.size, out.ctypes.data)
        return out

    def fwht(self, x):
        """fp32 fast Walsh-Hadamard transform (unnormalised) of every row of x [..., d]."""
        x = np.array(x, dtype=np.float32, copy=True, order="C")
        d = x.shape[-1]
        self.lib.oracle_fwht_rows(x.ctypes.data, x.size // d, d)
        return x

    def fp8_quantize(self, X, block, transform=False, sign_lo=0, sign_hi=0, post_scale=1.0):
        """bf16 X [..., N, d] (uint16 bits) -> (codes uint8 [..., N, d], scales float32 [..., ceil(N/block)])."""
        X = np.ascontiguousarray(X)
        if X.dtype != np.uint16:
            raise TypeError("X must hold bf16 bits (uint16)")
        *lead, N, d = X.shape
        n_heads = int(np.prod(lead)) if lead else 1
        n_blocks = -(-N // block)
        codes = np.empty(X.shape, dtype=np.uint8)
        scales = np.empty(tuple(lead) + (n_blocks,), dtype=np.float32)
        rc = self.lib.oracle_fp8_quantize(X.ctypes.data, n_heads, N, d, block, int(bool(transform)),
                                          int(sign_lo) & (2**64 - 1), int(sign_hi) & (2**64 - 1),
                                          float(post_scale), codes.ctypes.data, scales.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_fp8_quantize failed with code %d" % rc)
        return codes, scales


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(*args, **kwargs):
    return default().attention(*args, **kwargs)


def online_row(*args, **kwargs):
    return default().online_row(*args, **kwargs)


def merge(*args, **kwargs):
    return default().merge(*args, **kwargs)


def lse_combine(*args, **kwargs):
    return default().lse_combine(*args, **kwargs)


def attention_bwd(*args, **kwargs):
    return default().attention_bwd(*args, **kwargs)
