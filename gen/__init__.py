"""Seeded synthetic inputs shared by the oracle and the GPU path.

Only random numbers and bf16 rounding live here (no attention arithmetic).
The stream is defined in ``gen.c``: counter-based SplitMix64 words, a
Box-Muller pair per two words, float rounding, a float multiply by ``scale``
and (for bf16) round-to-nearest-even.  Every element is addressable by
(seed, tensor id, linear index), so any slice can be regenerated on its own.

Tensor ids used by the tests and the bench: Q = 0, K = 1, V = 2, dO (the upstream
gradient of the backward pass) = 3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libgen.so")
_lib = None

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile gen.c into libgen.so next to it (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        u64, u32, i64, f32, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        vp = ctypes.c_void_p
        lib.gen_normal_f32.argtypes = [u64, u32, i64, i64, f32, vp, i32]
        lib.gen_normal_bf16.argtypes = [u64, u32, i64, i64, f32, vp, i32]
        lib.gen_f32_to_bf16.argtypes = [vp, vp, i64]
        lib.gen_words.argtypes = [u64, u32, i64, i64, vp]
        lib.gen_bf16_rne.argtypes = [f32]
        lib.gen_bf16_rne.restype = ctypes.c_uint16
        lib.gen_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.gen_bf16_to_f32.restype = f32
        for fn in (lib.gen_normal_f32, lib.gen_normal_bf16, lib.gen_f32_to_bf16, lib.gen_words):
            fn.restype = None
        _lib = lib
    return _lib


def _threads(nthreads):
    if nthreads is not None:
        return int(nthreads)
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, tensor_id: int, shape, scale: float = 1.0, offset: int = 0, nthreads=None) -> np.ndarray:
    """float32 N(0,1)*scale, elements [offset, offset + prod(shape)) of the stream."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)
    _load().gen_normal_f32(seed, tensor_id, offset, n, scale, out.ctypes.data, _threads(nthreads))
    return out.reshape(shape)


def normal_bf16(seed: int, tensor_id: int, shape, scale: float = 1.0, offset: int = 0, nthreads=None) -> np.ndarray:
    """The same values as normal_f32, rounded to bf16; returned as uint16 bit patterns."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    _load().gen_normal_bf16(seed, tensor_id, offset, n, scale, out.ctypes.data, _threads(nthreads))
    return out.reshape(shape)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round a float32 array to bf16 (RNE); uint16 bit patterns of the same shape."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().gen_f32_to_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def words(seed: int, tensor_id: int, k0: int, n: int) -> np.ndarray:
    """Raw 64-bit stream words k0 .. k0+n-1."""
    out = np.empty(n, dtype=np.uint64)
    _load().gen_words(seed, tensor_id, k0, n, out.ctypes.data)
    return out


def bf16_rne_scalar(f: float) -> int:
    return int(_load().gen_bf16_rne(f))
