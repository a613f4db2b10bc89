"""exact_attention_59_amd -- exact attention on MI355X through the C ABI of libfa.so.

A thin ctypes binding: every function below validates torch tensors, passes their
device pointers and the current HIP stream to the function of the same name in
``include/fa.h``, and raises on a non-zero status.  All arithmetic runs in the
gfx950 kernels; there is no CPU fallback.  PyTorch is used only to hold device
memory and to name the stream.

    fwd(q, k, v, causal=False, scale=None)   -> (o, lse)          fa_fwd
    bwd(q, k, v, o, lse, do, causal, scale)  -> (dq, dk, dv)      fa_bwd
    fp8_quantize(q, k, v, signs, incoherent) -> (q8, k8, vt8, qs, ks, vs)  fa_fp8_quantize
    fwd_fp8(q8, k8, vt8, qs, ks, vs, causal, scale) -> (o, lse)  fa_fwd_fp8
    decode_split(q, k, v, num_splits, scale) -> (o_part, lse_part) fa_decode_split
    combine(o_part, lse_part)                -> (o, lse)          fa_combine
    decode(q, k, v, num_splits=None, scale)  -> (o, lse)          both, on one stream
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fwd", "bwd", "bwd_workspace_bytes", "fp8_quantize", "fwd_fp8", "fp8_block_rows", "decode_split", "decode_split_paged", "combine", "decode", "decode_num_splits",
           "decode_workspace_bytes",
           "fwd_tile_shape", "fwd_tile_count", "strerror", "library", "library_path", "FAError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libfa.so")
_lib = None

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_ARG, FA_ERR_HIP, FA_ERR_CAPACITY = range(8)


class FAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: status %d (%s)" % (fn, status, strerror(status)))
        self.status = status


def library_path() -> str:
    return LIBRARY


def library():
    """Load libfa.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError("libfa.so is not built (%s); run `python -m exact_attention_59_amd.build` "
                              "or __graft_entry__.build()" % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_fwd_poly_exp2.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp]
        lib.fa_exp2_poly.argtypes = [vp, vp, ctypes.c_longlong, vp]
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        u64 = ctypes.c_uint64
        lib.fa_fp8_quantize.argtypes = [vp, vp, vp, i32, u64, u64, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                        i32, vp]
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_fp8_block_rows.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.fa_decode_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_decode_split_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                              f32, vp]
        lib.fa_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp]
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                        i32, f32, vp]
        lib.fa_decode_static.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
        lib.fa_decode_counters_reset.argtypes = [vp, i32, i32, i32, vp]
        lib.fa_decode_counters_check.argtypes = [vp, i32, i32, i32, vp, vp]
        lib.fa_decode_counter_bytes.argtypes = [i32, i32, i32]
        lib.fa_decode_counter_bytes.restype = ctypes.c_size_t
        lib.fa_decode_num_splits.argtypes = [i32, i32, i32, i32]
        lib.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_tile_shape.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.fa_fwd_tile_count.argtypes = [i32, i32, i32, i32]
        lib.fa_fwd_tile_count.restype = ctypes.c_longlong
        lib.fa_strerror.argtypes = [i32]
        lib.fa_strerror.restype = ctypes.c_char_p
        for fn in (lib.fa_fwd, lib.fa_bwd, lib.fa_fp8_quantize, lib.fa_fwd_fp8, lib.fa_fp8_block_rows, lib.fa_decode_split, lib.fa_decode_split_paged, lib.fa_combine, lib.fa_decode_num_splits, lib.fa_decode_static,
                   lib.fa_decode_counters_reset, lib.fa_decode_counters_check,
                   lib.fa_fwd_tile_shape):
            fn.restype = i32
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return library().fa_strerror(int(status)).decode()


def _check(fn: str, status: int):
    if status != FA_OK:
        raise FAError(fn, status)


_torch_mod = None


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch

        _torch_mod = torch
    return _torch_mod


def _stream_ptr(t):
    """Raw hipStream_t of torch's current stream on t's device (no Stream object built)."""
    torch = _torch()
    return torch._C._cuda_getCurrentRawStream(t.device.index)


def _need(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a HIP device (got %s); the library has no CPU path" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions (got shape %s)" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None, poly_exp2: int = 0):
    """fa_fwd.  q [B,H,N_q,d], k/v [B,H_kv,N_k,d] bf16 -> o [B,H,N_q,d] bf16, lse [B,H,N_q] fp32.
    poly_exp2 in (1, 2, 4): fa_fwd_poly_exp2 with that many of every four softmax exponentials
    taken by the FMA-unit polynomial (0: fa_fwd)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, N_q, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, N_q):
        raise ValueError("output shapes do not match q")
    if poly_exp2:
        _check("fa_fwd_poly_exp2", library().fa_fwd_poly_exp2(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv, N_q, N_k, d,
            int(bool(causal)), float(scale), int(poly_exp2), _stream_ptr(q)))
    else:
        _check("fa_fwd", library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                          B, H, H_kv, N_q, N_k, d, int(bool(causal)), float(scale), _stream_ptr(q)))
    return out, lse


def exp2_poly(x, out=None):
    """fa_exp2_poly: y = 2^x with the forward's polynomial (x: fp32 CUDA tensor, any shape)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 CUDA tensor")
    out = torch.empty_like(x) if out is None else out
    if out.dtype != torch.float32 or out.shape != x.shape or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous float32 tensor shaped like x")
    _check("fa_exp2_poly", library().fa_exp2_poly(x.data_ptr(), out.data_ptr(), x.numel(), _stream_ptr(x)))
    return out


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
        workspace=None):
    """fa_bwd.  q, o, do [B,H,N_q,d], k/v [B,H_kv,N_k,d] bf16, lse [B,H,N_q] fp32 (the forward's)
    -> dq [B,H,N_q,d], dk/dv [B,H_kv,N_k,d] bf16.  workspace: fp32 tensor of at least B*H*N_q
    elements (allocated when None)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, H, N_q, d = q.shape
    Bk, H_kv, N_k, dk_ = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk_ != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape) or tuple(lse.shape) != (B, H, N_q):
        raise ValueError("o, do and lse must match q: o %s do %s lse %s" % (tuple(o.shape), tuple(do.shape),
                                                                           tuple(lse.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _need(t, n, torch.bfloat16, 4)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError("%s must have shape %s" % (n, tuple(ref.shape)))
    if workspace is None:
        workspace = torch.empty(B * H * N_q, dtype=torch.float32, device=q.device)
    _need(workspace, "workspace", torch.float32, 1)
    if workspace.numel() * 4 < bwd_workspace_bytes(B, H, N_q):
        raise ValueError("workspace too small: %d floats, need %d" % (workspace.numel(), B * H * N_q))
    _check("fa_bwd", library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                      workspace.data_ptr(), B, H, H_kv, N_q, N_k, d, int(bool(causal)),
                                      float(scale), _stream_ptr(q)))
    return dq, dk, dv


def bwd_workspace_bytes(B: int, H: int, N_q: int) -> int:
    return int(library().fa_bwd_workspace_bytes(B, H, N_q))


def fp8_block_rows():
    """(query rows, keys) per FP8 quantisation block."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _check("fa_fp8_block_rows", library().fa_fp8_block_rows(ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def fp8_quantize(q, k, v, sign_lo: int = 0, sign_hi: int = 0, incoherent: bool = True):
    """fa_fp8_quantize.  q [B,H,N_q,d], k/v [B,H_kv,N_k,d] bf16 -> (q8, k8, vt8, q_scale, k_scale,
    v_scale): e4m3 codes as uint8 (q8 like q, k8 like k, vt8 [B,H_kv,T_c,d,64]) and fp32 block
    scales.  sign_lo / sign_hi: the 128-bit random sign mask of the transform."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, H, N_q, d = q.shape
    Bk, H_kv, N_k, dk_ = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk_ != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    qr, kr = fp8_block_rows()
    TQ, TC = -(-N_q // qr), -(-N_k // kr)
    dev = q.device
    q8 = torch.empty((B, H, N_q, d), dtype=torch.uint8, device=dev)
    k8 = torch.empty((B, H_kv, N_k, d), dtype=torch.uint8, device=dev)
    vt8 = torch.empty((B, H_kv, TC, d, kr), dtype=torch.uint8, device=dev)
    qs = torch.empty((B, H, TQ), dtype=torch.float32, device=dev)
    ks = torch.empty((B, H_kv, TC), dtype=torch.float32, device=dev)
    vs = torch.empty((B, H_kv, TC), dtype=torch.float32, device=dev)
    _check("fa_fp8_quantize", library().fa_fp8_quantize(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), int(bool(incoherent)), int(sign_lo) & (2**64 - 1),
        int(sign_hi) & (2**64 - 1), q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs.data_ptr(), ks.data_ptr(),
        vs.data_ptr(), B, H, H_kv, N_q, N_k, d, _stream_ptr(q)))
    return q8, k8, vt8, qs, ks, vs


def fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal: bool = False, scale: float | None = None, out=None,
            lse=None):
    """fa_fwd_fp8 on fp8_quantize's outputs -> o [B,H,N_q,d] bf16, lse [B,H,N_q] fp32."""
    torch = _torch()
    _need(q8, "q8", torch.uint8, 4)
    _need(k8, "k8", torch.uint8, 4)
    _need(vt8, "vt8", torch.uint8, 5)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _need(t, n, torch.float32, 3)
    B, H, N_q, d = q8.shape
    Bk, H_kv, N_k, dk_ = k8.shape
    qr, kr = fp8_block_rows()
    TQ, TC = -(-N_q // qr), -(-N_k // kr)
    if (Bk != B or dk_ != d or tuple(vt8.shape) != (B, H_kv, TC, d, kr) or tuple(q_scale.shape) != (B, H, TQ)
            or tuple(k_scale.shape) != (B, H_kv, TC) or tuple(v_scale.shape) != (B, H_kv, TC)):
        raise ValueError("fp8 operand shapes do not match fp8_quantize's layout")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N_q, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q8.device)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    _check("fa_fwd_fp8", library().fa_fwd_fp8(
        q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
        out.data_ptr(), lse.data_ptr(), B, H, H_kv, N_q, N_k, d, int(bool(causal)), float(scale), _stream_ptr(q8)))
    return out, lse


def decode_split(q, k, v, num_splits: int, scale: float | None = None, o_part=None, lse_part=None):
    """fa_decode_split.  q [B,H,d], k/v [B,H_kv,N_k,d] bf16 -> o_part [B,H,S,d], lse_part [B,H,S] fp32."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    S = int(num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o_part is None:
        o_part = torch.empty((B, H, S, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    if tuple(o_part.shape) != (B, H, S, d) or tuple(lse_part.shape) != (B, H, S):
        raise ValueError("partial output shapes do not match")
    _check("fa_decode_split",
           library().fa_decode_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                     lse_part.data_ptr(), B, H, H_kv, N_k, d, S, float(scale), _stream_ptr(q)))
    return o_part, lse_part


def decode_split_paged(q, k_pages, v_pages, block_table, seq_lens, num_splits: int, scale: float | None = None,
                       o_part=None, lse_part=None):
    """fa_decode_split_paged.  q [B,H,d] bf16; k/v pages [num_pages,H_kv,P,d] bf16; block_table
    [B,max_pages] int32; seq_lens [B] int32 -> o_part [B,H,S,d], lse_part [B,H,S] fp32."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, H, d = q.shape
    num_pages, H_kv, P, dk = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape) or dk != d:
        raise ValueError("shape mismatch: q %s k_pages %s v_pages %s" % (tuple(q.shape), tuple(k_pages.shape),
                                                                      tuple(v_pages.shape)))
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    max_pages = block_table.shape[1]
    S = int(num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o_part is None:
        o_part = torch.empty((B, H, S, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    if tuple(o_part.shape) != (B, H, S, d) or tuple(lse_part.shape) != (B, H, S):
        raise ValueError("partial output shapes do not match")
    _check("fa_decode_split_paged",
           library().fa_decode_split_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                           block_table.data_ptr(), seq_lens.data_ptr(), o_part.data_ptr(),
                                           lse_part.data_ptr(), B, H, H_kv, P, max_pages, num_pages, d, S,
                                           float(scale), _stream_ptr(q)))
    return o_part, lse_part


def combine(o_part, lse_part, out=None, lse=None):
    """fa_combine.  o_part [B,H,S,d], lse_part [B,H,S] fp32 -> o [B,H,d] bf16, lse [B,H] fp32."""
    torch = _torch()
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    B, H, S, d = o_part.shape
    if tuple(lse_part.shape) != (B, H, S):
        raise ValueError("lse_part shape does not match o_part")
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=o_part.device)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    _check("fa_combine", library().fa_combine(o_part.data_ptr(), lse_part.data_ptr(), out.data_ptr(),
                                              lse.data_ptr(), B, H, d, S, _stream_ptr(o_part)))
    return out, lse


def decode(q, k, v, num_splits: int | None = None, scale: float | None = None, counters=None, o_part=None,
           lse_part=None, out=None, lse=None, check_counters: bool = False):
    """fa_decode: split and merge in one launch.  q [B,H,d], k/v [B,H_kv,N_k,d] bf16 -> (o [B,H,d] bf16,
    lse [B,H] fp32).  counters: int32 [fa_decode_counter_bytes / 4], zero before the first call and
    left zero by every completed call (a new zeroed one is made if None); o_part / lse_part: the
    workspace of decode_split.  check_counters: verify (with fa_decode_counters_check and a
    synchronisation) that caller-provided counters are zero, and raise instead of launching if not."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    S = int(num_splits) if num_splits is not None else decode_num_splits(B, H_kv, N_k, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n_counters = decode_counter_bytes(B, H, H_kv) // 4
    if counters is None:
        counters = torch.zeros((max(n_counters, 1),), dtype=torch.int32, device=q.device)
    _need(counters, "counters", torch.int32, 1)
    if counters.numel() < n_counters:
        raise ValueError("counters must hold at least %d elements" % n_counters)
    if check_counters:
        bad = decode_counters_check(counters, B, H, H_kv)
        if bad:
            raise RuntimeError("fa_decode: %d group counter(s) are not zero (never cleared, or shared by overlapping "
                               "calls); clear them with decode_counters_reset" % bad)
    if o_part is None:
        o_part = torch.empty((B, H, S, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    if tuple(o_part.shape) != (B, H, S, d) or tuple(lse_part.shape) != (B, H, S):
        raise ValueError("partial output shapes do not match")
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, H, d) or tuple(lse.shape) != (B, H):
        raise ValueError("output shapes do not match")
    _check("fa_decode",
           library().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(), lse_part.data_ptr(),
                               counters.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv, N_k, d, S,
                               float(scale), _stream_ptr(q)))
    return out, lse



def decode_counters_reset(counters, B: int, H: int, H_kv: int):
    """fa_decode_counters_reset: zero the group counters of fa_decode on the current stream."""
    torch = _torch()
    _need(counters, "counters", torch.int32, 1)
    if counters.numel() < decode_counter_bytes(B, H, H_kv) // 4:
        raise ValueError("counters too small")
    _check("fa_decode_counters_reset",
           library().fa_decode_counters_reset(counters.data_ptr(), B, H, H_kv, _stream_ptr(counters)))


def decode_counters_check(counters, B: int, H: int, H_kv: int) -> int:
    """fa_decode_counters_check: the number of non-zero group counters (synchronises the stream)."""
    torch = _torch()
    _need(counters, "counters", torch.int32, 1)
    if counters.numel() < decode_counter_bytes(B, H, H_kv) // 4:
        raise ValueError("counters too small")
    out = torch.full((1,), -1, dtype=torch.int32, device=counters.device)
    _check("fa_decode_counters_check",
           library().fa_decode_counters_check(counters.data_ptr(), B, H, H_kv, out.data_ptr(), _stream_ptr(counters)))
    return int(out.item())


def decode_static(q, k, v, num_splits: int | None = None, scale: float | None = None, out=None, lse=None):
    """fa_decode_static: fa_decode with its partials and counters in the library's static device
    scratch array (no workspace from the caller, no allocation in the call).  q [B,H,d], k/v
    [B,H_kv,N_k,d] bf16 -> (o [B,H,d] bf16, lse [B,H] fp32).  Calls that overlap on one device race."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, H, d = q.shape
    Bk, H_kv, N_k, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    S = int(num_splits) if num_splits is not None else decode_num_splits(B, H_kv, N_k, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, H, d) or tuple(lse.shape) != (B, H):
        raise ValueError("output shapes do not match")
    _check("fa_decode_static",
           library().fa_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      B, H, H_kv, N_k, d, S, float(scale), _stream_ptr(q)))
    return out, lse

def decode_paged(q, k_pages, v_pages, block_table, seq_lens, num_splits: int, scale: float | None = None,
                 counters=None, o_part=None, lse_part=None, out=None, lse=None):
    """fa_decode_paged: decode_split_paged and the merge in one launch -> (o [B,H,d] bf16, lse [B,H]
    fp32).  counters as for decode (a new zeroed one is made if None)."""
    torch = _torch()
    for t, nm, dt, nd in ((q, "q", torch.bfloat16, 3), (k_pages, "k_pages", torch.bfloat16, 4),
                          (v_pages, "v_pages", torch.bfloat16, 4), (block_table, "block_table", torch.int32, 2),
                          (seq_lens, "seq_lens", torch.int32, 1)):
        _need(t, nm, dt, nd)
    B, H, d = q.shape
    num_pages, H_kv, P, dk = k_pages.shape
    if tuple(v_pages.shape) != tuple(k_pages.shape) or dk != d:
        raise ValueError("shape mismatch: q %s k_pages %s v_pages %s" % (tuple(q.shape), tuple(k_pages.shape),
                                                                      tuple(v_pages.shape)))
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    max_pages = block_table.shape[1]
    S = int(num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    n_counters = decode_counter_bytes(B, H, H_kv) // 4
    if counters is None:
        counters = torch.zeros((max(n_counters, 1),), dtype=torch.int32, device=q.device)
    _need(counters, "counters", torch.int32, 1)
    if counters.numel() < n_counters:
        raise ValueError("counters must hold at least %d elements" % n_counters)
    if o_part is None:
        o_part = torch.empty((B, H, S, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    if tuple(o_part.shape) != (B, H, S, d) or tuple(lse_part.shape) != (B, H, S):
        raise ValueError("partial output shapes do not match")
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, H, d) or tuple(lse.shape) != (B, H):
        raise ValueError("output shapes do not match")
    _check("fa_decode_paged",
           library().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                     seq_lens.data_ptr(), o_part.data_ptr(), lse_part.data_ptr(),
                                     counters.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, H_kv, P, max_pages,
                                     num_pages, d, S, float(scale), _stream_ptr(q)))
    return out, lse


def decode_counter_bytes(B: int, H: int, H_kv: int) -> int:
    return int(library().fa_decode_counter_bytes(B, H, H_kv))


def decode_num_splits(B: int, H_kv: int, N_k: int, d: int) -> int:
    return int(library().fa_decode_num_splits(B, H_kv, N_k, d))


def decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(library().fa_decode_workspace_bytes(B, H, d, num_splits))


def fwd_tile_shape(d: int):
    r, c = ctypes.c_int(), ctypes.c_int()
    _check("fa_fwd_tile_shape", library().fa_fwd_tile_shape(d, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def fwd_tile_count(N_q: int, N_k: int, d: int, causal: bool) -> int:
    return int(library().fa_fwd_tile_count(N_q, N_k, d, int(bool(causal))))
