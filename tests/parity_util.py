"""Helpers for the GPU parity tests: seeded inputs, device upload, the gates.

Gates (GPU result vs the fp64 oracle on the same bf16 inputs):
  O:   max |err| <= 2e-2 and mean |err| <= 2e-3 (bf16 output, fp32 accumulation)
  LSE: max |err| <= 1e-3
  every output finite where the oracle is finite; -inf LSE / zero O where no key is visible.
"""
from __future__ import annotations

import math
import sys

import numpy as np

import gen

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(*args):
    """Name the case before a GPU step, flushed, so a failing run still shows it."""
    print("[parity]", *args, flush=True)
    sys.stdout.flush()


def fwd_inputs(seed, B, H, H_kv, N_q, N_k, d, f32_draw=False):
    """bf16 Q/K/V (uint16 bits) from the seeded generator; with f32_draw also the raw fp32 draws."""
    Q = gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, N_q, d))
    K = gen.normal_bf16(seed, gen.TENSOR_K, (B, H_kv, N_k, d))
    V = gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N_k, d))
    if not f32_draw:
        return Q, K, V
    raw = (gen.normal_f32(seed, gen.TENSOR_Q, (B, H, N_q, d)), gen.normal_f32(seed, gen.TENSOR_K, (B, H_kv, N_k, d)),
           gen.normal_f32(seed, gen.TENSOR_V, (B, H_kv, N_k, d)))
    return Q, K, V, raw


def decode_inputs(seed, B, H, H_kv, N_k, d, q_scale=3.0):
    Q = gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, 1, d), q_scale)
    K = gen.normal_bf16(seed, gen.TENSOR_K, (B, H_kv, N_k, d))
    V = gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N_k, d))
    return Q, K, V


def to_dev(a):
    """uint16 bf16 bit patterns (numpy) -> torch bfloat16 on cuda:0."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def bf16_dev_to_f64(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def sample_rows(B, H, N_q, n_random, seed, tile=128):
    """Flat row ids (b*H + h)*N_q + i: tile edges, the ragged tail and random rows, in every (b, h)."""
    rng = np.random.default_rng(seed)
    edge = sorted({i for i in (0, 1, 31, 32, 63, 64, tile - 1, tile, tile + 1, N_q // 2, N_q - 2, N_q - 1)
                   if 0 <= i < N_q})
    rows = []
    for bh in range(B * H):
        rows.extend(bh * N_q + i for i in edge)
    rows.extend(rng.integers(0, B * H * N_q, size=n_random).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))


def check(name, O_gpu, O_ref, L_gpu, L_ref):
    """Apply the gates; returns a dict of the measured errors."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    L_gpu = np.asarray(L_gpu, dtype=np.float64)
    L_ref = np.asarray(L_ref, dtype=np.float64)
    assert O_gpu.shape == O_ref.shape and L_gpu.shape == L_ref.shape, name
    assert np.all(np.isfinite(O_gpu)), "%s: non-finite O" % name
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L_gpu), empty), "%s: -inf LSE pattern differs" % name
    assert np.all(np.isfinite(L_gpu[~empty])), "%s: non-finite LSE" % name
    err = np.abs(O_gpu - O_ref)
    lerr = np.abs(L_gpu[~empty] - L_ref[~empty]) if (~empty).any() else np.zeros(1)
    res = {"o_max": float(err.max()) if err.size else 0.0, "o_mean": float(err.mean()) if err.size else 0.0,
           "lse_max": float(lerr.max())}
    say(name, res)
    assert res["o_max"] <= O_MAX, "%s: O max-abs %.3g > %.3g" % (name, res["o_max"], O_MAX)
    assert res["o_mean"] <= O_MEAN, "%s: O mean-abs %.3g > %.3g" % (name, res["o_mean"], O_MEAN)
    assert res["lse_max"] <= LSE_MAX, "%s: LSE max-abs %.3g > %.3g" % (name, res["lse_max"], LSE_MAX)
    return res


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def scale_for(d):
    return 1.0 / math.sqrt(d)
