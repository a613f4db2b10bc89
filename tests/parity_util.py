"""Helpers for the GPU parity tests: seeded inputs, device upload, the gates.

Gates (GPU result vs the fp64 oracle on the same bf16 inputs):
  O:   max |err| <= 2e-2 and mean |err| <= 2e-3 (bf16 output, fp32 accumulation)
  LSE: max |err| <= 1e-3
  every output finite where the oracle is finite; -inf LSE / zero O where no key is visible.

Gradient gates (dQ, dK, dV of the backward; each tensor on its own), normwise with
u = 2^-9, the unit roundoff of bf16 (m = max(max |ref|, 1e-2), a = max(mean |ref|, 1e-2);
the floor only matters for all-zero gradients):
  max |err| <= 4u m = 2^-7 m   and   mean |err| <= 2u a = 2^-8 a.
Derivation: every gradient element is rounded to bf16 once at the end (error at most
u |x|, about u |x| / 2 on average), and one factor of each product (P for dV, dS for dQ
and dK) is rounded to bf16 before it (at most u per term; the terms' signs are random, so
the sum's error stays of the order of u times the element's own size).  Both together
put the largest error near 2u of the largest element and the mean near u of the mean
element; an fp64 emulation of exactly these rounding points reproduces the kernel's
error statistics.  The gates allow twice that.

FP8 gates (fa_fwd_fp8; u8 = 2^-4, the unit roundoff of e4m3; m = max |O_ref|, a = mean |O_ref|):
  against the oracle on the dequantised tensors (what the kernel computes; its only extra
  rounding is P to e4m3, relative error at most u8 per weight, about 0.027 rms):
    max |err| <= u8 m, mean |err| <= u8 a, LSE max-abs <= 1e-3 (l sums the fp32 p);
  against the oracle on the original bf16 tensors (adds the e4m3 rounding of the
  transformed Q, K and of V, each at most u8 relative per element):
    max |err| <= 3 u8 m, mean |err| <= 2 u8 a, LSE max-abs <= 4 u8 (a score error of the
    order of u8 times the score, averaged over the row's weights).
  Measured on eight shapes: against the dequantised tensors max 0.53 u8 m and mean errors
  matching an fp64 emulation of the rounding of P to two digits; against the bf16 tensors
  max 1.3 u8 m, LSE 0.08.
"""
from __future__ import annotations

import math
import sys

import numpy as np

import gen

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
G_MAX, G_MEAN, G_FLOOR = 2.0 ** -7, 2.0 ** -8, 1e-2
U8 = 2.0 ** -4


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


def key_scale(pattern, N_k):
    """Per-key factor of a score-range stress pattern.

    ramp_up: the row maximum keeps growing along the keys, by more than any fixed slack
    per 64 keys; ramp_down: the first keys dominate and later ones never raise it;
    alternating: blocks of 64 keys switch between large and small scores."""
    j = np.arange(N_k, dtype=np.float64)
    if pattern == "ramp_up":
        return 0.2 + 3.0 * j / max(1, N_k - 1)
    if pattern == "ramp_down":
        return 3.2 - 3.0 * j / max(1, N_k - 1)
    if pattern == "alternating":
        return np.where((j // 64) % 2 == 1, 3.0, 0.3)
    raise ValueError(pattern)


def stress_inputs(seed, B, H, H_kv, N_q, N_k, d, pattern, q_scale=4.0):
    """bf16 Q/K/V whose scaled scores span tens of units: Q ~ N(0, q_scale^2), key j's row
    ~ N(0, key_scale(pattern)[j]^2), rounded to bf16 after scaling."""
    Q = gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, N_q, d), q_scale)
    Kf = gen.normal_f32(seed, gen.TENSOR_K, (B, H_kv, N_k, d))
    K = gen.f32_to_bf16((Kf * key_scale(pattern, N_k)[None, None, :, None]).astype(np.float32))
    V = gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N_k, d))
    return Q, K, V


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


def check_grads(name, gpu, ref, allow=None):
    """Apply the gradient gates to (dQ, dK, dV); returns the errors relative to m and a.

    allow: optional per-element allowances (arrays shaped like the gradients, or None) for
    error that an input carries in, e.g. o_rounding_allowance; each element's error is
    reduced by its allowance (not below zero) before the gates."""
    out = {}
    allow = allow or (None, None, None)
    for label, g, r, al in zip(("dQ", "dK", "dV"), gpu, ref, allow):
        g = np.asarray(g, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        assert g.shape == r.shape, "%s %s: shape %s vs %s" % (name, label, g.shape, r.shape)
        assert np.all(np.isfinite(g)), "%s: non-finite %s" % (name, label)
        m = max(float(np.abs(r).max()), G_FLOOR)
        a = max(float(np.abs(r).mean()), G_FLOOR)
        err = np.abs(g - r)
        if al is not None:
            err = np.maximum(err - np.abs(al), 0.0)
        out[label] = (float(err.max()) / m, float(err.mean()) / a, m)
    say(name, {k: "max %.2e m, mean %.2e a (m %.3g)" % v for k, v in out.items()})
    for label, (mx, mn, _) in out.items():
        assert mx <= G_MAX, "%s: %s max-abs %.3g m > %.3g m" % (name, label, mx, G_MAX)
        assert mn <= G_MEAN, "%s: %s mean-abs %.3g a > %.3g a" % (name, label, mn, G_MEAN)
    return out


def o_rounding_allowance(Q, K, dO, O_ref, O_bf16, L_ref, scale, causal):
    """First-order effect on (dQ, dK) of the O handed to the backward being O_bf16 (the bf16
    rounding of the exact O) instead of O itself.

    The backward's row term D_i = dO_i . O_i is taken from the stored O, so its rounding
    enters dS = P o (dP - D) as -P_ij dD_i with dD_i = dO_i . (O_bf16 - O)_i, giving
    dQ_i += -scale dD_i (P K)_i and dK_j += -scale sum_i P_ij dD_i Q_i.  In rows whose
    softmax is sharply peaked, dQ_i itself nearly cancels while this term does not, so it can
    exceed the gates that bound the backward's own rounding.  Inputs as the oracle takes
    them (uint16 bf16 bits for Q, K, dO, O_bf16; float64 O_ref, L_ref); P is rebuilt here
    from the oracle's L_ref.  Returns (allow_dQ, allow_dK, None)."""
    q = gen.bf16_to_f32(Q).astype(np.float64)
    k = gen.bf16_to_f32(K).astype(np.float64)
    do = gen.bf16_to_f32(dO).astype(np.float64)
    ob = gen.bf16_to_f32(O_bf16).astype(np.float64)
    B, H, N_q, d = q.shape
    H_kv, N_k = k.shape[1], k.shape[2]
    g = H // H_kv
    kk = np.repeat(k, g, axis=1)
    s = np.einsum("bhqd,bhkd->bhqk", q, kk) * scale
    if causal:
        hidden = np.arange(N_k)[None, :] > (np.arange(N_q)[:, None] + (N_k - N_q))
        s = np.where(hidden, -np.inf, s)
    finite = np.isfinite(L_ref)
    P = np.where(finite[..., None], np.exp(s - np.where(finite, L_ref, 0.0)[..., None]), 0.0)
    dD = (do * (ob - O_ref)).sum(-1)
    dQ = -scale * dD[..., None] * np.einsum("bhqk,bhkd->bhqd", P, kk)
    dK = -scale * np.einsum("bhqk,bhqd->bhkd", P, dD[..., None] * q)
    dK = dK.reshape(B, H_kv, g, N_k, d).sum(2)
    return dQ, dK, None


def check_fp8(name, O_gpu, O_q, L_gpu, L_q, O_x=None, L_x=None, lse_slack=None):
    """FP8 gates against the dequantised-tensor oracle (O_q, L_q) and, when given, the
    original-tensor oracle (O_x, L_x).  lse_slack: per-row bound of the fp8 matrix cores'
    product truncation (mfma_fp8_score_bound), added to the dequantised LSE gate."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    L_gpu = np.asarray(L_gpu, dtype=np.float64)
    assert np.all(np.isfinite(O_gpu)), "%s: non-finite O" % name
    out = {}
    for label, O_r, L_r, kmax, kmean, lmax in (("deq", O_q, L_q, U8, U8, 1e-3),
                                               ("exact", O_x, L_x, 3 * U8, 2 * U8, 4 * U8)):
        if O_r is None:
            continue
        O_r = np.asarray(O_r, dtype=np.float64)
        L_r = np.asarray(L_r, dtype=np.float64)
        empty = np.isneginf(L_r)
        assert np.array_equal(np.isneginf(L_gpu), empty), "%s: -inf LSE pattern differs" % name
        m = max(float(np.abs(O_r).max()), 1e-6)
        a = max(float(np.abs(O_r).mean()), 1e-6)
        err = np.abs(O_gpu - O_r)
        ldiff = np.abs(L_gpu - np.where(empty, 0.0, L_r))[~empty]
        lerr = float(ldiff.max()) if ldiff.size else 0.0
        out[label] = (float(err.max()) / m, float(err.mean()) / a, lerr)
        assert err.max() <= kmax * m, "%s: O max-abs %.3g m > %.3g m (%s)" % (name, err.max() / m, kmax, label)
        assert err.mean() <= kmean * a, "%s: O mean-abs %.3g a > %.3g a (%s)" % (name, err.mean() / a, kmean, label)
        if label == "deq" and lse_slack is not None:
            bound = (lmax + np.broadcast_to(np.asarray(lse_slack, dtype=np.float64), L_gpu.shape))[~empty]
            assert np.all(ldiff <= bound), "%s: LSE beyond the truncation bound by %.3g" % (name, (ldiff - bound).max())
        else:
            assert lerr <= lmax, "%s: LSE max-abs %.3g > %.3g (%s)" % (name, lerr, lmax, label)
    say(name, {k: "max %.3f u8*m, mean %.3f u8*a, lse %.1e" % (v[0] / U8, v[1] / U8, v[2]) for k, v in out.items()})
    return out


def mfma_fp8_score_bound(qd, kd, scale, rows_per_chunk=64):
    """Per query row, a bound on the score error of gfx950's fp8 matrix cores.  Within each group
    of 8 consecutive contraction slots (8 consecutive channels here) every product is truncated
    toward zero to a multiple of 2^(E - 13), E the group's largest exponent(q) + exponent(k)
    (pinned by test_fp8_gpu.py::test_fp8_matrix_core_product_truncation).  The group's largest
    product is at least 2^E and is not truncated, so the group loses less than 7 * 2^-13 times
    its largest product.  qd [B,H,N_q,d], kd [B,H_kv,N_k,d] dequantised (float64); returns
    [B,H,N_q]: scale * 7 * 2^-13 * max over keys of sum over groups of max |q_k k_k|, which
    bounds the row's LSE error from this source."""
    B, H, N_q, d = qd.shape
    H_kv = kd.shape[1]
    out = np.zeros((B, H, N_q))
    for b in range(B):
        for h in range(H):
            k = np.abs(kd[b, h // (H // H_kv)]).reshape(-1, d // 8, 8)  # [N_k, groups, 8]
            for r0 in range(0, N_q, rows_per_chunk):
                q = np.abs(qd[b, h, r0:r0 + rows_per_chunk]).reshape(-1, 1, d // 8, 8)
                g = (q * k[None]).max(axis=-1).sum(axis=-1)  # [rows, N_k]
                out[b, h, r0:r0 + rows_per_chunk] = g.max(axis=-1)
    return scale * 7.0 * 2.0 ** -13 * out


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def scale_for(d):
    return 1.0 / math.sqrt(d)
