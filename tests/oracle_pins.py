"""Pins of the fp64 oracle against facts the pages or the mathematics fix.

Every function takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees.  They are shared by ``test_oracle.py`` (the real oracle) and
``test_oracle_mutants.py`` (oracle builds with a planted mistake, each of
which must fail at least one pin).

None of these pins re-types the oracle's formula: each compares it with a
closed form, a worked example printed on the pages, exact high-precision
arithmetic, an independent library routine, or an invariant.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16_inputs(seed, B, H, H_kv, N_q, N_k, d, q_scale=1.0):
    Q = gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, N_q, d), q_scale)
    K = gen.normal_bf16(seed, gen.TENSOR_K, (B, H_kv, N_k, d))
    V = gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N_k, d))
    return Q, K, V


def _f64(x):
    return gen.bf16_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _visible(i, N_q, N_k, causal):
    """Number of visible keys of query i under bottom-right causal alignment."""
    if not causal:
        return N_k
    return max(0, min(N_k, i + N_k - N_q + 1))


# --------------------------------------------------------------------------- Algorithm 0
def pin_rows_sum_to_one(orc):
    """Each row of P is a probability vector over exactly the visible keys."""
    for causal in (False, True):
        Q, K, V = _bf16_inputs(11, 2, 4, 2, 33, 47, 16)
        O, LSE, P = orc.attention(Q, K, V, causal=causal, return_p=True)
        for i in range(33):
            n_vis = _visible(i, 33, 47, causal)
            row = P[:, :, i, :]
            assert np.all(row >= 0.0)
            assert np.all(row[..., n_vis:] == 0.0), "mass on a masked key"
            assert np.all(row[..., :n_vis] > 0.0)
            assert np.max(np.abs(row.sum(-1) - 1.0)) <= 1e-14


def pin_single_key(orc):
    """N_k = 1: the output is the value row itself and LSE is the one score."""
    B, H, H_kv, N_q, d = 2, 4, 2, 5, 8
    Q, K, V = _bf16_inputs(12, B, H, H_kv, N_q, 1, d)
    scale = 0.25
    O, LSE = orc.attention(Q, K, V, causal=False, scale=scale)
    Qf, Kf, Vf = _f64(Q), _f64(K), _f64(V)
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            assert np.array_equal(O[b, h], np.broadcast_to(Vf[b, g, 0], (N_q, d)))
            for i in range(N_q):
                s = Fraction(scale) * sum(Fraction(float(Qf[b, h, i, k])) * Fraction(float(Kf[b, g, 0, k]))
                                          for k in range(d))
                assert abs(LSE[b, h, i] - float(s)) <= 1e-15 * max(1.0, abs(float(s)))


def pin_equal_scores(orc):
    """Q = 0 makes every score 0: O is the mean of the visible V rows, LSE = ln(count)."""
    B, H, H_kv, N_q, N_k, d = 1, 2, 1, 7, 12, 8
    _, K, V = _bf16_inputs(13, B, H, H_kv, N_q, N_k, d)
    Q = np.zeros((B, H, N_q, d), dtype=np.uint16)
    Vf = _f64(V)
    for causal in (False, True):
        O, LSE = orc.attention(Q, K, V, causal=causal)
        for i in range(N_q):
            n = _visible(i, N_q, N_k, causal)
            want = Vf[0, 0, :n].mean(axis=0)
            assert np.max(np.abs(O[0, :, i] - want)) <= 1e-14
            assert np.all(np.abs(LSE[0, :, i] - math.log(n)) <= 1e-14)
    # all key rows equal (Q arbitrary): same mean, LSE = s + ln N_k
    Q2, K2, _ = _bf16_inputs(14, B, H, H_kv, N_q, N_k, d)
    K2[:] = K2[:, :, :1, :]
    O, LSE = orc.attention(Q2, K2, V, causal=False, scale=0.5)
    want = Vf[0, 0].mean(axis=0)
    Qf, Kf = _f64(Q2), _f64(K2)
    for h in range(H):
        for i in range(N_q):
            s = 0.5 * float(sum(Fraction(float(Qf[0, h, i, k])) * Fraction(float(Kf[0, 0, 0, k])) for k in range(d)))
            assert abs(LSE[0, h, i] - (s + math.log(N_k))) <= 1e-13
            assert np.max(np.abs(O[0, h, i] - want)) <= 1e-14


def pin_causal_first_row(orc):
    """Under the causal mask with N_q = N_k the first query sees only key 0: O_0 = V_0 exactly."""
    Q, K, V = _bf16_inputs(15, 2, 2, 2, 9, 9, 16)
    O, LSE = orc.attention(Q, K, V, causal=True, scale=0.125)
    Vf = _f64(V)
    assert np.array_equal(O[:, :, 0, :], Vf[:, :, 0, :])
    # bottom-right alignment with N_q < N_k: query 0 sees N_k - N_q + 1 keys
    Q2 = np.zeros((1, 1, 3, 16), dtype=np.uint16)
    O2, LSE2 = orc.attention(Q2, K[:1, :1], V[:1, :1], causal=True)
    for i in range(3):
        n = 9 - 3 + i + 1
        assert np.max(np.abs(O2[0, 0, i] - Vf[0, 0, :n].mean(axis=0))) <= 1e-14
        assert abs(LSE2[0, 0, i] - math.log(n)) <= 1e-14


def pin_fully_masked_rows(orc):
    """N_q > N_k under the causal mask: the first N_q - N_k queries see no key (O = 0, LSE = -inf)."""
    Q, K, V = _bf16_inputs(16, 1, 2, 1, 6, 4, 8)
    O, LSE = orc.attention(Q, K, V, causal=True)
    assert np.all(O[:, :, :2] == 0.0) and np.all(np.isneginf(LSE[:, :, :2]))
    assert np.all(np.isfinite(LSE[:, :, 2:]))
    assert np.array_equal(O[0, :, 2, :], np.broadcast_to(_f64(V)[0, 0, 0], (2, 8)))


def pin_large_scores(orc):
    """Lecture 11 section 3.4: subtracting the row maximum keeps exp finite for huge scores.
    Scores (0, 1000, 1): the softmax is one-hot on key 1 to double precision, LSE = 1000."""
    Q = np.ones((1, 1, 1, 1))
    K = np.array([0.0, 1000.0, 1.0]).reshape(1, 1, 3, 1)
    V = np.array([5.0, -2.0, 7.0]).reshape(1, 1, 3, 1)
    for perm in ([0, 1, 2], [1, 0, 2], [2, 0, 1]):
        O, L = orc.attention(Q, K[:, :, perm], V[:, :, perm], scale=1.0)
        assert O[0, 0, 0, 0] == -2.0 and L[0, 0, 0] == 1000.0


def pin_torch_sdpa(orc):
    """Agreement with torch's CPU scaled_dot_product_attention in float64 (an independent implementation)."""
    import torch

    for (B, H, H_kv, N, d, causal, scale) in [(2, 4, 4, 37, 16, False, None), (1, 4, 2, 50, 32, True, 0.3),
                                              (2, 8, 2, 20, 64, False, 0.125), (1, 2, 1, 64, 8, True, None)]:
        Q, K, V = _bf16_inputs(17 + N, B, H, H_kv, N, N, d)
        O, LSE = orc.attention(Q, K, V, causal=causal, scale=scale)
        sc = scale if scale is not None else 1.0 / math.sqrt(d)
        q, k, v = (torch.from_numpy(_f64(x)) for x in (Q, K, V))
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=sc,
                                                               enable_gqa=(H != H_kv))
        assert np.max(np.abs(O - ref.numpy())) <= 1e-12
        kk = k.repeat_interleave(H // H_kv, dim=1)
        logits = torch.matmul(q, kk.transpose(-1, -2).contiguous()) * sc
        if causal:
            mask = torch.ones(N, N, dtype=torch.bool).tril()
            logits = logits.masked_fill(~mask, float("-inf"))
        assert np.max(np.abs(LSE - torch.logsumexp(logits, dim=-1).numpy())) <= 1e-12


def pin_brute_force_decimal(orc):
    """Tiny inputs in exact rational scores and 40-digit decimal exp/log (N_k <= 3, d <= 2)."""
    getcontext().prec = 40
    rng = np.random.default_rng(5)
    for N_k in (1, 2, 3):
        for d in (1, 2):
            for causal in (False, True):
                N_q = 3
                Q = rng.integers(-8, 9, size=(1, 1, N_q, d)).astype(np.float64) / 4
                K = rng.integers(-8, 9, size=(1, 1, N_k, d)).astype(np.float64) / 4
                V = rng.integers(-8, 9, size=(1, 1, N_k, d)).astype(np.float64) / 8
                scale = 0.75
                O, LSE = orc.attention(Q, K, V, causal=causal, scale=scale)
                for i in range(N_q):
                    n = _visible(i, N_q, N_k, causal)
                    if n == 0:
                        assert np.all(O[0, 0, i] == 0) and LSE[0, 0, i] == -math.inf
                        continue
                    s = [Fraction(scale) * sum(Fraction(Q[0, 0, i, t]) * Fraction(K[0, 0, j, t]) for t in range(d))
                         for j in range(n)]
                    sd = [Decimal(x.numerator) / Decimal(x.denominator) for x in s]
                    e = [x.exp() for x in sd]
                    tot = sum(e)
                    for t in range(d):
                        o = sum(e[j] * Decimal(V[0, 0, j, t]) for j in range(n)) / tot
                        assert abs(O[0, 0, i, t] - float(o)) <= 1e-15
                    assert abs(LSE[0, 0, i] - float(tot.ln())) <= 1e-15


def pin_linearity_and_permutation(orc):
    """O is linear in V; without a mask, permuting (K, V) rows together changes nothing."""
    B, H, N_q, N_k, d = 1, 2, 10, 23, 8
    Q, K, V = _bf16_inputs(18, B, H, H, N_q, N_k, d)
    Qf, Kf, Vf = _f64(Q), _f64(K), _f64(V)
    V2 = _f64(gen.normal_bf16(19, gen.TENSOR_V, (B, H, N_k, d)))
    O1, L1 = orc.attention(Qf, Kf, Vf)
    O2, _ = orc.attention(Qf, Kf, V2)
    O3, L3 = orc.attention(Qf, Kf, 2.0 * Vf - 3.0 * V2)
    assert np.max(np.abs(O3 - (2.0 * O1 - 3.0 * O2))) <= 1e-13
    assert np.max(np.abs(L3 - L1)) == 0.0
    perm = np.random.default_rng(3).permutation(N_k)
    O4, L4 = orc.attention(Qf, Kf[:, :, perm], Vf[:, :, perm])
    assert np.max(np.abs(O4 - O1)) <= 1e-14 and np.max(np.abs(L4 - L1)) <= 1e-14


def pin_gqa(orc):
    """A query head reads the K/V head of its contiguous group: GQA equals MHA with K/V repeated."""
    B, H, H_kv, N, d = 2, 8, 2, 19, 16
    Q, K, V = _bf16_inputs(20, B, H, H_kv, N, N, d)
    for causal in (False, True):
        O, L = orc.attention(Q, K, V, causal=causal)
        Kr, Vr = np.repeat(K, H // H_kv, axis=1), np.repeat(V, H // H_kv, axis=1)
        O2, L2 = orc.attention(Q, Kr, Vr, causal=causal)
        assert np.array_equal(O, O2) and np.array_equal(L, L2)
        # a single head on its own, against the sliced K/V head
        h = 5
        O3, L3 = orc.attention(Q[:, h:h + 1], K[:, h // 4:h // 4 + 1], V[:, h // 4:h // 4 + 1], causal=causal)
        assert np.array_equal(O3[:, 0], O[:, h]) and np.array_equal(L3[:, 0], L[:, h])


def pin_row_selection(orc):
    """Computing a sampled list of rows gives the same values as the full computation."""
    B, H, H_kv, N, d = 2, 4, 2, 31, 16
    Q, K, V = _bf16_inputs(21, B, H, H_kv, N, N, d)
    O, L = orc.attention(Q, K, V, causal=True)
    rows = np.array([0, 5, 30, 31, 77, B * H * N - 1])
    Os, Ls = orc.attention(Q, K, V, causal=True, rows=rows)
    assert np.array_equal(Os, O.reshape(-1, d)[rows]) and np.array_equal(Ls, L.reshape(-1)[rows])


# --------------------------------------------------------------------------- online softmax
def pin_exercise1(orc):
    """Lecture 11, Exercise 1: blocks [1, 3] then [2, 5]."""
    with open(os.path.join(GOLDEN, "lecture11_ex1_online_softmax.json")) as f:
        g = json.load(f)
    s = np.array(g["blocks"][0] + g["blocks"][1], dtype=np.float64)
    r = orc.online_row(s, np.eye(4), block=2)
    tol = g["tolerance"]
    assert r["m_trace"][0] == g["after_block_1"]["m"] and abs(r["l_trace"][0] - g["after_block_1"]["l"]) <= tol
    assert r["m_trace"][1] == g["after_block_2"]["m"]
    assert abs(r["alpha_trace"][1] - g["after_block_2"]["alpha"]) <= tol
    assert abs(r["l_trace"][1] - g["after_block_2"]["l"]) <= tol
    assert abs(r["l"] - g["one_shot_l"]) <= tol
    # with identity value rows, o is the softmax of the row itself
    e = np.exp(s - s.max())
    assert np.max(np.abs(r["o"] - e / e.sum())) <= 1e-15


def pin_online_equals_full(orc):
    """One pass over blocks equals the full-row softmax times V (fp64, <= 1e-12), any block size."""
    rng = np.random.default_rng(7)
    n, d = 4096, 64
    for trial in range(3):
        q = rng.standard_normal(d)
        Kr = rng.standard_normal((n, d))
        Vr = rng.standard_normal((n, d))
        O, L = orc.attention(q.reshape(1, 1, 1, d), Kr.reshape(1, 1, n, d), Vr.reshape(1, 1, n, d), scale=0.5 + trial)
        s = (0.5 + trial) * (Kr @ q)
        for block in (1, 7, 256, n):
            r = orc.online_row(s, Vr, block)
            assert np.max(np.abs(r["o"] - O[0, 0, 0])) <= 1e-12
            assert abs((r["m"] + math.log(r["l"])) - L[0, 0, 0]) <= 1e-12


# --------------------------------------------------------------------------- merges
def _segment_state(orc, s, Vr, lo, hi):
    r = orc.online_row(s[lo:hi], Vr[lo:hi], max(1, hi - lo))
    return r["m"], r["l"], r["o"]


def pin_merge_orders(orc):
    """Lecture 11 section 3.2: a length-3000 row cut at random into 12 segments;
    sequential, tree and shuffled merges all equal the one-pass result."""
    rng = np.random.default_rng(9)
    n, d = 3000, 32
    for trial in range(3):
        s = 3.0 * rng.standard_normal(n)
        Vr = rng.standard_normal((n, d))
        full = orc.online_row(s, Vr, n)
        cuts = np.sort(rng.choice(np.arange(1, n), size=11, replace=False))
        bounds = [0, *cuts.tolist(), n]
        states = [_segment_state(orc, s, Vr, bounds[t], bounds[t + 1]) for t in range(12)]

        def check(st):
            m, l, o = st
            assert np.max(np.abs(o - full["o"])) <= 1e-12
            assert abs(m - full["m"]) == 0.0 and abs(l - full["l"]) <= 1e-12 * full["l"]

        acc = states[0]
        for st in states[1:]:
            acc = orc.merge(acc, st)
        check(acc)
        layer = list(states)
        while len(layer) > 1:
            layer = [orc.merge(layer[t], layer[t + 1]) if t + 1 < len(layer) else layer[t]
                     for t in range(0, len(layer), 2)]
        check(layer[0])
        order = rng.permutation(12)
        acc = states[order[0]]
        for t in order[1:]:
            acc = orc.merge(states[t], acc) if t % 2 else orc.merge(acc, states[t])
        check(acc)
        # an empty state is the identity
        empty = (-math.inf, 0.0, np.zeros(d))
        check(orc.merge(orc.merge(empty, acc), empty))


def pin_split_combine(orc):
    """Lecture 11 section 6.2: split into 1, 7, 64 or 1000 segments; the LSE combine equals direct."""
    B, H, H_kv, N_k, d = 1, 4, 2, 1000, 16
    Q, K, V = _bf16_inputs(22, B, H, H_kv, 1, N_k, d, q_scale=3.0)
    O, L = orc.attention(Q, K, V)
    for S in (1, 7, 64, 1000):
        seg = -(-N_k // S)
        lse_s = np.empty((H, S))
        o_s = np.empty((H, S, d))
        for t in range(S):
            lo, hi = min(t * seg, N_k), min((t + 1) * seg, N_k)
            Ot, Lt = orc.attention(Q, K, V, k_range=(lo, hi))
            lse_s[:, t], o_s[:, t] = Lt[0, :, 0], Ot[0, :, 0]
        for h in range(H):
            lse, o = orc.lse_combine(lse_s[h], o_s[h])
            assert np.max(np.abs(o - O[0, h, 0])) <= 1e-12
            assert abs(lse - L[0, h, 0]) <= 1e-12
        if S == 1:
            assert np.array_equal(o_s[:, 0], O[0, :, 0]) and np.array_equal(lse_s[:, 0], L[0, :, 0])
    # a segment past the end is empty (lse = -inf, o = 0) and contributes nothing
    Ot, Lt = orc.attention(Q, K, V, k_range=(N_k, N_k))
    assert np.all(Ot == 0) and np.all(np.isneginf(Lt))
    lse, o = orc.lse_combine(np.array([L[0, 0, 0], -math.inf]), np.stack([O[0, 0, 0], np.zeros(d)]))
    assert np.array_equal(o, O[0, 0, 0]) and lse == L[0, 0, 0]
    lse, o = orc.lse_combine(np.array([-math.inf, -math.inf]), np.ones((2, d)))
    assert lse == -math.inf and np.all(o == 0)


def pin_lse_matches_state(orc):
    """LSE of Algorithm 0 equals m + ln l of the one-pass state on the same scores."""
    Q, K, V = _bf16_inputs(23, 1, 1, 1, 4, 300, 32)
    O, L = orc.attention(Q, K, V, scale=0.2)
    Qf, Kf, Vf = _f64(Q), _f64(K), _f64(V)
    for i in range(4):
        s = 0.2 * (Kf[0, 0] @ Qf[0, 0, i])
        r = orc.online_row(s, Vf[0, 0], 64)
        assert abs(r["m"] + math.log(r["l"]) - L[0, 0, i]) <= 1e-12
        assert r["m"] == s.max()


# --------------------------------------------------------------------------- backward (section 5.1)
def _loss(orc, Q, K, V, dO, causal):
    O, _ = orc.attention(Q, K, V, causal=causal, nthreads=1)
    return float(np.sum(dO * O))


def pin_bwd_finite_differences(orc):
    """Every gradient equals the central difference of sum(dO * O) (fp64, h = 1e-5): with the
    causal mask, a query longer than the keys (bottom-right alignment) and two query heads
    sharing one key/value head.  Independent of the backward formulas: only the forward is used."""
    rng = np.random.default_rng(7)
    h = 1e-5
    for causal, (N_q, N_k) in ((False, (4, 6)), (True, (5, 4)), (True, (3, 6))):
        Q = rng.standard_normal((1, 2, N_q, 3))
        K = rng.standard_normal((1, 1, N_k, 3))
        V = rng.standard_normal((1, 1, N_k, 3))
        dO = rng.standard_normal((1, 2, N_q, 3))
        dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO, causal=causal, nthreads=1)
        for X, G in ((Q, dQ), (K, dK), (V, dV)):
            num = np.empty_like(X)
            for idx in np.ndindex(X.shape):
                keep = X[idx]
                X[idx] = keep + h
                up = _loss(orc, Q, K, V, dO, causal)
                X[idx] = keep - h
                down = _loss(orc, Q, K, V, dO, causal)
                X[idx] = keep
                num[idx] = (up - down) / (2 * h)
            assert np.max(np.abs(num - G)) <= 1e-7, (causal, N_q, N_k, np.max(np.abs(num - G)))


def pin_bwd_d_identity(orc):
    """Exercise 6 of Lecture 11: D_i = sum_j dP_ij P_ij equals dO_i . O_i."""
    Q, K, V = _bf16_inputs(21, 2, 4, 2, 37, 29, 16)
    dO = gen.normal_bf16(21, 3, (2, 4, 37, 16))
    for causal in (False, True):
        O, _ = orc.attention(Q, K, V, causal=causal)
        _, _, _, D = orc.attention_bwd(Q, K, V, dO, causal=causal)
        assert np.max(np.abs(D - np.sum(_f64(dO) * O, axis=-1))) <= 1e-12


def pin_bwd_single_key(orc):
    """One key: P = 1, so the scores do not matter (dQ = dK = 0) and dV is the sum of dO over
    the group's query heads and rows."""
    Q, K, V = _bf16_inputs(22, 2, 4, 2, 9, 1, 8)
    dO = gen.normal_bf16(22, 3, (2, 4, 9, 8))
    dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO)
    assert np.all(dQ == 0.0) and np.all(dK == 0.0)
    want = _f64(dO).reshape(2, 2, 2, 9, 8).sum(axis=(2, 3))  # heads (g, within-group), rows
    assert np.max(np.abs(dV[:, :, 0, :] - want)) <= 1e-12


# ---------------------------------------------------------------------------------- FP8 quantisation
def _torch_e4m3(x):
    """Independent encoder: torch's float32 -> float8_e4m3fn conversion (nearest-even)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def pin_e4m3_codec(orc):
    """The e4m3 encoder and decoder against torch's float8_e4m3fn: every code decodes to the
    same value and re-encodes to itself; midpoints between neighbours round to the even code;
    random values over the whole range (overflow beyond 464 included) encode identically."""
    import torch

    codes = np.arange(256, dtype=np.uint8)
    dec = orc.e4m3_decode(codes)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(dec), nan) and np.array_equal(dec[~nan], want[~nan])
    finite = dec[~nan].astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(finite), _torch_e4m3(finite))
    pos = np.unique(dec[(~nan) & (dec >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)  # exact halfway points (ties)
    mids = np.concatenate([mids, -mids, mids * np.float32(1 + 2 ** -20), mids * np.float32(1 - 2 ** -20)])
    assert np.array_equal(orc.e4m3_encode(mids), _torch_e4m3(mids))
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.uniform(-520, 520, 4000), rng.standard_normal(4000) * 2.0 ** rng.integers(-12, 9, 4000)])
    x = x.astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x), _torch_e4m3(x))


def _hadamard(d):
    from scipy.linalg import hadamard

    return hadamard(d).astype(np.int64)


def pin_fwht_exact(orc):
    """On integer rows the fp32 transform is exact and equals x @ H (scipy's Sylvester
    Hadamard matrix); applying it twice gives d * x (H H^T = d I)."""
    rng = np.random.default_rng(41)
    for d in (2, 8, 64, 128):
        x = rng.integers(-100, 101, size=(5, d))
        y = orc.fwht(x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), x @ _hadamard(d))
        assert np.array_equal(orc.fwht(y).astype(np.int64), d * x)


def _bf16_ints(rng, shape, lo=-8, hi=9):
    """Small integers as bf16 bits (exact)."""
    v = rng.integers(lo, hi, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16), v.astype(np.int64)


def pin_fp8_quantize_composition(orc):
    """Integer inputs, so the transform is exact: codes and scales equal the composition of
    independent pieces -- the random signs, scipy's Hadamard matrix, the block max, numpy
    float32 arithmetic for r = 448 / amax and x * r, torch's e4m3 encoder -- with the mask's
    high word acting on channels 64..127 and a ragged last block."""
    rng = np.random.default_rng(42)
    d, N, block = 128, 150, 64
    Xb, Xi = _bf16_ints(rng, (2, N, d))
    lo, hi = 0x9E3779B97F4A7C15, 0x0123456789ABCDEF
    signs = np.array([-1 if ((lo >> j) & 1 if j < 64 else (hi >> (j - 64)) & 1) else 1 for j in range(d)])
    for transform, post in ((True, 1.0 / d), (False, 1.0)):
        codes, scales = orc.fp8_quantize(Xb, block, transform, lo, hi, post)
        Y = (Xi * signs) @ _hadamard(d) if transform else Xi
        for h in range(2):
            for t in range(-(-N // block)):
                blk = Y[h, t * block:(t + 1) * block].astype(np.float32)  # exact (|y| < 2^24)
                amax = np.float32(np.abs(blk).max())
                r = np.float32(448.0) / amax
                assert np.array_equal(codes[h, t * block:(t + 1) * block], _torch_e4m3(blk * r))
                assert scales[h, t] == np.float32(amax / np.float32(448.0)) * np.float32(post)


def pin_fp8_block_edges(orc):
    """A block's largest element encodes to +-448 exactly; an all-zero block gives zero codes
    and scale 0; blocks are independent (quantising two blocks together equals quantising each)."""
    rng = np.random.default_rng(43)
    Xb = gen.normal_bf16(43, 0, (1, 96, 64))
    Xb[0, 32:64] = 0  # second block of 32 rows all zero
    codes, scales = orc.fp8_quantize(Xb, 32, True, 0x1234, 0, 1.0 / 64)
    assert np.all(codes[0, 32:64] == 0) and scales[0, 1] == 0.0
    for t in (0, 2):
        blk = codes[0, 32 * t:32 * t + 32]
        assert np.sum((blk & 0x7F) == 0x7E) >= 1 and np.all((blk & 0x7F) <= 0x7E)
    c0, s0 = orc.fp8_quantize(Xb[:, :32], 32, True, 0x1234, 0, 1.0 / 64)
    c2, s2 = orc.fp8_quantize(Xb[:, 64:], 32, True, 0x1234, 0, 1.0 / 64)
    assert np.array_equal(c0, codes[:, :32]) and np.array_equal(c2, codes[:, 64:])
    assert s0[0, 0] == scales[0, 0] and s2[0, 0] == scales[0, 2]
    del rng


def pin_fp8_scores_preserved(orc):
    """Dequantised transformed queries and keys reproduce the original scores q . k: the
    orthogonal transform cancels (H H^T = d I, the 1/d carried by the query scales), and the
    error stays within the bound that e4m3 rounding (at most 2^-4 relative, or half a
    subnormal step) of each factor allows."""
    B, H, N, d = 1, 2, 64, 128
    Q = gen.normal_bf16(44, 0, (B, H, N, d))
    K = gen.normal_bf16(44, 1, (B, H, N, d))
    lo, hi = 0xF0F0F0F0A5A5A5A5, 0x0F0F0F0F5A5A5A5A
    cq, sq = orc.fp8_quantize(Q, 32, True, lo, hi, 1.0 / d)
    ck, sk = orc.fp8_quantize(K, 32, True, lo, hi, 1.0)
    qd = orc.e4m3_decode(cq) * np.repeat(sq.astype(np.float64), 32, axis=-1)[..., None]
    kd = orc.e4m3_decode(ck) * np.repeat(sk.astype(np.float64), 32, axis=-1)[..., None]
    signs = np.array([-1.0 if ((lo >> j) & 1 if j < 64 else (hi >> (j - 64)) & 1) else 1.0 for j in range(d)])
    Hm = _hadamard(d).astype(np.float64)
    qt, kt = (_f64(Q) * signs) @ Hm / d, (_f64(K) * signs) @ Hm  # exact transformed rows
    s_true = _f64(Q) @ np.swapaxes(_f64(K), -1, -2)
    s_deq = qd @ np.swapaxes(kd, -1, -2)
    eq, ek = np.abs(qd - qt), np.abs(kd - kt)
    # per-element rounding bound, then the product bound |dq||k| + |q||dk| + |dq||dk|
    sub_q = np.repeat(sq.astype(np.float64), 32, axis=-1)[..., None] * 2.0 ** -10
    sub_k = np.repeat(sk.astype(np.float64), 32, axis=-1)[..., None] * 2.0 ** -10
    assert np.all(eq <= 2.0 ** -4 * np.abs(qt) + sub_q * (1 + 1e-9))
    assert np.all(ek <= 2.0 ** -4 * np.abs(kt) + sub_k * (1 + 1e-9))
    bound = eq @ np.swapaxes(np.abs(kt), -1, -2) + np.abs(qt) @ np.swapaxes(ek, -1, -2) + eq @ np.swapaxes(ek, -1, -2)
    assert np.all(np.abs(s_deq - s_true) <= bound * (1 + 1e-9) + 1e-12)
    assert np.max(np.abs(s_deq - s_true)) < 0.1 * np.max(np.abs(s_true))


ALL_PINS = [pin_rows_sum_to_one, pin_single_key, pin_equal_scores, pin_causal_first_row,
            pin_fully_masked_rows, pin_large_scores, pin_torch_sdpa, pin_brute_force_decimal, pin_linearity_and_permutation,
            pin_gqa, pin_row_selection, pin_exercise1, pin_online_equals_full, pin_merge_orders,
            pin_split_combine, pin_lse_matches_state, pin_bwd_finite_differences, pin_bwd_d_identity,
            pin_bwd_single_key, pin_e4m3_codec, pin_fwht_exact, pin_fp8_quantize_composition,
            pin_fp8_block_edges, pin_fp8_scores_preserved]
