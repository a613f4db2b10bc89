"""GPU parity of the FP8 path (fa_fp8_quantize, fa_fwd_fp8).

The quantiser's output is integer data (e4m3 codes) decided by fp32 arithmetic, so it must
equal the oracle quantiser's bit for bit, scales included.  The forward is checked against
the fp64 oracle twice: on the dequantised tensors (what the kernel computes, up to the e4m3
rounding of P and fp32 accumulation) and on the original bf16 tensors (the whole FP8 error);
the gates are in parity_util (FP8_*).
"""
import math

import numpy as np
import pytest

import gen
import oracle
from fp8_util import dequantize, sign_mask, vt_to_logical
from parity_util import bf16_dev_to_f64, check_fp8, fwd_inputs, mfma_fp8_score_bound, say, scale_for, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_59_amd")


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def quantize_both(orc, Q, K, V, lo, hi, incoherent):
    """GPU quantiser outputs (as numpy, value tiles mapped back to logical order) and the
    oracle quantiser's."""
    d = Q.shape[-1]
    N_k = K.shape[2]
    g = fa.fp8_quantize(to_dev(Q), to_dev(K), to_dev(V), lo, hi, incoherent)
    torch.cuda.synchronize()
    q8, k8, vt8, qs, ks, vs = (t.cpu().numpy() for t in g)
    v8, pad = vt_to_logical(vt8, N_k)
    oq = orc.fp8_quantize(Q, 128, incoherent, lo, hi, 1.0 / d if incoherent else 1.0)
    ok = orc.fp8_quantize(K, 64, incoherent, lo, hi, 1.0)
    ov = orc.fp8_quantize(V, 64, False)
    return (q8, qs, k8, ks, v8, vs, pad), (oq, ok, ov), g


QUANT = [
    # B, H, H_kv, N_q, N_k, d, incoherent
    (1, 2, 1, 300, 190, 128, True),
    (2, 2, 2, 128, 64, 64, True),
    (1, 4, 2, 1000, 777, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (2, 4, 4, 129, 65, 128, False),
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,inc", QUANT)
def test_fp8_quantize_bit_exact(orc, B, H, H_kv, N_q, N_k, d, inc):
    name = "fp8 quantize %s" % str((B, H, H_kv, N_q, N_k, d, inc))
    say(name)
    Q, K, V = fwd_inputs(600 + N_q + d, B, H, H_kv, N_q, N_k, d)
    if N_q > 128:
        Q[0, 0, 128:256] = 0  # an all-zero query block: scale 0, codes 0
    lo, hi = sign_mask(N_q + N_k)
    (q8, qs, k8, ks, v8, vs, pad), (oq, ok, ov), _ = quantize_both(orc, Q, K, V, lo, hi, inc)
    assert np.array_equal(q8, oq[0]) and np.array_equal(qs.view(np.uint32), oq[1].view(np.uint32)), name + " Q"
    assert np.array_equal(k8, ok[0]) and np.array_equal(ks.view(np.uint32), ok[1].view(np.uint32)), name + " K"
    assert np.array_equal(v8, ov[0]) and np.array_equal(vs.view(np.uint32), ov[1].view(np.uint32)), name + " V"
    assert np.all(pad == 0), name + " value tile padding"
    if N_q > 128:
        assert qs[0, 0, 1] == 0.0 and np.all(q8[0, 0, 128:256] == 0)


def run_fp8(orc, Q, K, V, causal, lo, hi, inc=True):
    d = Q.shape[-1]
    _, (oq, ok, ov), g = quantize_both(orc, Q, K, V, lo, hi, inc)
    o, l = fa.fwd_fp8(*g, causal=causal, scale=scale_for(d))
    torch.cuda.synchronize()
    deq = (dequantize(orc, oq[0], oq[1], 128), dequantize(orc, ok[0], ok[1], 64), dequantize(orc, ov[0], ov[1], 64))
    return bf16_dev_to_f64(o), l.cpu().numpy(), deq


FWD = [
    # B, H, H_kv, N_q, N_k, d, causal
    (1, 2, 1, 300, 190, 128, True),
    (2, 4, 2, 256, 256, 64, False),
    (1, 2, 2, 1, 500, 128, False),
    (1, 4, 1, 257, 190, 128, True),   # N_q > N_k: leading rows see no key
    (1, 2, 2, 640, 1000, 64, True),
    (2, 2, 1, 1024, 1024, 128, False),
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", FWD)
def test_fp8_fwd(orc, B, H, H_kv, N_q, N_k, d, causal):
    name = "fp8 fwd %s" % str((B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    Q, K, V = fwd_inputs(700 + N_q + N_k + d, B, H, H_kv, N_q, N_k, d)
    lo, hi = sign_mask(N_k)
    o, l, (qd, kd, vd) = run_fp8(orc, Q, K, V, causal, lo, hi)
    sc = scale_for(d)
    O_q, L_q = orc.attention(qd, kd, vd, causal=causal, scale=sc)
    O_x, L_x = orc.attention(Q, K, V, causal=causal, scale=sc)
    check_fp8(name, o, O_q, l, L_q, O_x, L_x)


def test_fp8_incoherent_processing_lowers_error(orc):
    """Queries and keys with two outlier channels (x8): the random-sign Hadamard transform
    spreads them over all channels, so the scores' rounding error -- and the output's --
    drops (the pages report a lower FP8 error with incoherent processing)."""
    B, H, N, d = 1, 4, 512, 128
    say("fp8 incoherent processing, outlier channels")
    Q, K, V = fwd_inputs(811, B, H, H, N, N, d)
    for X in (Q, K):
        f = gen.bf16_to_f32(X)
        f[..., [5, 77]] *= 8.0
        X[...] = gen.f32_to_bf16(f)
    lo, hi = sign_mask(99)
    O_x, L_x = orc.attention(Q, K, V, scale=scale_for(d))
    errs = {}
    for inc in (True, False):
        o, l, (qd, kd, vd) = run_fp8(orc, Q, K, V, False, lo, hi, inc)
        O_q, L_q = orc.attention(qd, kd, vd, scale=scale_for(d))
        slack = mfma_fp8_score_bound(qd, kd, scale_for(d))
        check_fp8("fp8 outliers incoherent=%s" % inc, o, O_q, l, L_q, lse_slack=slack)
        errs[inc] = (np.abs(o - O_x).mean(), np.abs(l - L_x).mean())
    say("fp8 outliers: mean |O err| %.3e with transform, %.3e without; mean |LSE err| %.3e vs %.3e"
        % (errs[True][0], errs[False][0], errs[True][1], errs[False][1]))
    assert errs[True][0] < 0.6 * errs[False][0] and errs[True][1] < 0.6 * errs[False][1]


@pytest.mark.parametrize("B,H,H_kv,N,d,causal", [(16, 16, 16, 1024, 64, False), (16, 16, 16, 1024, 64, True),
                                                (2, 16, 16, 8192, 128, True), (4, 32, 8, 4095, 128, True)])
def test_fp8_fwd_workload_sampled(orc, B, H, H_kv, N, d, causal):
    """Full workload shapes (batched prefill, long causal, grouped heads with a ragged length)
    on sampled rows."""
    from parity_util import sample_rows

    name = "fp8 fwd B=%d H=%d/%d N=%d d=%d causal=%s (sampled rows)" % (B, H, H_kv, N, d, causal)
    say(name)
    Q, K, V = fwd_inputs(900 + d, B, H, H_kv, N, N, d)
    lo, hi = sign_mask(N)
    o, l, (qd, kd, vd) = run_fp8(orc, Q, K, V, causal, lo, hi)
    rows = sample_rows(B, H, N, 96, seed=N)
    O_q, L_q = orc.attention(qd, kd, vd, causal=causal, scale=scale_for(d), rows=rows)
    O_x, L_x = orc.attention(Q, K, V, causal=causal, scale=scale_for(d), rows=rows)
    check_fp8(name, o.reshape(-1, d)[rows], O_q, l.reshape(-1)[rows], L_q, O_x, L_x)


# ---------------------------------------------------------------------------- fp8 product truncation
def _e4m3_grid(e_lo, e_hi):
    """Positive normal e4m3 values (1 + m/8) * 2^e, e_lo <= e <= e_hi, up to the format's 448."""
    return [v for e in range(e_lo, e_hi + 1) for m in range(8) if (v := (1 + m / 8) * 2.0 ** e) <= 448.0]


def truncated_dot(q, k, group=8):
    """The fp8 matrix cores' dot product of e4m3 values, as measured through fa_fwd_fp8: in every
    group of `group` consecutive contraction slots (8 consecutive channels here), each product
    q_i k_i is truncated toward zero to a multiple of 2^(E - 13), where E is the largest sum
    exponent(q_i) + exponent(k_i) in the group (so a product loses less than 2^-13 times the
    group's largest product); the groups' sums are added exactly (fp32 is exact on these rows)."""
    from fractions import Fraction
    total = Fraction(0)
    for g0 in range(0, len(q), group):
        qs, ks = q[g0:g0 + group], k[g0:g0 + group]
        p = [Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qs, ks)]
        ex = [math.frexp(float(a))[1] + math.frexp(float(b))[1] - 2 for a, b in zip(qs, ks) if a != 0 and b != 0]
        if not ex:
            continue
        grid = Fraction(2) ** (max(ex) - 13)
        total += sum(int(x / grid) * grid for x in p)  # int() truncates toward zero
    return total


def truncation_rows(seed, H, d, big_e):
    """Per head one query and one key row of e4m3 values (bf16 bit patterns): in every group of
    8 channels one large product (factors with exponents big_e) and seven small ones (factors
    in [0.5, 8)), random signs; channel 0 holds +-448 in both rows, so that the quantiser's
    block scales are exactly 1 and the codes are the values themselves."""
    rng = np.random.default_rng(seed)
    small = _e4m3_grid(-1, 2)
    big = _e4m3_grid(big_e[0], big_e[1])
    Qf = np.zeros((H, d), dtype=np.float32)
    Kf = np.zeros((H, d), dtype=np.float32)
    for h in range(H):
        for g0 in range(0, d, 8):
            pos = g0 + int(rng.integers(8))
            for c in range(g0, g0 + 8):
                pool = big if c == pos else small
                Qf[h, c] = rng.choice(pool) * rng.choice([-1.0, 1.0])
                Kf[h, c] = rng.choice(pool) * rng.choice([-1.0, 1.0])
        Qf[h, 0], Kf[h, 0] = 448.0 * np.sign(Qf[h, 0] or 1.0), 448.0 * np.sign(Kf[h, 0] or 1.0)
    return gen.f32_to_bf16(Qf), gen.f32_to_bf16(Kf)


@pytest.mark.parametrize("big_e", [(8, 8), (7, 8), (4, 8)],
                         ids=["large factors 2^8", "large factors 2^7..2^8", "large factors 2^4..2^8"])
def test_fp8_matrix_core_product_truncation(big_e):
    """fa_fwd_fp8 with one query and one key per head returns LSE = scale * score, so the LSE
    exposes the fp8 matrix cores' dot product.  On operands whose codes are the values
    themselves (block scales 1, no transform), it equals the truncation model of
    truncated_dot to fp32 rounding, and differs from the exact dot product.  This is the model
    the LSE gate's allowance for the fp8 scores (parity_util.mfma_fp8_score_bound) rests on."""
    H, d = 32, 128
    say("fp8 product truncation, big factors 2^%d..2^%d" % big_e)
    Qb, Kb = truncation_rows(4242 + big_e[0], H, d, big_e)
    Q, K = Qb.reshape(1, H, 1, d), Kb.reshape(1, H, 1, d)
    V = gen.f32_to_bf16(np.ones((1, H, 1, d), dtype=np.float32))
    g = fa.fp8_quantize(to_dev(Q), to_dev(K), to_dev(V), 0, 0, False)
    o, l = fa.fwd_fp8(*g, causal=False, scale=scale_for(d))
    torch.cuda.synchronize()
    assert np.all(g[3].cpu().numpy() == 1.0) and np.all(g[4].cpu().numpy() == 1.0), "block scales must be 1"
    q8 = g[0].cpu().numpy().reshape(H, d)
    qv = gen.bf16_to_f32(Qb)
    lse = l.cpu().numpy().reshape(H).astype(np.float64)
    sc = scale_for(d)
    worst, apart = 0.0, 0
    for h in range(H):
        model = float(truncated_dot(gen.bf16_to_f32(Qb)[h], gen.bf16_to_f32(Kb)[h])) * sc
        exact = float(np.dot(qv[h].astype(np.float64), gen.bf16_to_f32(Kb)[h].astype(np.float64))) * sc
        err = abs(lse[h] - model)
        worst = max(worst, err / abs(model))
        assert err <= 1e-6 * abs(model), "head %d: LSE %.6f, truncation model %.6f, exact %.6f" % (h, lse[h], model, exact)
        apart += abs(exact - model) > 10 * 1e-6 * abs(model)
    # the exact dot product is clearly off on most heads: the case exercises the truncation
    assert apart >= H // 2, "only %d of %d heads tell the model from the exact product" % (apart, H)
    assert q8.any()
    say("fp8 product truncation: max relative |LSE - model| %.2e over %d heads" % (worst, H))
