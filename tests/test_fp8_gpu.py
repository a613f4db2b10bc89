"""GPU parity of the FP8 path (fa_fp8_quantize, fa_fwd_fp8).

The quantiser's output is integer data (e4m3 codes) decided by fp32 arithmetic, so it must
equal the oracle quantiser's bit for bit, scales included.  The forward is checked against
the fp64 oracle twice: on the dequantised tensors (what the kernel computes, up to the e4m3
rounding of P and fp32 accumulation) and on the original bf16 tensors (the whole FP8 error);
the gates are in parity_util (FP8_*).
"""
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


@pytest.mark.parametrize("B,H,H_kv,N,d,causal", [(16, 16, 16, 1024, 64, False), (2, 16, 16, 8192, 128, True),
                                                (4, 32, 8, 4095, 128, True)])
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
