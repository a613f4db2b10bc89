"""GPU parity of the FlashAttention backward (fa_bwd) against the fp64 oracle.

As in a training step, the GPU forward supplies O and LSE; the oracle computes the exact
gradients of sum(dO * O) from the same bf16 Q, K, V and dO.  The gates (derived from the
bf16 rounding of P, dS, O and the outputs) are in parity_util.check_grads.
"""
import numpy as np
import pytest

import gen
import oracle
from parity_util import (bf16_dev_to_f64, check_grads, fwd_inputs, o_rounding_allowance, say, scale_for,
                         stress_inputs, to_dev)

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


def run(Q, K, V, dO, causal, scale):
    q, k, v, do = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def case(seed, B, H, H_kv, N_q, N_k, d, causal):
    Q, K, V = fwd_inputs(seed, B, H, H_kv, N_q, N_k, d)
    dO = gen.normal_bf16(seed, gen.TENSOR_DO, (B, H, N_q, d))
    return Q, K, V, dO


SMALL = [
    # B, H, H_kv, N_q, N_k, d, causal
    (1, 2, 2, 128, 128, 64, False),
    (1, 2, 2, 128, 128, 128, False),
    (2, 4, 2, 200, 333, 64, True),       # ragged, grouped heads, bottom-right mask
    (1, 4, 1, 257, 190, 128, True),      # N_q > N_k: leading rows see no key (dQ = 0)
    (1, 2, 1, 300, 513, 128, False),
    (2, 2, 2, 77, 77, 64, True),
    (1, 1, 1, 1, 1, 64, False),          # one query, one key: P = 1, dQ = dK = 0, dV = dO
    (1, 3, 3, 1, 300, 128, True),        # a single query row sees every key
    (1, 8, 1, 33, 700, 64, False),       # eight query heads summed into one dK/dV
    (1, 2, 2, 640, 96, 64, True),
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", SMALL)
def test_bwd_small(orc, B, H, H_kv, N_q, N_k, d, causal):
    name = "bwd%s" % str((B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    scale = scale_for(d)
    Q, K, V, dO = case(11 + N_q + N_k + d, B, H, H_kv, N_q, N_k, d, causal)
    dq, dk, dv = run(Q, K, V, dO, causal, scale)
    dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO, causal=causal, scale=scale)
    check_grads(name, (bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)), (dQ, dK, dV))
    if causal and N_q > N_k:  # rows that see no key get exactly zero
        assert np.all(bf16_dev_to_f64(dq)[:, :, :N_q - N_k] == 0.0), name


@pytest.mark.parametrize("pattern", ["ramp_up", "alternating"])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_bwd_score_range_stress(orc, pattern, d, causal):
    """P recomputed from the saved LSE when scores span tens of units (peaked rows).

    The backward is fed the oracle's O (rounded to bf16, as a forward stores it) and LSE, so
    that the allowance for O's rounding (o_rounding_allowance) is computed from oracle values
    only; the gates then bound the backward's own arithmetic."""
    B, H, H_kv, N_q, N_k = 1, 4, 2, 300, 520
    name = "bwd stress %s d=%d causal=%s" % (pattern, d, causal)
    say(name)
    scale = scale_for(d)
    Q, K, V = stress_inputs(900 + d, B, H, H_kv, N_q, N_k, d, pattern)
    dO = gen.normal_bf16(900 + d, gen.TENSOR_DO, (B, H, N_q, d))
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, scale=scale)
    O_b = gen.f32_to_bf16(O_ref.astype(np.float32))
    q, k, v, do, o = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO), to_dev(O_b)
    lse = torch.from_numpy(L_ref.astype(np.float32)).to("cuda:0")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO, causal=causal, scale=scale)
    allow = o_rounding_allowance(Q, K, dO, O_ref, O_b, L_ref, scale, causal)
    check_grads(name, (bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)), (dQ, dK, dV), allow)


def test_bwd_is_deterministic():
    """Each gradient row has one writer: two calls agree bit for bit."""
    B, H, H_kv, N, d = 2, 4, 2, 384, 128
    say("bwd determinism", (B, H, H_kv, N, d))
    Q, K, V, dO = case(5, B, H, H_kv, N, N, d, True)
    a = run(Q, K, V, dO, True, scale_for(d))
    b = run(Q, K, V, dO, True, scale_for(d))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("d,causal", [(64, False), (64, True), (128, False), (128, True)])
def test_bwd_training_shape_sampled(orc, d, causal):
    """B=16, H=16, N=1024 (the prefill workload) checked on four whole (b, h) slices: a
    slice's gradients depend on that slice only, so the oracle runs on the slices alone."""
    B, H, N = 16, 16, 1024
    name = "bwd B=16 H=16 N=1024 d=%d causal=%s" % (d, causal)
    say(name)
    scale = scale_for(d)
    Q, K, V, dO = case(23, B, H, H, N, N, d, causal)
    dq, dk, dv = run(Q, K, V, dO, causal, scale)
    dq, dk, dv = bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)
    for b, h in ((0, 0), (3, 15), (9, 7), (15, 8)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        dQ, dK, dV, _ = orc.attention_bwd(Q[sl], K[sl], V[sl], dO[sl], causal=causal, scale=scale)
        check_grads("%s slice b=%d h=%d" % (name, b, h), (dq[sl], dk[sl], dv[sl]), (dQ, dK, dV))


def test_bwd_gqa_ragged_sampled(orc):
    """B=4, H=32 query heads over H_kv=8 key/value heads, N=4095 (a ragged last tile), d=128,
    causal, checked on whole key/value groups: a group's gradients (its four query heads' dQ,
    its dK and dV) depend on that group only, so the oracle runs on the group alone."""
    B, H, H_kv, N, d = 4, 32, 8, 4095, 128
    name = "bwd GQA ragged B=4 H=32/8 N=4095 d=128 causal"
    say(name)
    scale = scale_for(d)
    Q, K, V, dO = case(29, B, H, H_kv, N, N, d, True)
    dq, dk, dv = run(Q, K, V, dO, True, scale)
    dq, dk, dv = bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)
    G = H // H_kv
    for b, g in ((0, 0), (3, 5)):
        qs, ks = (slice(b, b + 1), slice(g * G, g * G + G)), (slice(b, b + 1), slice(g, g + 1))
        dQ, dK, dV, _ = orc.attention_bwd(Q[qs], K[ks], V[ks], dO[qs], causal=True, scale=scale)
        check_grads("%s group b=%d g=%d" % (name, b, g), (dq[qs], dk[ks], dv[ks]), (dQ, dK, dV))


@pytest.mark.parametrize("scale", [0.02, 0.5])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_bwd_scale_range(orc, scale, d, causal):
    """Gradients at a nearly flat (0.02) and a peaked (0.5: scores of a row span tens of units)
    softmax scale, fed the oracle's O (as bf16) and LSE, with the O-rounding allowance."""
    B, H, H_kv, N_q, N_k = 1, 4, 2, 200, 333
    name = "bwd scale %g d=%d causal=%s" % (scale, d, causal)
    say(name)
    Q, K, V = fwd_inputs(950 + d, B, H, H_kv, N_q, N_k, d)
    dO = gen.normal_bf16(950 + d, gen.TENSOR_DO, (B, H, N_q, d))
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, scale=scale)
    O_b = gen.f32_to_bf16(O_ref.astype(np.float32))
    q, k, v, do, o = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO), to_dev(O_b)
    lse = torch.from_numpy(L_ref.astype(np.float32)).to("cuda:0")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO, causal=causal, scale=scale)
    allow = o_rounding_allowance(Q, K, dO, O_ref, O_b, L_ref, scale, causal)
    check_grads(name, (bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)), (dQ, dK, dV), allow)
