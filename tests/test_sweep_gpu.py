"""GPU parity on seeded random shapes: forward, flash-decoding (two launches and one, over a
contiguous and over a paged cache), backward and the FP8 path against the fp64 oracle, element
by element.

The shapes are drawn once from a fixed seed and mix ragged lengths (values next to the
tile sizes 32, 64 and 128 are favoured), query/key length mismatches under the causal
mask, several query heads per key/value head, both head dimensions, and segment counts
up to one key per segment; they stay small enough for the oracle to finish in seconds.
"""
import os

import numpy as np
import pytest

import gen
import oracle
from parity_util import (bf16_dev_to_f64, check, check_grads, decode_inputs, fwd_inputs, o_rounding_allowance, say,
                         scale_for, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_59_amd")


def _length(rng, hi):
    """A length in [1, hi]: half the draws land within one of a multiple of 32."""
    if rng.random() < 0.5:
        base = 32 * int(rng.integers(1, max(2, hi // 32)))
        return int(min(hi, max(1, base + int(rng.integers(-1, 2)))))
    return int(rng.integers(1, hi + 1))


SEED = int(os.environ.get("FA_SWEEP_SEED", "59"))  # another seed draws another set of shapes


def _shapes():
    rng = np.random.default_rng(SEED)
    fwd, dec, bwd = [], [], []
    for _ in range(16):
        H_kv = int(rng.integers(1, 4))
        group = int(rng.choice([1, 2, 3, 4, 5, 8]))
        B = int(rng.integers(1, 3)) if H_kv * group > 6 else int(rng.integers(1, 4))
        fwd.append((B, H_kv * group, H_kv, _length(rng, 700), _length(rng, 700), int(rng.choice([64, 128])),
                    bool(rng.integers(0, 2))))
    for _ in range(10):
        H_kv = int(rng.integers(1, 4))
        group = int(rng.choice([1, 4, 7, 16, 20]))
        N_k = _length(rng, 3000)
        S = int(rng.integers(1, min(N_k, 100) + 1))
        dec.append((int(rng.integers(1, 3)), H_kv * group, H_kv, N_k, int(rng.choice([64, 128])), S))
    for _ in range(8):
        H_kv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 3]))
        bwd.append((int(rng.integers(1, 3)), H_kv * group, H_kv, _length(rng, 400), _length(rng, 400),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return fwd, dec, bwd


FWD, DEC, BWD = _shapes()


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()  # fail loudly if libfa.so is missing
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", FWD)
def test_sweep_fwd(orc, B, H, H_kv, N_q, N_k, d, causal):
    name = "sweep fwd%s" % str((B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    Q, K, V = fwd_inputs(5900 + N_q + 3 * N_k + d, B, H, H_kv, N_q, N_k, d)
    o, lse = fa.fwd(to_dev(Q), to_dev(K), to_dev(V), causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal)
    check(name, bf16_dev_to_f64(o), O_ref, lse.cpu().numpy(), L_ref)


@pytest.mark.parametrize("B,H,H_kv,N_k,d,S", DEC)
def test_sweep_decode(orc, B, H, H_kv, N_k, d, S):
    name = "sweep decode%s" % str((B, H, H_kv, N_k, d, S))
    say(name)
    Q, K, V = decode_inputs(5950 + N_k + S, B, H, H_kv, N_k, d)
    o_part, l_part = fa.decode_split(to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V), S)
    o, l = fa.combine(o_part, l_part)
    torch.cuda.synchronize()
    # every segment's partial (o_s, lse_s), then the merged output
    L = -(-N_k // S)
    op = o_part.cpu().numpy().astype(np.float64)
    lp = l_part.cpu().numpy().astype(np.float64)
    for t in range(S):
        lo, hi = min(t * L, N_k), min((t + 1) * L, N_k)
        O_s, L_s = orc.attention(Q, K, V, k_range=(lo, hi))
        check("%s segment %d" % (name, t), op[:, :, t], O_s[:, :, 0], lp[:, :, t], L_s[:, :, 0])
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name + " combined", bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", BWD)
def test_sweep_bwd(orc, B, H, H_kv, N_q, N_k, d, causal):
    name = "sweep bwd%s" % str((B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    scale = scale_for(d)
    seed = 5990 + N_q + 3 * N_k + d
    Q, K, V = fwd_inputs(seed, B, H, H_kv, N_q, N_k, d)
    dO = gen.normal_bf16(seed, gen.TENSOR_DO, (B, H, N_q, d))
    q, k, v, do = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = orc.attention_bwd(Q, K, V, dO, causal=causal, scale=scale)
    # The backward takes D = dO . O from the stored bf16 O; in rows that see one or two keys
    # its rounding is not small against the nearly cancelling gradient, so the gates are
    # applied after subtracting that first-order effect (o_rounding_allowance).
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, scale=scale)
    O_b = o.view(torch.int16).cpu().numpy().view(np.uint16)
    allow = o_rounding_allowance(Q, K, dO, O_ref, O_b, L_ref, scale, causal)
    check_grads(name, (bf16_dev_to_f64(dq), bf16_dev_to_f64(dk), bf16_dev_to_f64(dv)), (dQ, dK, dV), allow)
    if causal and N_q > N_k:  # rows that see no key get exactly zero
        assert np.all(bf16_dev_to_f64(dq)[:, :, :N_q - N_k] == 0.0), name


@pytest.fixture(scope="module")
def shared_counters():
    """One counter array for every one-launch decode below, sized for the largest shape: each
    completed call must leave it zero for the next."""
    n = max(fa.decode_counter_bytes(B, H, H_kv) for B, H, H_kv, _, _, _ in DEC) // 4
    return torch.zeros(n, dtype=torch.int32, device="cuda:0")


@pytest.mark.parametrize("B,H,H_kv,N_k,d,S", DEC)
def test_sweep_decode_one_launch(orc, shared_counters, B, H, H_kv, N_k, d, S):
    name = "sweep one-launch decode%s" % str((B, H, H_kv, N_k, d, S))
    say(name)
    Q, K, V = decode_inputs(5950 + N_k + S, B, H, H_kv, N_k, d)
    o, l = fa.decode(to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V), S, counters=shared_counters)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name, bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    assert int(shared_counters.abs().sum()) == 0, name + ": a group counter was left non-zero"


def _paged_shapes():
    rng = np.random.default_rng(SEED + 1000)
    out = []
    for _ in range(8):
        H_kv = int(rng.integers(1, 4))
        group = int(rng.choice([1, 2, 4, 7, 16, 20]))
        B = int(rng.integers(1, 4))
        lens = tuple(int(rng.integers(0, 1500)) if rng.random() < 0.8 else _length(rng, 1500) for _ in range(B))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        S = int(rng.integers(1, 40))
        out.append((B, H_kv * group, H_kv, lens, int(rng.choice([64, 128])), P, S))
    return out


PAGED = _paged_shapes()


@pytest.mark.parametrize("B,H,H_kv,lens,d,P,S", PAGED)
def test_sweep_paged(orc, B, H, H_kv, lens, d, P, S):
    """Paged flash-decoding (split + combine, and the one-launch form) over a shuffled pool
    whose unowned pages hold NaN, on random lengths (empty sequences included), page sizes
    and segment counts."""
    from test_paged_gpu import make_paged, reference

    name = "sweep paged%s" % str((B, H, H_kv, lens, d, P, S))
    say(name)
    N = max(1, max(lens))
    Q, K, V = decode_inputs(5900 + N + P + S, B, H, H_kv, N, d)
    Kp, Vp, table = make_paged(K, V, lens, P, seed=N + S + P)
    q, kp, vp = to_dev(Q[:, :, 0, :]), to_dev(Kp), to_dev(Vp)
    t = torch.from_numpy(table).cuda()
    ln = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o_part, l_part = fa.decode_split_paged(q, kp, vp, t, ln, S)
    o, l = fa.combine(o_part, l_part)
    o1, l1 = fa.decode_paged(q, kp, vp, t, ln, S)
    torch.cuda.synchronize()
    O_ref, L_ref = reference(orc, Q, K, V, lens)
    check(name, bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)
    check(name + " one launch", bf16_dev_to_f64(o1), O_ref, l1.cpu().numpy(), L_ref)


def _fp8_shapes():
    rng = np.random.default_rng(SEED + 2000)
    out = []
    for _ in range(6):
        H_kv = int(rng.integers(1, 3))
        group = int(rng.choice([1, 2, 4]))
        out.append((int(rng.integers(1, 3)), H_kv * group, H_kv, _length(rng, 600), _length(rng, 600),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2))))
    return out


FP8 = _fp8_shapes()


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", FP8)
def test_sweep_fp8(orc, B, H, H_kv, N_q, N_k, d, causal):
    """The FP8 path on random shapes: quantiser codes and scales bit for bit against the
    oracle's quantiser, the forward against the oracle on the dequantised and on the original
    tensors (the FP8 gates)."""
    from fp8_util import sign_mask
    from parity_util import check_fp8
    from test_fp8_gpu import quantize_both, run_fp8

    name = "sweep fp8%s" % str((B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    Q, K, V = fwd_inputs(5800 + N_q + 2 * N_k + d, B, H, H_kv, N_q, N_k, d)
    lo, hi = sign_mask(N_q + 5 * N_k)
    (q8, qs, k8, ks, v8, vs, pad), (oq, ok, ov), _ = quantize_both(orc, Q, K, V, lo, hi, True)
    assert np.array_equal(q8, oq[0]) and np.array_equal(qs.view(np.uint32), oq[1].view(np.uint32)), name + " Q"
    assert np.array_equal(k8, ok[0]) and np.array_equal(ks.view(np.uint32), ok[1].view(np.uint32)), name + " K"
    assert np.array_equal(v8, ov[0]) and np.array_equal(vs.view(np.uint32), ov[1].view(np.uint32)), name + " V"
    o, l, (qd, kd, vd) = run_fp8(orc, Q, K, V, causal, lo, hi)
    sc = scale_for(d)
    O_q, L_q = orc.attention(qd, kd, vd, causal=causal, scale=sc)
    O_x, L_x = orc.attention(Q, K, V, causal=causal, scale=sc)
    check_fp8(name, o, O_q, l, L_q, O_x, L_x)
