"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes are compared element by element over every output; the full-size
workloads (launched exactly as the benchmark launches them) are compared on sampled
rows that the oracle computes one by one, plus properties that hold for every row.
"""
import math

import numpy as np
import pytest

import oracle
from parity_util import (bf16_dev_to_f64, check, decode_inputs, fwd_inputs, key_scale, sample_rows, say,
                         scale_for, stress_inputs, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_59_amd")


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


def run_fwd(Q, K, V, causal, scale=None):
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------------------- forward, small shapes
SMALL = [
    # B, H, H_kv, N_q, N_k, d, causal
    (1, 1, 1, 256, 256, 64, False),
    (2, 4, 4, 300, 300, 64, True),
    (1, 4, 2, 513, 513, 128, True),
    (2, 2, 1, 200, 333, 128, False),
    (1, 2, 2, 333, 200, 64, True),     # N_q > N_k: leading rows see no key
    (1, 2, 2, 200, 333, 128, True),    # N_q < N_k: bottom-right alignment
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 1, 1, 1000, 128, True),     # one query sees every key
    (1, 2, 1, 2, 2, 128, True),
    (3, 2, 2, 63, 63, 128, True),
    (1, 2, 1, 64, 64, 64, True),
    (1, 2, 1, 65, 65, 64, True),
    (1, 2, 2, 127, 129, 128, False),
    (1, 2, 2, 129, 127, 64, True),
    (1, 1, 1, 1000, 64, 128, False),
    (2, 8, 1, 130, 70, 64, False),
]


@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", SMALL)
def test_fwd_small(orc, B, H, H_kv, N_q, N_k, d, causal):
    say("fwd small", B, H, H_kv, N_q, N_k, d, causal)
    Q, K, V = fwd_inputs(1000 + N_q + 7 * N_k + d, B, H, H_kv, N_q, N_k, d)
    o, lse = run_fwd(Q, K, V, causal)
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal)
    check("fwd%s" % str((B, H, H_kv, N_q, N_k, d, causal)), bf16_dev_to_f64(o), O_ref, lse.cpu().numpy(), L_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_exact_cases(orc, d):
    # N_k = 1: O is the value row (bit-exact after bf16 rounding); LSE is the score.
    say("fwd exact cases d=%d" % d)
    Q, K, V = fwd_inputs(31, 2, 4, 2, 70, 1, d)
    o, lse = run_fwd(Q, K, V, False)
    Vd = to_dev(V)
    want = Vd[:, [0, 0, 1, 1]].expand(2, 4, 70, d)
    assert torch.equal(o, want)
    _, L_ref = orc.attention(Q, K, V)
    assert np.max(np.abs(lse.cpu().numpy() - L_ref)) <= 1e-3
    # causal first row: O_0 = V_0 exactly
    Q, K, V = fwd_inputs(32, 2, 2, 2, 150, 150, d)
    o, lse = run_fwd(Q, K, V, True)
    assert torch.equal(o[:, :, 0], to_dev(V)[:, :, 0])
    # Q = 0: every score is 0, O = mean of V rows (bf16 rounding), LSE = ln N_k
    Q = np.zeros_like(Q)
    o, lse = run_fwd(Q, K, V, False)
    O_ref, L_ref = orc.attention(Q, K, V)
    check("fwd Q=0 d=%d" % d, bf16_dev_to_f64(o), O_ref, lse.cpu().numpy(), L_ref)
    assert np.max(np.abs(lse.cpu().numpy() - math.log(150))) <= 1e-5


STRESS = [
    # B, H, H_kv, N_q, N_k, d, causal
    (1, 4, 2, 300, 700, 64, False),
    (1, 4, 2, 300, 700, 64, True),
    (2, 2, 1, 257, 513, 128, True),
    (1, 2, 2, 200, 1000, 128, False),
]


@pytest.mark.parametrize("pattern", ["ramp_up", "ramp_down", "alternating"])
@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", STRESS)
def test_fwd_score_range_stress(orc, pattern, B, H, H_kv, N_q, N_k, d, causal):
    """Scores spanning tens of units whose row maximum jumps many times along the keys (the
    running max and the rescale of acc and l, including factors that underflow to zero),
    never moves after the first keys, or alternates between key blocks."""
    name = "fwd stress %s %s" % (pattern, str((B, H, H_kv, N_q, N_k, d, causal)))
    say(name)
    Q, K, V = stress_inputs(500 + N_k + d, B, H, H_kv, N_q, N_k, d, pattern)
    o, lse = run_fwd(Q, K, V, causal)
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal)
    # the inputs do stress the range: scaled scores of a row spread over more than 8 log2 units
    spread = (L_ref.max() - L_ref.min()) / math.log(2)
    assert spread > 8.0, spread
    check(name, bf16_dev_to_f64(o), O_ref, lse.cpu().numpy(), L_ref)


def test_fwd_scale_and_determinism(orc):
    say("fwd scale/determinism")
    Q, K, V = fwd_inputs(33, 2, 4, 2, 257, 257, 128)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o1, l1 = fa.fwd(q, k, v, causal=True, scale=0.3)
    o2, l2 = fa.fwd(q, k, v, causal=True, scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    O_ref, L_ref = orc.attention(Q, K, V, causal=True, scale=0.3)
    check("fwd scale=0.3", bf16_dev_to_f64(o1), O_ref, l1.cpu().numpy(), L_ref)


def test_fwd_on_side_stream(orc):
    say("fwd on a side stream")
    Q, K, V = fwd_inputs(34, 1, 2, 2, 200, 200, 64)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, l = fa.fwd(q, k, v, causal=True)
    s.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V, causal=True)
    check("fwd side stream", bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)


def test_fwd_rejects_bad_input():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fwd(q, q, q)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    q = torch.zeros(1, 3, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.fwd(q, k, k)
    assert e.value.status == fa.FA_ERR_SHAPE
    with pytest.raises(ValueError):
        fa.fwd(q.cpu(), k.cpu(), k.cpu())


# ---------------------------------------------------------------------------- forward, full workloads
FULL = [
    # name, seed, B, H, H_kv, N, d, causal, random sampled rows
    ("single-head N=256 d=64 (fp32 draw)", 1, 1, 1, 1, 256, 64, False, 0),
    ("batched prefill 16x16 N=1024 d=64", 2, 16, 16, 16, 1024, 64, False, 1024),
    ("batched prefill 16x16 N=1024 d=64 causal", 2, 16, 16, 16, 1024, 64, True, 1024),
    ("batched prefill 16x16 N=1024 d=128", 2, 16, 16, 16, 1024, 128, False, 1024),
    ("long causal 2x16 N=8192 d=128", 3, 2, 16, 16, 8192, 128, True, 512),
    ("GQA ragged 4x32/8 N=4095 d=128 causal", 4, 4, 32, 8, 4095, 128, True, 512),
]


@pytest.mark.parametrize("name,seed,B,H,H_kv,N,d,causal,n_rand", FULL, ids=[f[0] for f in FULL])
def test_fwd_full_workloads(orc, name, seed, B, H, H_kv, N, d, causal, n_rand):
    say("fwd full", name)
    f32_draw = B * H * N <= 4096
    ins = fwd_inputs(seed, B, H, H_kv, N, N, d, f32_draw=f32_draw)
    Q, K, V = ins[:3]
    o, lse = run_fwd(Q, K, V, causal)
    O_gpu = bf16_dev_to_f64(o)
    L_gpu = lse.cpu().numpy().astype(np.float64)
    # properties of every row: finite, convex combination of V rows, causal row 0 = V_0
    assert np.all(np.isfinite(O_gpu)) and np.all(np.isfinite(L_gpu))
    vmax = float(to_dev(V).abs().max().float())
    assert np.abs(O_gpu).max() <= vmax * (1 + 2 ** -7)
    if causal:
        g = torch.arange(H, device="cuda") // (H // H_kv)
        assert torch.equal(o[:, :, 0], to_dev(V)[:, g, 0])
    if B * H * N <= 4096:
        O_ref, L_ref = orc.attention(Q, K, V, causal=causal)
        check(name, O_gpu, O_ref, L_gpu, L_ref)
        raw = ins[3]
        O_raw, L_raw = orc.attention(*raw, causal=causal)
        say(name, "error vs oracle on the unrounded fp32 draws (reported, not gated):",
            float(np.abs(O_gpu - O_raw).max()), float(np.abs(L_gpu - L_raw).max()))
        return
    rows = sample_rows(B, H, N, n_rand, seed)
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, rows=rows)
    check(name + " (%d sampled rows)" % rows.size, O_gpu.reshape(-1, d)[rows], O_ref, L_gpu.reshape(-1)[rows],
          L_ref)


# ---------------------------------------------------------------------------- decode
def run_decode(Q, K, V, S):
    q = to_dev(Q[:, :, 0, :])
    k, v = to_dev(K), to_dev(V)
    o_part, l_part = fa.decode_split(q, k, v, S)
    o, l = fa.combine(o_part, l_part)
    torch.cuda.synchronize()
    return o_part, l_part, o, l


def check_segments(orc, name, Q, K, V, S, o_part, l_part, heads=None):
    B, H = Q.shape[:2]
    N_k, d = K.shape[2], K.shape[3]
    L = -(-N_k // S)
    op = o_part.cpu().numpy().astype(np.float64)
    lp = l_part.cpu().numpy().astype(np.float64)
    segs = range(S) if S <= 80 else sorted({0, 1, S // 2, S - 2, S - 1})
    for t in segs:
        lo, hi = min(t * L, N_k), min((t + 1) * L, N_k)
        O_ref, L_ref = orc.attention(Q, K, V, k_range=(lo, hi))
        check("%s segment %d/%d" % (name, t, S), op[:, :, t], O_ref[:, :, 0], lp[:, :, t], L_ref[:, :, 0])


DECODE = [
    # B, H, H_kv, N_k, d, S
    (1, 4, 1, 100, 128, 1),
    (2, 8, 2, 1000, 128, 7),
    (2, 8, 2, 1000, 64, 64),
    (1, 4, 4, 333, 64, 333),     # one key per segment
    (1, 2, 1, 100, 128, 60),     # L = 2: trailing segments are empty
    (2, 20, 1, 515, 128, 5),     # 20 query heads per K/V head: two head chunks
    (1, 16, 1, 64, 64, 3),
    (3, 6, 3, 37, 128, 2),
    (1, 64, 1, 300, 128, 3),     # the largest group (64 query heads per K/V head): four head chunks
    (2, 128, 2, 257, 64, 4),
]


@pytest.mark.parametrize("B,H,H_kv,N_k,d,S", DECODE)
def test_decode_small(orc, B, H, H_kv, N_k, d, S):
    name = "decode%s" % str((B, H, H_kv, N_k, d, S))
    say(name)
    Q, K, V = decode_inputs(2000 + N_k + S, B, H, H_kv, N_k, d)
    o_part, l_part, o, l = run_decode(Q, K, V, S)
    check_segments(orc, name, Q, K, V, S, o_part, l_part)
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name + " combined", bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])


@pytest.mark.parametrize("pattern", ["ramp_up", "ramp_down", "alternating"])
@pytest.mark.parametrize("B,H,H_kv,N_k,d,S", [(2, 8, 2, 3000, 128, 7), (1, 4, 1, 1500, 64, 24)])
def test_decode_score_range_stress(orc, pattern, B, H, H_kv, N_k, d, S):
    """Segments whose log-sum-exps differ by tens of units: the merge weights e^(lse_s - lse)
    span many orders of magnitude (ramp_up: the last segment dominates; ramp_down: the first)."""
    name = "decode stress %s %s" % (pattern, str((B, H, H_kv, N_k, d, S)))
    say(name)
    Q, K, V = stress_inputs(3000 + N_k + S, B, H, H_kv, 1, N_k, d, pattern)
    o_part, l_part, o, l = run_decode(Q, K, V, S)
    check_segments(orc, name, Q, K, V, S, o_part, l_part)
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name + " combined", bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    lp = l_part.cpu().numpy()
    assert float((lp.max(-1) - lp.min(-1)).max()) > 10.0  # the segments' LSEs do spread


@pytest.mark.parametrize("N_k,seed", [(4096, 5), (65536, 6)])
def test_decode_full_workloads(orc, N_k, seed):
    B, H, H_kv, d = 4, 32, 8, 128
    S = fa.decode_num_splits(B, H_kv, N_k, d)
    name = "flash-decoding B=4 H=32/8 N_k=%d d=128 S=%d" % (N_k, S)
    say(name)
    Q, K, V = decode_inputs(seed, B, H, H_kv, N_k, d)
    o_part, l_part, o, l = run_decode(Q, K, V, S)
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name, bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    if N_k <= 4096:
        check_segments(orc, name, Q, K, V, S, o_part, l_part)
    for S2 in (1, 64):
        o_part, l_part, o, l = run_decode(Q, K, V, S2)
        check(name.replace("S=%d" % S, "S=%d" % S2), bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(),
              L_ref[:, :, 0])


@pytest.mark.parametrize("S,d", [(9, 128), (9, 64), (1, 128), (32, 128), (33, 128), (64, 64), (100, 128)])
def test_combine_synthetic_partials(orc, S, d):
    """fa_combine alone on seeded partials, including segments with lse = -inf, at both head
    dimensions and segment counts from 1 to more than one 64-lane pass."""
    import gen

    say("combine synthetic S=%d d=%d" % (S, d))
    B, H = 2, 3
    o_s = gen.normal_f32(41, 0, (B, H, S, d))
    lse_s = gen.normal_f32(41, 1, (B, H, S), scale=4.0)
    lse_s[0, 0, [t for t in (1, 4) if t < S]] = -np.inf
    lse_s[1, 2, :] = -np.inf   # every segment empty
    o_s[1, 2] = 0.0
    o, l = fa.combine(torch.from_numpy(o_s).cuda(), torch.from_numpy(lse_s).cuda())
    torch.cuda.synchronize()
    O_ref = np.empty((B, H, d))
    L_ref = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            L_ref[b, h], O_ref[b, h] = orc.lse_combine(lse_s[b, h].astype(np.float64), o_s[b, h].astype(np.float64))
    check("combine synthetic S=%d d=%d" % (S, d), bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)
    assert np.all(bf16_dev_to_f64(o)[1, 2] == 0.0)


@pytest.mark.parametrize("scale", [1e-3, 0.05, 1.0, 4.0])
@pytest.mark.parametrize("d,causal", [(64, True), (128, False)])
def test_fwd_and_decode_scale_range(orc, scale, d, causal):
    """Softmax scales from nearly uniform (1e-3) to sharply peaked (4.0: scores span hundreds of
    units, the running max moves on most tiles) in the forward and in flash-decoding."""
    B, H, H_kv, N = 1, 4, 2, 333
    name = "scale %g d=%d causal=%s" % (scale, d, causal)
    say(name)
    Q, K, V = fwd_inputs(4400 + d, B, H, H_kv, N, N, d)
    o, l = run_fwd(Q, K, V, causal, scale=scale)
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, scale=scale)
    check("fwd " + name, bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)
    q = to_dev(Q[:, :, :1, :])
    o_part, l_part = fa.decode_split(q[:, :, 0, :], to_dev(K), to_dev(V), 5, scale=scale)
    od, ld = fa.combine(o_part, l_part)
    o1, l1 = fa.decode(q[:, :, 0, :], to_dev(K), to_dev(V), 5, scale=scale)
    torch.cuda.synchronize()
    O_d, L_d = orc.attention(Q[:, :, :1], K, V, scale=scale)
    check("decode " + name, bf16_dev_to_f64(od), O_d[:, :, 0], ld.cpu().numpy(), L_d[:, :, 0])
    check("one-launch decode " + name, bf16_dev_to_f64(o1), O_d[:, :, 0], l1.cpu().numpy(), L_d[:, :, 0])


def test_fwd_long_sequence_sampled(orc):
    """N_q = N_k = 32768 causal (256 query tiles per head, 512 key tiles): sampled rows against
    the oracle, including the last rows, which see every key."""
    B, H, H_kv, N, d = 1, 2, 1, 32768, 128
    name = "fwd long sequence N=%d" % N
    say(name)
    Q, K, V = fwd_inputs(4500, B, H, H_kv, N, N, d)
    o, lse = run_fwd(Q, K, V, True)
    rows = np.unique(np.concatenate([sample_rows(B, H, N, 48, 4500), [N - 1, 2 * N - 1, N // 2]]))
    O_ref, L_ref = orc.attention(Q, K, V, causal=True, rows=rows)
    check(name + " (%d sampled rows)" % rows.size, bf16_dev_to_f64(o).reshape(-1, d)[rows], O_ref,
          lse.cpu().numpy().astype(np.float64).reshape(-1)[rows], L_ref)


def test_decode_million_key_cache(orc):
    """One sequence with 2^20 cached keys (512 MB of K and V): the split + combine and the
    one-launch decode against the oracle."""
    B, H, H_kv, N_k, d = 1, 8, 1, 1 << 20, 128
    name = "decode N_k=2^20"
    say(name)
    Q, K, V = decode_inputs(4600, B, H, H_kv, N_k, d)
    q, k, v = to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V)
    S = fa.decode_num_splits(B, H_kv, N_k, d)
    o_part, l_part = fa.decode_split(q, k, v, S)
    o, l = fa.combine(o_part, l_part)
    o1, l1 = fa.decode(q, k, v, S)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name + " S=%d" % S, bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    check(name + " one launch", bf16_dev_to_f64(o1), O_ref[:, :, 0], l1.cpu().numpy(), L_ref[:, :, 0])
