"""GPU parity of fa_decode (flash-decoding in one launch: the split kernel's last workgroup
of each group merges the segments) against the fp64 oracle, on the shapes of the two-launch
path, on repeated calls that share one counter array, and at the full decode workload."""
import numpy as np
import pytest

import oracle
from parity_util import bf16_dev_to_f64, check, decode_inputs, say, to_dev

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


def check_fused(orc, name, Q, K, V, S, counters=None):
    """Run fa_decode and check the merged output, every segment's partial, and that the
    counters are back to zero."""
    B, H, d = Q.shape[0], Q.shape[1], Q.shape[3]
    N_k = K.shape[2]
    q, k, v = to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V)
    if counters is None:
        counters = torch.zeros(fa.decode_counter_bytes(B, H, K.shape[1]) // 4, dtype=torch.int32, device="cuda")
    o_part = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
    l_part = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    o, l = fa.decode(q, k, v, S, counters=counters, o_part=o_part, lse_part=l_part)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V)
    check(name, bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    L = -(-N_k // S)
    op = o_part.cpu().numpy().astype(np.float64)
    lp = l_part.cpu().numpy().astype(np.float64)
    for t in (range(S) if S <= 40 else sorted({0, 1, S // 2, S - 1})):
        lo, hi = min(t * L, N_k), min((t + 1) * L, N_k)
        O_s, L_s = orc.attention(Q, K, V, k_range=(lo, hi))
        check("%s segment %d" % (name, t), op[:, :, t], O_s[:, :, 0], lp[:, :, t], L_s[:, :, 0])
    assert int(counters.abs().sum().item()) == 0, name + ": counters not reset"
    return o, l


FUSED = [
    # B, H, H_kv, N_k, d, S
    (1, 4, 1, 100, 128, 1),      # one segment: the only workgroup merges
    (2, 8, 2, 1000, 128, 7),
    (2, 8, 2, 1000, 64, 64),
    (1, 4, 4, 333, 64, 333),     # one key per segment
    (1, 2, 1, 100, 128, 60),     # trailing segments empty
    (2, 20, 1, 515, 128, 5),     # 20 query heads per K/V head: two head groups, two counters
    (3, 6, 3, 37, 128, 2),
    (1, 64, 1, 300, 128, 3),     # 64 query heads per K/V head: four head chunks, four counters
    (2, 128, 2, 257, 64, 4),
]


@pytest.mark.parametrize("B,H,H_kv,N_k,d,S", FUSED)
def test_decode_fused_small(orc, B, H, H_kv, N_k, d, S):
    name = "fused decode%s" % str((B, H, H_kv, N_k, d, S))
    say(name)
    Q, K, V = decode_inputs(7000 + N_k + S, B, H, H_kv, N_k, d)
    check_fused(orc, name, Q, K, V, S)


def test_decode_fused_calls_share_counters(orc):
    """Three calls on one counter array (different inputs and segment counts): each merges
    correctly, so each left the counters at zero for the next."""
    B, H, H_kv, d = 2, 8, 2, 128
    counters = torch.zeros(fa.decode_counter_bytes(B, H, H_kv) // 4, dtype=torch.int32, device="cuda")
    for i, (N_k, S) in enumerate([(900, 9), (300, 3), (2000, 40)]):
        Q, K, V = decode_inputs(7100 + i, B, H, H_kv, N_k, d)
        check_fused(orc, "fused decode call %d N_k=%d S=%d" % (i, N_k, S), Q, K, V, S, counters=counters)


@pytest.mark.parametrize("N_k,seed", [(4096, 5), (65536, 6)])
def test_decode_fused_full_workload(orc, N_k, seed):
    """Both cache lengths of the flash-decoding workload, at the split count the library picks
    (the long cache's partials are checked on sampled segments, check_fused)."""
    B, H, H_kv, d = 4, 32, 8, 128
    S = fa.decode_num_splits(B, H_kv, N_k, d)
    name = "fused flash-decoding B=4 H=32/8 N_k=%d d=128 S=%d" % (N_k, S)
    say(name)
    Q, K, V = decode_inputs(seed, B, H, H_kv, N_k, d)
    o, l = check_fused(orc, name, Q, K, V, S)
    # the same result as the two-launch path up to the merge's summation order
    o_part, l_part = fa.decode_split(to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V), S)
    o2, l2 = fa.combine(o_part, l_part)
    torch.cuda.synchronize()
    # at most one bf16 ulp apart: the spacing of bf16 values in [2^e, 2^(e+1)) is 2^(e-7) <= 2^-7 |x|
    a, b = o.float(), o2.float()
    ratio = float(((a - b).abs() / (2 ** -7 * torch.maximum(a.abs(), b.abs()) + 1e-6)).max())
    assert ratio <= 1.0, "%s: |fused - two-launch| reaches %.3f bf16 ulp" % (name, ratio)
    assert float((l - l2).abs().max()) <= 1e-4, name


def test_decode_fused_is_deterministic():
    """The merging workgroup sums the S segments in index order, whichever workgroup finishes
    last: repeated calls agree bit for bit, also on the paged cache."""
    B, H, H_kv, N_k, d = 4, 32, 8, 4096, 128
    say("fused decode determinism", (B, H, H_kv, N_k, d))
    Q, K, V = decode_inputs(17, B, H, H_kv, N_k, d)
    q, k, v = to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V)
    # S fixed (not the CU-count heuristic): the paged path rounds segments up to 32-key blocks, so
    # paged and contiguous segments coincide only when N_k / S is a multiple of 32
    S = 16
    assert (N_k // S) % 32 == 0 and N_k % S == 0
    runs = [fa.decode(q, k, v, S) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(l.view(torch.int32), runs[0][1].view(torch.int32))
    # the same cache as one page pool in order (pages of 64 tokens), every sequence full length
    P = 64
    npp = N_k // P
    kp = k.view(B, H_kv, npp, P, d).permute(0, 2, 1, 3, 4).reshape(B * npp, H_kv, P, d).contiguous()
    vp = v.view(B, H_kv, npp, P, d).permute(0, 2, 1, 3, 4).reshape(B * npp, H_kv, P, d).contiguous()
    table = torch.arange(B * npp, dtype=torch.int32, device="cuda").view(B, npp)
    lens = torch.full((B,), N_k, dtype=torch.int32, device="cuda")
    pruns = [fa.decode_paged(q, kp, vp, table, lens, S) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in pruns[1:]:
        assert torch.equal(o.view(torch.int16), pruns[0][0].view(torch.int16))
        assert torch.equal(l.view(torch.int32), pruns[0][1].view(torch.int32))
    # paged and contiguous: the same keys in the same segments, so the same bits
    assert torch.equal(pruns[0][0].view(torch.int16), runs[0][0].view(torch.int16))


def test_poisoned_counters_are_reported_not_used(orc):
    """A counter array that is not zero on entry is reported (fa_decode_counters_check), the
    checked binding refuses to launch on it, and fa_decode_counters_reset makes it usable."""
    B, H, H_kv, N_k, d, S = 2, 8, 2, 1000, 128, 7
    Q, K, V = decode_inputs(7401, B, H, H_kv, N_k, d)
    q, k, v = to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V)
    n = fa.decode_counter_bytes(B, H, H_kv) // 4
    counters = torch.zeros(n, dtype=torch.int32, device="cuda")
    assert fa.decode_counters_check(counters, B, H, H_kv) == 0
    counters[0] = 3  # as if a group had been counted and never cleared
    counters[-1] = -1
    assert fa.decode_counters_check(counters, B, H, H_kv) == (2 if n > 1 else 1)
    with pytest.raises(RuntimeError, match="not zero"):
        fa.decode(q, k, v, S, counters=counters, check_counters=True)
    fa.decode_counters_reset(counters, B, H, H_kv)
    assert fa.decode_counters_check(counters, B, H, H_kv) == 0
    o, l = fa.decode(q, k, v, S, counters=counters, check_counters=True)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V)
    check("decode after counters reset", bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    assert fa.decode_counters_check(counters, B, H, H_kv) == 0
