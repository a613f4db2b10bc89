"""GPU parity of flash-decoding over a paged key/value cache (fa_decode_split_paged, and
fa_decode_paged: the same split and the merge in one launch).

The cache of each sequence is drawn contiguously by the seeded generator and then
scattered over a shuffled pool of pages; the oracle computes plain attention on the
contiguous copy.  Pages no sequence owns are filled with NaN, so a kernel that touched
a wrong page (or a row past a sequence's length) would fail the finite-output gate.
"""
import math

import numpy as np
import pytest

import oracle
from parity_util import bf16_dev_to_f64, check, decode_inputs, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_59_amd")

BF16_NAN = np.uint16(0x7FC0)


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


def make_paged(K, V, lens, P, seed, spare=3):
    """Scatter K/V [B,H_kv,N,d] (first lens[b] tokens valid) over a shuffled page pool."""
    B, H_kv, N, d = K.shape
    rng = np.random.default_rng(seed)
    n_pages = [-(-int(n) // P) for n in lens]
    max_pages = max(1, max(n_pages))
    num_pages = sum(n_pages) + spare
    perm = rng.permutation(num_pages)
    Kp = np.full((num_pages, H_kv, P, d), BF16_NAN, dtype=np.uint16)
    Vp = np.full((num_pages, H_kv, P, d), BF16_NAN, dtype=np.uint16)
    table = np.empty((B, max_pages), dtype=np.int32)
    spare_pages = perm[sum(n_pages):]
    nxt = 0
    for b in range(B):
        for i in range(max_pages):
            if i < n_pages[b]:
                p = int(perm[nxt])
                nxt += 1
                rows = min(P, int(lens[b]) - i * P)
                Kp[p, :, :rows] = K[b, :, i * P:i * P + rows]
                Vp[p, :, :rows] = V[b, :, i * P:i * P + rows]
                table[b, i] = p
            else:  # unused slots point at NaN pages: they must never be read
                table[b, i] = int(spare_pages[i % len(spare_pages)])
    return Kp, Vp, table


def run_paged(Q, Kp, Vp, table, lens, S):
    q = to_dev(Q[:, :, 0, :])
    kp, vp = to_dev(Kp), to_dev(Vp)
    t = torch.from_numpy(table).cuda()
    ln = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o_part, l_part = fa.decode_split_paged(q, kp, vp, t, ln, S)
    o, l = fa.combine(o_part, l_part)
    torch.cuda.synchronize()
    return o_part, l_part, o, l


def segment_bounds(n, S):
    """Segments of the paged split: ceil(n / S) rounded up to whole 32-key blocks."""
    L = -(-(-(-n // S)) // 32) * 32 if n > 0 else 0
    return [(min(t * L, n), min(t * L + L, n)) for t in range(S)]


def reference(orc, Q, K, V, lens):
    B, H, _, d = Q.shape
    O = np.zeros((B, H, d))
    Lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        o, l = orc.attention(Q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n])
        O[b], Lse[b] = o[0, :, 0], l[0, :, 0]
    return O, Lse


def check_segments(orc, name, Q, K, V, lens, S, o_part, l_part):
    op = o_part.cpu().numpy().astype(np.float64)
    lp = l_part.cpu().numpy().astype(np.float64)
    for b, n in enumerate(lens):
        for t, (lo, hi) in enumerate(segment_bounds(int(n), S)):
            if hi <= lo:
                assert np.all(np.isneginf(lp[b, :, t])), "%s: empty segment lse" % name
                assert np.all(op[b, :, t] == 0.0), "%s: empty segment o" % name
                continue
            o, l = orc.attention(Q[b:b + 1], K[b:b + 1], V[b:b + 1], k_range=(lo, hi))
            check("%s seq %d segment %d" % (name, b, t), op[b:b + 1, :, t], o[:, :, 0], lp[b:b + 1, :, t],
                  l[:, :, 0])


PAGED = [
    # B, H, H_kv, lens, d, page, S
    (3, 8, 2, (1000, 1, 513), 128, 16, 7),
    (2, 4, 4, (4095, 0), 64, 64, 4),          # an empty sequence: O = 0, LSE = -inf
    (2, 20, 1, (515, 77), 128, 32, 5),        # 20 query heads per K/V head
    (2, 8, 2, (300, 5000), 128, 256, 3),
    (1, 16, 1, (64,), 64, 16, 3),             # trailing segments empty
    (2, 4, 1, (33, 47), 128, 16, 1),
    (2, 128, 2, (300, 129), 64, 32, 3),       # 64 query heads per K/V head: four head chunks
    (1, 4, 1, (20000,), 128, 16, 1),         # one segment of 625 blocks: a wave's blocks past its
                                             # 128th read the block table directly
]


@pytest.mark.parametrize("B,H,H_kv,lens,d,P,S", PAGED)
def test_paged_small(orc, B, H, H_kv, lens, d, P, S):
    name = "paged%s" % str((B, H, H_kv, lens, d, P, S))
    say(name)
    N = max(1, max(lens))
    Q, K, V = decode_inputs(3000 + N + P + S, B, H, H_kv, N, d)
    Kp, Vp, table = make_paged(K, V, lens, P, seed=N + S)
    o_part, l_part, o, l = run_paged(Q, Kp, Vp, table, lens, S)
    check_segments(orc, name, Q, K, V, lens, S, o_part, l_part)
    O_ref, L_ref = reference(orc, Q, K, V, lens)
    check(name + " combined", bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)


@pytest.mark.parametrize("P", [16, 128])
def test_paged_decode_workload(orc, P):
    """The decode benchmark shape (B=4, H=32/8, d=128, 4096 cached tokens) over shuffled pages."""
    B, H, H_kv, d, N = 4, 32, 8, 128, 4096
    S = fa.decode_num_splits(B, H_kv, N, d)
    name = "paged decode B=4 H=32/8 N=4096 d=128 P=%d S=%d" % (P, S)
    say(name)
    Q, K, V = decode_inputs(5, B, H, H_kv, N, d)
    lens = (N, N - 1, N // 2 + 3, 1)
    Kp, Vp, table = make_paged(K, V, lens, P, seed=P)
    o_part, l_part, o, l = run_paged(Q, Kp, Vp, table, lens, S)
    O_ref, L_ref = reference(orc, Q, K, V, lens)
    check(name, bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)
    check_segments(orc, name, Q[:2], K[:2], V[:2], lens[:2], S, o_part[:2], l_part[:2])


@pytest.mark.parametrize("B,H,H_kv,lens,d,P,S", PAGED)
def test_paged_one_launch(orc, shared_paged_counters, B, H, H_kv, lens, d, P, S):
    """fa_decode_paged against the oracle, and its partials against fa_decode_split_paged's; one
    counter array serves every case and must be left zero by each."""
    name = "paged one-launch%s" % str((B, H, H_kv, lens, d, P, S))
    say(name)
    N = max(1, max(lens))
    Q, K, V = decode_inputs(3000 + N + P + S, B, H, H_kv, N, d)
    Kp, Vp, table = make_paged(K, V, lens, P, seed=N + S)
    q, kp, vp = to_dev(Q[:, :, 0, :]), to_dev(Kp), to_dev(Vp)
    t = torch.from_numpy(table).cuda()
    ln = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o_part = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
    l_part = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    o, l = fa.decode_paged(q, kp, vp, t, ln, S, counters=shared_paged_counters, o_part=o_part, lse_part=l_part)
    torch.cuda.synchronize()
    O_ref, L_ref = reference(orc, Q, K, V, lens)
    check(name, bf16_dev_to_f64(o), O_ref, l.cpu().numpy(), L_ref)
    check_segments(orc, name, Q, K, V, lens, S, o_part, l_part)
    assert int(shared_paged_counters.abs().sum()) == 0, name + ": a group counter was left non-zero"


@pytest.fixture(scope="module")
def shared_paged_counters():
    n = max(fa.decode_counter_bytes(B, H, H_kv) for B, H, H_kv, _, _, _, _ in PAGED) // 4
    return torch.zeros(n, dtype=torch.int32, device="cuda:0")


def test_paged_full_long_cache(orc):
    """The flash-decoding workload's long cache (B=4, H=32, H_kv=8, N_k=65536, d=128) scattered
    over a shuffled pool of 16-token pages: the paged split + combine and the one-launch
    fa_decode_paged against the oracle on the contiguous cache."""
    B, H, H_kv, N_k, d, P = 4, 32, 8, 65536, 128, 16
    S = fa.decode_num_splits(B, H_kv, N_k, d)
    name = "paged flash-decoding B=4 H=32/8 N_k=65536 d=128 page=16 S=%d" % S
    say(name)
    Q, K, V = decode_inputs(6, B, H, H_kv, N_k, d)
    lens = [N_k] * B
    Kp, Vp, table = make_paged(K, V, lens, P, seed=66, spare=2)
    O_ref, L_ref = orc.attention(Q, K, V)
    o_part, l_part, o, l = run_paged(Q, Kp, Vp, table, lens, S)
    check(name + " split + combine", bf16_dev_to_f64(o), O_ref[:, :, 0], l.cpu().numpy(), L_ref[:, :, 0])
    q = to_dev(Q[:, :, 0, :])
    kp, vp = to_dev(Kp), to_dev(Vp)
    t = torch.from_numpy(table).cuda()
    ln = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o1, l1 = fa.decode_paged(q, kp, vp, t, ln, S)
    torch.cuda.synchronize()
    check(name + " one launch", bf16_dev_to_f64(o1), O_ref[:, :, 0], l1.cpu().numpy(), L_ref[:, :, 0])
