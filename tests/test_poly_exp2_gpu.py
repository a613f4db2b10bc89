"""GPU checks of the forward with polynomial exponentials (fa_fwd_poly_exp2, FA4's softmax trick;
CUDA Kernel interview course, FlashAttention v4 card): the polynomial's own error on the GPU,
and the forward's parity with the fp64 oracle under the standard gates, plus the derived
bound on how far its LSE may move from fa_fwd's."""
import numpy as np
import pytest

import oracle
from parity_util import bf16_dev_to_f64, check, fwd_inputs, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_59_amd")

BOUND = 8.6e-5              # relative error of the cubic in exact arithmetic (fit_exp2_poly)
EVAL = 8 * 2.0 ** -24       # fp32 evaluation: three FMAs and the reduction, a few ulp


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


def test_exp2_poly_error_on_gpu():
    rng = np.random.default_rng(11)
    ints = np.arange(-125, 9, dtype=np.float32)
    # just below and above every integer (where the reduction's floor changes), and tiny
    # magnitudes of both signs (the row maximum's argument is a rounding residue near 0)
    edges = np.concatenate([np.nextafter(ints, np.float32(-np.inf)), np.nextafter(ints, np.float32(np.inf)),
                            np.float32([-1e-30, -1e-12, -1e-8, -3e-8, -6e-8, 1e-30, 1e-8, -2.0 ** -24, -2.0 ** -25])])
    x = np.concatenate([np.linspace(-126.0, 8.0, 1 << 22), rng.uniform(-126.0, 8.0, 1 << 20),
                        rng.uniform(-1e-6, 1e-6, 1 << 16), edges.astype(np.float64)]).astype(np.float32)
    y = fa.exp2_poly(torch.from_numpy(x).cuda()).cpu().numpy().astype(np.float64)
    exact = np.exp2(x.astype(np.float64))
    rel = np.abs(y / exact - 1.0)
    say("exp2_poly max relative error", float(rel.max()))
    assert rel.max() <= BOUND + EVAL
    # integers: p(0) = 1, so 2^n exactly
    ints = np.arange(-126, 9, dtype=np.float32)
    yi = fa.exp2_poly(torch.from_numpy(ints).cuda()).cpu().numpy()
    assert np.array_equal(yi, np.exp2(ints.astype(np.float64)).astype(np.float32))
    # underflow: exactly 0 at and below -200 and for -inf; tiny in between
    low = np.array([-np.inf, -1e30, -1000.0, -200.0, -199.5, -150.0, -126.5], dtype=np.float32)
    yl = fa.exp2_poly(torch.from_numpy(low).cuda()).cpu().numpy()
    assert np.all(yl[:4] == 0.0)
    assert np.all((yl[4:] >= 0.0) & (yl[4:] < 2.0 ** -126))


CASES = [
    # B, H, H_kv, N_q, N_k, d, causal
    (1, 4, 2, 513, 513, 128, True),
    (2, 2, 1, 200, 333, 128, False),
    (2, 4, 4, 300, 300, 64, True),
    (1, 2, 2, 257, 700, 64, False),
    (1, 2, 2, 333, 200, 64, True),   # N_q > N_k: leading rows see no key (O = 0, LSE = -inf)
]


@pytest.mark.parametrize("quarters", [1, 2, 4])
@pytest.mark.parametrize("B,H,H_kv,N_q,N_k,d,causal", CASES)
def test_fwd_poly_exp2_parity(orc, quarters, B, H, H_kv, N_q, N_k, d, causal):
    name = "fwd poly exp2 q=%d %s" % (quarters, (B, H, H_kv, N_q, N_k, d, causal))
    say(name)
    Q, K, V = fwd_inputs(9100 + N_q + d + quarters, B, H, H_kv, N_q, N_k, d)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o, lse = fa.fwd(q, k, v, causal=causal, poly_exp2=quarters)
    o0, lse0 = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal)
    check(name, bf16_dev_to_f64(o), O_ref, lse.cpu().numpy(), L_ref)
    # Each probability carries a relative error <= BOUND + EVAL, so the row sum does too and
    # LSE moves by at most -ln(1 - that) ~ that; fp32 LSE evaluation adds a few ulp of |LSE|.
    l1, l0 = lse.cpu().numpy().astype(np.float64), lse0.cpu().numpy().astype(np.float64)
    fin = np.isfinite(l0)
    assert np.array_equal(fin, np.isfinite(l1)), name
    dl = np.abs(l1[fin] - l0[fin])
    allow = -np.log1p(-(BOUND + EVAL)) + 4 * 2.0 ** -23 * np.maximum(np.abs(l0[fin]), 1.0)
    say(name, "max |LSE - LSE(fa_fwd)| %.3g" % dl.max())
    assert np.all(dl <= allow), "%s: LSE moved %.3g from fa_fwd's" % (name, dl.max())
    assert dl.max() > 0.0, "%s: no exponential went through the polynomial" % name


WORKLOADS = [
    # name, seed, B, H, N, d, causal
    ("batched prefill N=1024 d=64", 2, 16, 16, 1024, 64, False),
    ("long causal N=8192 d=128", 3, 2, 16, 8192, 128, True),
]


@pytest.mark.parametrize("quarters", [1, 2, 4])
@pytest.mark.parametrize("name,seed,B,H,N,d,causal", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_fwd_poly_exp2_workloads(orc, quarters, name, seed, B, H, N, d, causal):
    """The workloads the benchmark times with polynomial exponentials, launched as it launches
    them: sampled rows against the oracle, every row's LSE within the derived bound of
    fa_fwd's."""
    from parity_util import sample_rows

    H_kv = H
    name = "fwd poly exp2 q=%d %s" % (quarters, name)
    say(name)
    Q, K, V = fwd_inputs(seed, B, H, H_kv, N, N, d)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o, lse = fa.fwd(q, k, v, causal=causal, poly_exp2=quarters)
    o0, lse0 = fa.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    rows = sample_rows(B, H, N, 256, seed)
    O_ref, L_ref = orc.attention(Q, K, V, causal=causal, rows=rows)
    O_gpu = bf16_dev_to_f64(o).reshape(-1, d)[rows]
    L_gpu = lse.cpu().numpy().astype(np.float64).reshape(-1)[rows]
    check(name + " (%d sampled rows)" % rows.size, O_gpu, O_ref, L_gpu, L_ref)
    l1, l0 = lse.double(), lse0.double()
    allow = -np.log1p(-(BOUND + EVAL)) + 4 * 2.0 ** -23 * torch.clamp(l0.abs(), min=1.0)
    assert bool(((l1 - l0).abs() <= allow).all()), name


@pytest.mark.parametrize("quarters", [1, 2, 4])
def test_fwd_poly_exp2_one_key_is_exact(quarters):
    """N_k = 1: the only score is the row maximum, whose exponent is exactly 0, and the
    polynomial gives 2^0 = 1 exactly, so O is the V row bit for bit, as with fa_fwd."""
    from parity_util import fwd_inputs as inputs

    Q, K, V = inputs(9300 + quarters, 2, 4, 2, 37, 1, 128)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o, _ = fa.fwd(q, k, v, poly_exp2=quarters)
    torch.cuda.synchronize()
    g = torch.arange(4, device="cuda") // 2
    assert torch.equal(o, v[:, g, :1].expand_as(o))
