"""fa_decode_static (the one-launch decode with its workspace in the library's static device
array, for callers that cannot allocate) against fa_decode on the same inputs and split count,
called through the C ABI: two calls in a row, the second on a smaller input; both outputs are
compared bit for bit with fa_decode's and against the fp64 oracle at the parity gates."""
import ctypes
import math

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


def run_static(q, k, v, S):
    """fa_decode_static through the C ABI (ctypes, plain device pointers)."""
    lib = fa.library()
    B, H, d = q.shape
    H_kv, N_k = k.shape[1], k.shape[2]
    o = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.fa_decode_static(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                              ctypes.c_void_p(lse.data_ptr()), B, H, H_kv, N_k, d, S, 1.0 / math.sqrt(d),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fa.strerror(st)
    return o, lse


CASES = [
    # B, H, H_kv, N_k, d, S: the flash-decoding workload's short cache, then a smaller input
    (4, 32, 8, 4096, 128, 16),
    (2, 8, 2, 1000, 64, 7),
]


def test_static_matches_fa_decode_two_calls():
    orc = oracle.Oracle()
    for i, (B, H, H_kv, N_k, d, S) in enumerate(CASES):
        name = "fa_decode_static call %d %s" % (i + 1, str((B, H, H_kv, N_k, d, S)))
        say(name)
        Q, K, V = decode_inputs(9100 + i, B, H, H_kv, N_k, d)
        q, k, v = to_dev(Q[:, :, 0, :]), to_dev(K), to_dev(V)
        o_s, l_s = run_static(q, k, v, S)
        o_f, l_f = fa.decode(q, k, v, S)
        torch.cuda.synchronize()
        # the same kernel and split count: the same bits
        assert torch.equal(o_s.view(torch.int16), o_f.view(torch.int16)), name + ": O differs from fa_decode"
        assert torch.equal(l_s, l_f), name + ": LSE differs from fa_decode"
        O_ref, L_ref = orc.attention(Q, K, V)
        check(name, bf16_dev_to_f64(o_s), O_ref[:, :, 0], l_s.cpu().numpy(), L_ref[:, :, 0])
