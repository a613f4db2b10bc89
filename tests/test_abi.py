"""The C ABI of libfa.so without a GPU: exports, validation statuses, host helpers.

Every compute call made here is invalid on purpose, so it returns from argument
validation before any HIP call; nothing is enqueued and no pointer is touched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("exact_attention_59_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        from exact_attention_59_amd import build

        build.build()
    return fa.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def exported_symbols(path):
    out = os.popen("nm -D --defined-only %s" % path).read()
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fp8_quantize", "fa_fwd_fp8", "fa_fp8_block_rows",
                 "fa_decode_split", "fa_decode_split_paged", "fa_combine", "fa_decode_num_splits",
                 "fa_decode_workspace_bytes", "fa_strerror", "fa_fwd_tile_shape", "fa_fwd_tile_count",
                 "fa_fwd_poly_exp2", "fa_exp2_poly"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    exported = exported_symbols(fa.library_path())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)
    # nothing else of ours leaks out of the library
    ours = {s for s in exported if s.startswith("fa_")}
    assert ours == set(declared_functions())


P = ctypes.c_void_p(0x100000)       # aligned, never dereferenced (validation fails first)
P_MIS = ctypes.c_void_p(0x100004)   # 4-byte aligned only


def fwd(lib, Q=P, K=P, V=P, O=P, L=P, B=1, H=1, H_kv=1, N_q=8, N_k=8, d=64, causal=0, scale=0.125):
    return lib.fa_fwd(Q, K, V, O, L, B, H, H_kv, N_q, N_k, d, causal, scale, None)


def fwd_poly(lib, Q=P, K=P, V=P, O=P, L=P, B=1, H=1, H_kv=1, N_q=8, N_k=8, d=64, causal=0, scale=0.125, quarters=1):
    return lib.fa_fwd_poly_exp2(Q, K, V, O, L, B, H, H_kv, N_q, N_k, d, causal, scale, quarters, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(L=None), fa.FA_ERR_NULL), (dict(B=0), fa.FA_ERR_SHAPE),
    (dict(H=3, H_kv=2), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED), (dict(O=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=0.0), fa.FA_ERR_ARG), (dict(causal=2), fa.FA_ERR_ARG),
    (dict(quarters=0), fa.FA_ERR_ARG), (dict(quarters=3), fa.FA_ERR_ARG), (dict(quarters=5), fa.FA_ERR_ARG),
    (dict(quarters=-1), fa.FA_ERR_ARG),
])
def test_fwd_poly_exp2_validation(lib, kw, status):
    assert fwd_poly(lib, **kw) == status


def test_exp2_poly_validation(lib):
    assert lib.fa_exp2_poly(None, P, 4, None) == fa.FA_ERR_NULL
    assert lib.fa_exp2_poly(P, None, 4, None) == fa.FA_ERR_NULL
    assert lib.fa_exp2_poly(P, P, -1, None) == fa.FA_ERR_SHAPE
    assert lib.fa_exp2_poly(ctypes.c_void_p(0x100002), P, 4, None) == fa.FA_ERR_ALIGN
    assert lib.fa_exp2_poly(P, P, 0, None) == fa.FA_OK  # nothing to do: no launch


def bwd(lib, Q=P, K=P, V=P, O=P, dO=P, L=P, dQ=P, dK=P, dV=P, W=P, B=1, H=2, H_kv=1, N_q=8, N_k=8, d=64, causal=0,
        scale=0.125):
    return lib.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, W, B, H, H_kv, N_q, N_k, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(O=None), fa.FA_ERR_NULL), (dict(dO=None), fa.FA_ERR_NULL),
    (dict(L=None), fa.FA_ERR_NULL), (dict(dQ=None), fa.FA_ERR_NULL), (dict(dK=None), fa.FA_ERR_NULL),
    (dict(dV=None), fa.FA_ERR_NULL), (dict(W=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N_q=0), fa.FA_ERR_SHAPE), (dict(N_k=-1), fa.FA_ERR_SHAPE),
    (dict(H=3, H_kv=2), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dO=P_MIS), fa.FA_ERR_ALIGN), (dict(dK=P_MIS), fa.FA_ERR_ALIGN), (dict(W=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=float("inf")), fa.FA_ERR_ARG), (dict(causal=3), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_ARG), (dict(scale=-0.125), fa.FA_ERR_ARG),
])
def test_bwd_validation(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_workspace_bytes(lib):
    assert fa.bwd_workspace_bytes(2, 16, 1000) == 2 * 16 * 1000 * 4
    assert fa.bwd_workspace_bytes(0, 16, 1000) == 0
    assert fa.bwd_workspace_bytes(1, 1, -3) == 0


def q8(lib, Q=P, K=P, V=P, inc=1, Q8=P, K8=P, Vt=P, qs=P, ks=P, vs=P, B=1, H=2, H_kv=1, N_q=8, N_k=8, d=64):
    return lib.fa_fp8_quantize(Q, K, V, inc, 1, 2, Q8, K8, Vt, qs, ks, vs, B, H, H_kv, N_q, N_k, d, None)


def f8(lib, Q8=P, K8=P, Vt=P, qs=P, ks=P, vs=P, O=P, L=P, B=1, H=2, H_kv=1, N_q=8, N_k=8, d=64, causal=0, scale=0.125):
    return lib.fa_fwd_fp8(Q8, K8, Vt, qs, ks, vs, O, L, B, H, H_kv, N_q, N_k, d, causal, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(Vt=None), fa.FA_ERR_NULL), (dict(vs=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N_k=-2), fa.FA_ERR_SHAPE), (dict(H=3, H_kv=2), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(Q8=P_MIS), fa.FA_ERR_ALIGN), (dict(Vt=P_MIS), fa.FA_ERR_ALIGN),
    (dict(qs=ctypes.c_void_p(0x100002)), fa.FA_ERR_ALIGN), (dict(inc=2), fa.FA_ERR_ARG),
])
def test_fp8_quantize_validation(lib, kw, status):
    assert q8(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(Q8=None), fa.FA_ERR_NULL), (dict(ks=None), fa.FA_ERR_NULL), (dict(L=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=5, H_kv=2), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(O=P_MIS), fa.FA_ERR_ALIGN), (dict(K8=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=0.0), fa.FA_ERR_ARG), (dict(scale=float("nan")), fa.FA_ERR_ARG), (dict(causal=2), fa.FA_ERR_ARG),
])
def test_fwd_fp8_validation(lib, kw, status):
    assert f8(lib, **kw) == status


def test_fp8_scale_arrays_need_only_4_bytes(lib):
    four = ctypes.c_void_p(0x100004)
    assert q8(lib, qs=four, ks=four, vs=four, inc=2) == fa.FA_ERR_ARG  # alignment passes, the flag fails
    assert fa.fp8_block_rows() == (128, 64)


def dec(lib, Q=P, K=P, V=P, Op=P, Lp=P, B=1, H=4, H_kv=1, N_k=64, d=128, S=4, scale=0.1):
    return lib.fa_decode_split(Q, K, V, Op, Lp, B, H, H_kv, N_k, d, S, scale, None)


def comb(lib, Op=P, Lp=P, O=P, L=P, B=1, H=4, d=128, S=4):
    return lib.fa_combine(Op, Lp, O, L, B, H, d, S, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(K=None), fa.FA_ERR_NULL), (dict(V=None), fa.FA_ERR_NULL),
    (dict(O=None), fa.FA_ERR_NULL), (dict(L=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=-1), fa.FA_ERR_SHAPE), (dict(H_kv=0), fa.FA_ERR_SHAPE),
    (dict(N_q=0), fa.FA_ERR_SHAPE), (dict(N_k=0), fa.FA_ERR_SHAPE), (dict(d=0), fa.FA_ERR_SHAPE),
    (dict(H=6, H_kv=4), fa.FA_ERR_SHAPE),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=256), fa.FA_ERR_UNSUPPORTED), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(Q=P_MIS), fa.FA_ERR_ALIGN), (dict(O=P_MIS), fa.FA_ERR_ALIGN), (dict(L=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=float("inf")), fa.FA_ERR_ARG), (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(causal=2), fa.FA_ERR_ARG), (dict(causal=-1), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_ARG), (dict(scale=-0.125), fa.FA_ERR_ARG), (dict(scale=-0.0), fa.FA_ERR_ARG),
])
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(Op=None), fa.FA_ERR_NULL), (dict(Lp=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N_k=-5), fa.FA_ERR_SHAPE), (dict(H=5, H_kv=2), fa.FA_ERR_SHAPE),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(S=65), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED), (dict(H=65, H_kv=1), fa.FA_ERR_UNSUPPORTED),
    (dict(K=P_MIS), fa.FA_ERR_ALIGN), (dict(Lp=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=float("-inf")), fa.FA_ERR_ARG), (dict(scale=0.0), fa.FA_ERR_ARG), (dict(scale=-1.0), fa.FA_ERR_ARG),
])
def test_decode_validation(lib, kw, status):
    assert dec(lib, **kw) == status


def dec_fused(lib, Q=P, K=P, V=P, Op=P, Lp=P, C=P, O=P, L=P, B=1, H=4, H_kv=1, N_k=64, d=128, S=4, scale=0.1):
    return lib.fa_decode(Q, K, V, Op, Lp, C, O, L, B, H, H_kv, N_k, d, S, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(Op=None), fa.FA_ERR_NULL), (dict(Lp=None), fa.FA_ERR_NULL),
    (dict(C=None), fa.FA_ERR_NULL), (dict(O=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(N_k=-5), fa.FA_ERR_SHAPE), (dict(H=5, H_kv=2), fa.FA_ERR_SHAPE),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(S=65), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED), (dict(H=65, H_kv=1), fa.FA_ERR_UNSUPPORTED),
    (dict(K=P_MIS), fa.FA_ERR_ALIGN), (dict(O=P_MIS), fa.FA_ERR_ALIGN), (dict(L=P_MIS), fa.FA_ERR_ALIGN),
    (dict(C=ctypes.c_void_p(0x100002)), fa.FA_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA_ERR_ARG), (dict(scale=0.0), fa.FA_ERR_ARG),
])
def test_decode_fused_validation(lib, kw, status):
    assert dec_fused(lib, **kw) == status


def test_decode_fused_counters_need_only_4_bytes_and_lse_is_optional(lib):
    # 4-byte aligned counters and no LSE output pass the alignment checks: the scale check, which
    # comes after them, is what fails (nothing runs)
    assert dec_fused(lib, C=P_MIS, L=None, scale=0.0) == fa.FA_ERR_ARG


def dec_static(lib, Q=P, K=P, V=P, O=P, L=P, B=1, H=4, H_kv=1, N_k=64, d=128, S=4, scale=0.1):
    return lib.fa_decode_static(Q, K, V, O, L, B, H, H_kv, N_k, d, S, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(O=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=5, H_kv=2), fa.FA_ERR_SHAPE), (dict(S=65), fa.FA_ERR_SHAPE),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED), (dict(H=65, H_kv=1), fa.FA_ERR_UNSUPPORTED),
    # beyond the 16 MiB static array: 4*32*1000*(128+1)*4 bytes of partials
    (dict(B=4, H=32, H_kv=8, N_k=4096, S=1000), fa.FA_ERR_CAPACITY),
    # more group counters than its 64 KiB hold
    (dict(B=20000, H=8, H_kv=1, N_k=64, S=1), fa.FA_ERR_CAPACITY),
    (dict(K=P_MIS), fa.FA_ERR_ALIGN), (dict(L=P_MIS), fa.FA_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA_ERR_ARG), (dict(scale=0.0), fa.FA_ERR_ARG),
])
def test_decode_static_validation(lib, kw, status):
    assert dec_static(lib, **kw) == status


def test_decode_static_capacity_boundary(lib):
    # the flash-decoding workload fits at 16 and 64 segments (checks pass up to the scale check) ...
    assert dec_static(lib, B=4, H=32, H_kv=8, N_k=65536, S=16, scale=0.0) == fa.FA_ERR_ARG
    assert dec_static(lib, B=4, H=32, H_kv=8, N_k=65536, S=64, scale=0.0) == fa.FA_ERR_ARG
    # ... and 4*32*S*129*4 bytes (+ 64 KiB of counters) first exceeds 16 MiB at S = 254
    assert dec_static(lib, B=4, H=32, H_kv=8, N_k=65536, S=253, scale=0.0) == fa.FA_ERR_ARG
    assert dec_static(lib, B=4, H=32, H_kv=8, N_k=65536, S=254, scale=0.0) == fa.FA_ERR_CAPACITY
    # LSE is optional
    assert dec_static(lib, L=None, scale=0.0) == fa.FA_ERR_ARG


@pytest.mark.parametrize("fn", ["reset", "check"])
@pytest.mark.parametrize("kw,status", [
    (dict(C=None), fa.FA_ERR_NULL), (dict(B=0), fa.FA_ERR_SHAPE), (dict(H=6, H_kv=4), fa.FA_ERR_SHAPE),
    (dict(C=ctypes.c_void_p(0x100002)), fa.FA_ERR_ALIGN),
])
def test_decode_counters_helpers_validation(lib, fn, kw, status):
    a = dict(C=P, B=2, H=8, H_kv=2)
    a.update(kw)
    if fn == "reset":
        st = lib.fa_decode_counters_reset(a["C"], a["B"], a["H"], a["H_kv"], None)
    else:
        st = lib.fa_decode_counters_check(a["C"], a["B"], a["H"], a["H_kv"], P, None)
    assert st == status


def test_decode_counters_check_needs_its_output(lib):
    assert lib.fa_decode_counters_check(P, 2, 8, 2, None, None) == fa.FA_ERR_NULL
    assert lib.fa_decode_counters_check(P, 2, 8, 2, ctypes.c_void_p(0x100001), None) == fa.FA_ERR_ALIGN


def test_decode_counter_bytes(lib):
    assert fa.decode_counter_bytes(4, 32, 8) == 4 * 8 * 1 * 4
    assert fa.decode_counter_bytes(2, 40, 2) == 2 * 2 * 2 * 4   # 20 query heads per K/V head: two chunks of 16
    assert fa.decode_counter_bytes(0, 32, 8) == 0
    assert fa.decode_counter_bytes(1, 6, 4) == 0


def paged_fused(lib, Q=P, K=P, V=P, T=P, Ls=P, Op=P, Lp=P, C=P, O=P, L=P, B=2, H=4, H_kv=1, page=16, max_pages=8,
                num_pages=16, d=128, S=4, scale=0.1):
    return lib.fa_decode_paged(Q, K, V, T, Ls, Op, Lp, C, O, L, B, H, H_kv, page, max_pages, num_pages, d, S, scale,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(C=None), fa.FA_ERR_NULL), (dict(O=None), fa.FA_ERR_NULL), (dict(T=None), fa.FA_ERR_NULL),
    (dict(Lp=None), fa.FA_ERR_NULL), (dict(S=0), fa.FA_ERR_SHAPE), (dict(S=129), fa.FA_ERR_SHAPE),
    (dict(page=24), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(K=P_MIS), fa.FA_ERR_ALIGN), (dict(O=P_MIS), fa.FA_ERR_ALIGN), (dict(L=P_MIS), fa.FA_ERR_ALIGN),
    (dict(C=ctypes.c_void_p(0x100002)), fa.FA_ERR_ALIGN), (dict(scale=float("inf")), fa.FA_ERR_ARG),
])
def test_decode_paged_fused_validation(lib, kw, status):
    assert paged_fused(lib, **kw) == status


def paged(lib, Q=P, K=P, V=P, T=P, Ls=P, Op=P, Lp=P, B=2, H=4, H_kv=1, page=16, max_pages=8, num_pages=16,
          d=128, S=4, scale=0.1):
    return lib.fa_decode_split_paged(Q, K, V, T, Ls, Op, Lp, B, H, H_kv, page, max_pages, num_pages, d, S, scale,
                                     None)


P_INT = ctypes.c_void_p(0x100004)   # 4-byte aligned: fine for the int32 arrays
P_ODD = ctypes.c_void_p(0x100002)   # 2-byte aligned


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), fa.FA_ERR_NULL), (dict(T=None), fa.FA_ERR_NULL), (dict(Ls=None), fa.FA_ERR_NULL),
    (dict(K=None), fa.FA_ERR_NULL), (dict(Lp=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(page=0), fa.FA_ERR_SHAPE), (dict(max_pages=0), fa.FA_ERR_SHAPE),
    (dict(num_pages=-1), fa.FA_ERR_SHAPE), (dict(H=5, H_kv=2), fa.FA_ERR_SHAPE),
    (dict(S=0), fa.FA_ERR_SHAPE), (dict(S=16 * 8 + 1), fa.FA_ERR_SHAPE),
    (dict(page=24), fa.FA_ERR_UNSUPPORTED), (dict(page=8), fa.FA_ERR_UNSUPPORTED),
    (dict(page=8192), fa.FA_ERR_UNSUPPORTED), (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(H=65, H_kv=1), fa.FA_ERR_UNSUPPORTED),
    (dict(K=P_MIS), fa.FA_ERR_ALIGN), (dict(T=P_ODD), fa.FA_ERR_ALIGN), (dict(Ls=P_ODD), fa.FA_ERR_ALIGN),
    (dict(scale=float("nan")), fa.FA_ERR_ARG), (dict(scale=-0.5), fa.FA_ERR_ARG),
])
def test_decode_paged_validation(lib, kw, status):
    assert paged(lib, **kw) == status


def test_decode_paged_int_pointers_need_only_4_bytes(lib):
    # 4-byte aligned table and lengths pass the alignment check (a later check fails instead)
    assert paged(lib, T=P_INT, Ls=P_INT, S=0) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("kw,status", [
    (dict(Op=None), fa.FA_ERR_NULL), (dict(O=None), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_SHAPE), (dict(S=0), fa.FA_ERR_SHAPE), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(O=P_MIS), fa.FA_ERR_ALIGN), (dict(L=P_MIS), fa.FA_ERR_ALIGN),
])
def test_combine_validation(lib, kw, status):
    assert comb(lib, **kw) == status


def test_strerror_covers_every_status(lib):
    texts = {fa.strerror(s) for s in range(8)}
    assert len(texts) == 8
    assert fa.strerror(99) == "unknown status"


def test_workspace_bytes(lib):
    assert fa.decode_workspace_bytes(4, 32, 128, 16) == 4 * 32 * 16 * (128 + 1) * 4
    assert fa.decode_workspace_bytes(0, 32, 128, 16) == 0
    assert fa.decode_workspace_bytes(1, 1, 64, -1) == 0


def test_num_splits_range(lib):
    for (B, H_kv, N_k) in [(4, 8, 4096), (4, 8, 65536), (1, 1, 1), (1, 2, 300), (64, 8, 2048), (256, 8, 128)]:
        s = fa.decode_num_splits(B, H_kv, N_k, 128)
        assert 1 <= s <= N_k
        assert -(-N_k // s) >= min(N_k, 256) or s == 1  # segments are not shorter than 256 keys
    assert fa.decode_num_splits(0, 8, 4096, 128) == 0
    # more sequences need fewer splits (wave quantisation, Lecture 11 section 6.4)
    assert fa.decode_num_splits(1, 8, 65536, 128) >= fa.decode_num_splits(16, 8, 65536, 128)


def test_tile_shape(lib):
    # whole 32-row blocks per wave and whole 32-key MFMA blocks per tile
    for d in (64, 128):
        br, bc = fa.fwd_tile_shape(d)
        assert br % 32 == 0 and bc % 32 == 0
    with pytest.raises(fa.FAError):
        fa.fwd_tile_shape(96)
