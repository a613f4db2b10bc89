#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs fwd,fwd_other,decode,...]

One step = fa_fwd over the long-sequence causal workload (B=2, H=16, N_q=N_k=8192,
d=128, bf16, causal mask), the largest forward workload that the configurations name.
`value` is that step's nominal FLOPs (4*B*H*N_q*N_k*d, halved under the causal mask)
over its GPU time, in TFLOPS.  Before the timed steps the GPU runs the step for at least
30 ms (its clock drops for about 10 ms after sustained load starts) and then W more steps.
The other forward workloads (batched prefill B=16 H=16 N=1024 d=64 without and with the
causal mask, grouped-query ragged causal B=4 H=32/8 N=4095 d=128, and the batched-prefill
shape at d=128) are reported under "forward_workloads", each timed the same way.
The flash-decoding leg (B=4, H=32, H_kv=8, d=128, N_k = 4096 and 65536; split kernel
then combine kernel) runs in the same invocation and is reported under "decode" in
GB/s of K+V read once, against the 8 TB/s HBM peak.  The split kernel's rate comes from
back-to-back launches over rotated copies of the cache (at least 640 MB read between two
uses of a copy, beyond the 256 MB last-level cache); per-repetition timings, with a 640 MB
read sweep before each repetition, are reported beside it and for the combine.  The backward leg
(fa_bwd on the batched-prefill shape) is reported under "backward", in TFLOP/s of its five
N_q x N_k x d products.  The FP8 leg (quantiser + e4m3 forward) is reported under "fp8",
against the 5.03 PFLOP/s dense fp8 peak.  The poly leg times fa_fwd_poly_exp2 (a quarter, half
or all of the softmax exponentials by a cubic on the FMA units) against fa_fwd, under
"fwd_poly_exp2".

Inputs are synthetic and seeded (counter-based SplitMix64 + Box-Muller, see gen/),
already resident in device memory when timing starts.  GPU times come from HIP
events recorded on the stream the kernels run on.  The fp64 oracle is timed on the
host cores on a bounded sample of the step's workload (whole (batch, head) slices of the
long causal workload; cpu_baseline); it is a reported baseline, not a target.

Prints one JSON line.  --gpus N with N > 1 exits with an explanation: this build
measures one GPU's share only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 (e4m3) MFMA, twice the bf16 rate
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attn fwd TFLOPS & % bf16 MFMA peak; split-KV decode HBM GB/s & % peak"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
SQ_COUNTERS_FILE = os.path.join(ROOT, "profiles", "sq_counters.json")
# The sources each kernel family is compiled from: a counter summary stays valid for a kernel
# while these hash the same.
KERNEL_SOURCES = {"fwd_kernel": ["fa_common.hpp", "fa_launch.hpp", "fa_fwd.hip"],
                  "fwd_fp8_kernel": ["fa_common.hpp", "fa_launch.hpp", "fa_fp8.hip"],
                  "fp8_quant_kernel": ["fa_common.hpp", "fa_launch.hpp", "fa_fp8.hip"],
                  "bwd": ["fa_common.hpp", "fa_launch.hpp", "fa_bwd.hip"],
                  "decode_split_kernel": ["fa_common.hpp", "fa_launch.hpp", "fa_decode.hip"],
                  "combine_kernel": ["fa_common.hpp", "fa_launch.hpp", "fa_decode.hip"]}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources `kernel` (a name such as "fwd_kernel<128, true>") is built from."""
    family = kernel.split("<")[0].strip()
    family = "bwd" if family.startswith("bwd_") else family
    if family not in KERNEL_SOURCES:
        raise KeyError("no source list for kernel %r" % kernel)
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "exact_attention_59_amd", "csrc", name)) as f:
            text = f.read()
        # comments and layout do not change a kernel: hash the code tokens only
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def dev_bf16(a):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def fwd_inputs(seed, B, H, H_kv, N, d):
    import gen

    return (gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, N, d)), gen.normal_bf16(seed, gen.TENSOR_K, (B, H_kv, N, d)),
            gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N, d)))


def fwd_flops(B, H, N_q, N_k, d, causal):
    f = 4.0 * B * H * N_q * N_k * d
    return f / 2 if causal else f


# ---------------------------------------------------------------------------------- legs
HEADLINE = dict(name="long causal B=2 H=16 H_kv=16 N_q=N_k=8192 d=128 bf16", seed=3, B=2, H=16, H_kv=16, N=8192,
                d=128, causal=True)


def settle(torch, fn, ms=30.0, chunk=10):
    """Run fn until at least `ms` of GPU time has passed on the current stream (clock settle)."""
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(torch.cuda.current_stream())
    while True:
        for _ in range(chunk):
            fn()
        w1.record(torch.cuda.current_stream())
        w1.synchronize()
        if w0.elapsed_time(w1) >= ms:
            return


def leg_forward(fa, torch, steps, warmup, name, seed, B, H, H_kv, N, d, causal):
    """The step: one fa_fwd over the headline workload.

    After a >= 30 ms clock settle and `warmup` untimed steps, `steps` steps run between
    one pair of HIP events on the launch stream, with a device synchronisation on both
    sides; one launch per step, so the step time is also the kernel's average launch time.
    """
    Q, K, V = fwd_inputs(seed, B, H, H_kv, N, d)
    q, k, v = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse)

    settle(torch, step)
    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    fl = fwd_flops(B, H, N, N, d, causal)
    return {
        "step_ms": step_ms, "wall_ms_per_step": wall * 1e3 / steps, "flops": fl,
        "tflops": fl / (step_ms * 1e-3) / 1e12,
        # Q, K, V read once, O written once (bf16), LSE written once (fp32)
        "bytes": 2.0 * (2 * B * H * N * d + 2 * B * H_kv * N * d) + 4.0 * B * H * N,
    }


def leg_forward_other(fa, torch, reps, name, seed, B, H, H_kv, N, d, causal, poly_exp2=0):
    Q, K, V = fwd_inputs(seed, B, H, H_kv, N, d)
    q, k, v = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    # Warm up for at least 30 ms of GPU time, so the clock has settled (it dips for about
    # 10 ms after sustained load starts) before the timed launches; then `reps` back-to-back
    # launches between one event pair.
    settle(torch, lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse, poly_exp2=poly_exp2))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fa.fwd(q, k, v, causal=causal, out=o, lse=lse, poly_exp2=poly_exp2)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = fwd_flops(B, H, N, N, d, causal)
    return {"workload": name, "us": ms * 1e3, "tflops": fl / (ms * 1e-3) / 1e12,
            "pct_peak": 100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bwd_flops(B, H, N_q, N_k, d, causal):
    """Five N_q x N_k x d products (S recomputed, dV, dP, dQ, dK), halved under the causal mask."""
    return 5.0 * 2.0 * B * H * N_q * N_k * d / (2.0 if causal else 1.0)


def leg_backward(fa, torch, reps, B=16, H=16, H_kv=16, N=1024, seed=2):
    """fa_bwd (dQ kernel with D = rowsum(dO * O), then the dK/dV kernel) on the batched-prefill shape, O and LSE
    from fa_fwd on the same inputs; d = 64 with and without the causal mask, d = 128 without."""
    import gen

    res = {}
    for d, causal in ((64, False), (64, True), (128, False)):
        Q, K, V = fwd_inputs(seed, B, H, H_kv, N, d)
        q, k, v = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
        do = dev_bf16(gen.normal_bf16(seed, gen.TENSOR_DO, (B, H, N, d)))
        o, lse = fa.fwd(q, k, v, causal=causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(B * H * N, dtype=torch.float32, device="cuda")
        call = lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws)
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(torch.cuda.current_stream())
        while True:  # >= 30 ms of GPU time first, past the clock dip
            for _ in range(5):
                call()
            w1.record(torch.cuda.current_stream())
            w1.synchronize()
            if w0.elapsed_time(w1) >= 30.0:
                break
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        stream = torch.cuda.current_stream()
        ev[0].record(stream)
        for i in range(reps):
            call()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        times = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
        ms = sum(times) / reps
        fl = bwd_flops(B, H, N, N, d, causal)
        res["d=%d %s" % (d, "causal" if causal else "non-causal")] = {
            "us": round(ms * 1e3, 2), "us_min": round(times[0] * 1e3, 2),
            "tflops_5_products": round(fl / (ms * 1e-3) / 1e12, 1),
            "pct_bf16_peak": round(100.0 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        del q, k, v, do, o, lse, dq, dk, dv, ws
    return {"workload": "backward B=16 H=16 N_q=N_k=1024 bf16 (dO seeded N(0,1))", "flops_convention":
            "5 * 2*B*H*N_q*N_k*d, halved under the causal mask (the backward's five products)", "runs": res}


def leg_fp8(fa, torch, reps):
    """FP8 path: fa_fp8_quantize (HBM-bound: bf16 Q, K, V read, e4m3 codes written) and
    fa_fwd_fp8 (fp8 matrix cores) on the batched-prefill shape (both masks) and the
    long-sequence causal shape; the same nominal flops as the bf16 forward."""
    import gen

    runs = {}
    for name, seed, B, H, N, d, causal in (("batched prefill d=64 non-causal", 2, 16, 16, 1024, 64, False),
                                           ("batched prefill d=64 causal", 2, 16, 16, 1024, 64, True),
                                           ("long causal B=2 H=16 N=8192 d=128", 3, 2, 16, 8192, 128, True)):
        Q, K, V = fwd_inputs(seed, B, H, H, N, d)
        q, k, v = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
        lo, hi = (int(w) for w in gen.words(seed, 4, 0, 2))
        g = fa.fp8_quantize(q, k, v, lo, hi, True)
        o, lse = fa.fwd_fp8(*g, causal=causal)
        stream = torch.cuda.current_stream()

        def timed(fn):
            w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            w0.record(stream)
            while True:  # >= 30 ms first
                for _ in range(10):
                    fn()
                w1.record(stream)
                w1.synchronize()
                if w0.elapsed_time(w1) >= 30.0:
                    break
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(stream)
            for i in range(reps):
                fn()
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(reps)) / reps

        t_q = timed(lambda: fa.fp8_quantize(q, k, v, lo, hi, True))
        t_f = timed(lambda: fa.fwd_fp8(*g, causal=causal, out=o, lse=lse))
        fl = fwd_flops(B, H, N, N, d, causal)
        qbytes = 3.0 * B * H * N * d * 2 + 3.0 * B * H * N * d + 4.0 * (B * H * (-(-N // 128)) + 2 * B * H * (-(-N // 64)))
        runs[name] = {"fwd_us": round(t_f * 1e3, 2), "fwd_tflops": round(fl / (t_f * 1e-3) / 1e12, 1),
                      "pct_fp8_peak": round(100.0 * fl / (t_f * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2),
                      "quantize_us": round(t_q * 1e3, 2), "quantize_GBs": round(qbytes / (t_q * 1e-3) / 1e9, 1),
                      "quantize_pct_hbm_peak": round(100.0 * qbytes / (t_q * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        del q, k, v, g, o, lse
    return {"workload": "e4m3 forward with random-sign Hadamard transform, per-block scales (128 query rows, "
                        "64 keys)", "peak_fp8_tflops": PEAK_FP8_TFLOPS, "runs": runs}


def leg_decode(fa, torch, reps, N_k, seed, B=4, H=32, H_kv=8, d=128, num_splits=None):
    import gen

    Q = gen.normal_bf16(seed, gen.TENSOR_Q, (B, H, d), 3.0)
    K = gen.normal_bf16(seed, gen.TENSOR_K, (B, H_kv, N_k, d))
    V = gen.normal_bf16(seed, gen.TENSOR_V, (B, H_kv, N_k, d))
    q, k, v = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    del K, V
    S = num_splits or fa.decode_num_splits(B, H_kv, N_k, d)
    o_part = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
    l_part = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    kv_bytes = 2.0 * B * H_kv * N_k * d * 2
    # Before every timed repetition, sweep-read 640 MB so the 256 MB last-level cache holds
    # other (clean) lines and K/V come from HBM.  A read sweep, not a write: dirty lines
    # would be written back during the decode kernel and steal its bandwidth.
    flush = torch.ones(640 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fa.decode_split(q, k, v, S, o_part=o_part, lse_part=l_part)
        fa.combine(o_part, l_part, out=o, lse=lse)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for i in range(reps):
        torch.amax(flush)
        evs[i][0].record(stream)
        fa.decode_split(q, k, v, S, o_part=o_part, lse_part=l_part)
        evs[i][1].record(stream)
        fa.combine(o_part, l_part, out=o, lse=lse)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    split = sorted(e[0].elapsed_time(e[1]) for e in evs)
    comb = sorted(e[1].elapsed_time(e[2]) for e in evs)
    both = sorted(e[0].elapsed_time(e[2]) for e in evs)
    # The split kernel's own duration: back-to-back launches between one event pair, each
    # on the next of n_copies copies of the cache, so that the bytes read between two uses
    # of a copy ((n_copies - 1) * kv_bytes >= 640 MB) exceed the 256 MB last-level cache
    # and every launch reads K/V from HBM.  Per-repetition event pairs (above) also time
    # the gap between an event and the launch, several microseconds on this runtime.
    n_copies = max(2, int(math.ceil(640e6 / kv_bytes)) + 1)
    kc = [k] + [k.clone() for _ in range(n_copies - 1)]
    vc = [v] + [v.clone() for _ in range(n_copies - 1)]
    n_b2b = max(2 * n_copies, 8 * reps if N_k <= 8192 else reps)
    for i in range(2 * n_copies):
        fa.decode_split(q, kc[i % n_copies], vc[i % n_copies], S, o_part=o_part, lse_part=l_part)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(n_b2b):
        fa.decode_split(q, kc[i % n_copies], vc[i % n_copies], S, o_part=o_part, lse_part=l_part)
    b1.record(stream)
    torch.cuda.synchronize()
    b2b_ms = b0.elapsed_time(b1) / n_b2b
    # split + combine, timed the same way
    b0.record(stream)
    for i in range(n_b2b):
        fa.decode_split(q, kc[i % n_copies], vc[i % n_copies], S, o_part=o_part, lse_part=l_part)
        fa.combine(o_part, l_part, out=o, lse=lse)
    b1.record(stream)
    torch.cuda.synchronize()
    both_b2b_ms = b0.elapsed_time(b1) / n_b2b
    # Split and merge in one launch (fa_decode), timed the same way.  The first call goes
    # through the checked binding; the timed loop calls the C entry point with the same
    # arguments so that the host cost of the checks stays out of a ~15 us launch interval.
    counters = torch.zeros((max(1, fa.decode_counter_bytes(B, H, H_kv) // 4),), dtype=torch.int32, device="cuda")
    fa.decode(q, k, v, S, counters=counters, o_part=o_part, lse_part=l_part, out=o, lse=lse)
    lib, sptr, scale = fa.library(), torch.cuda.current_stream().cuda_stream, 1.0 / math.sqrt(d)
    fused_args = [(q.data_ptr(), kc[i].data_ptr(), vc[i].data_ptr(), o_part.data_ptr(), l_part.data_ptr(),
                   counters.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, H_kv, N_k, d, S, scale, sptr)
                  for i in range(n_copies)]
    for i in range(2 * n_copies):
        assert lib.fa_decode(*fused_args[i % n_copies]) == 0
    b0.record(stream)
    for i in range(n_b2b):
        lib.fa_decode(*fused_args[i % n_copies])
    b1.record(stream)
    torch.cuda.synchronize()
    fused_b2b_ms = b0.elapsed_time(b1) / n_b2b
    assert int(counters.abs().sum()) == 0, "fa_decode left a group counter non-zero"
    del kc, vc
    # For comparison (information only): the unsplit forward with N_q = 1 on the same shapes,
    # one workgroup per (b, h), reading each K/V head once per query head of its group.
    q4 = q.view(B, H, 1, d)
    o4 = torch.empty_like(q4)
    lse4 = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    fa.fwd(q4, k, v, causal=False, out=o4, lse=lse4)
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        torch.amax(flush)
        evf[i][0].record(stream)
        fa.fwd(q4, k, v, causal=False, out=o4, lse=lse4)
        evf[i][1].record(stream)
    torch.cuda.synchronize()
    unsplit_ms = sum(e[0].elapsed_time(e[1]) for e in evf) / reps
    # Paged cache (16-token pages, shuffled over the pool, every sequence full length): the
    # same split through a block table.
    P = 16
    npp = N_k // P
    perm = torch.randperm(B * npp, generator=torch.Generator().manual_seed(seed)).cuda()
    def to_pages(x):  # [B,H_kv,N_k,d] -> pool [B*npp, H_kv, P, d], logical page i of b at perm[b*npp+i]
        logical = x.view(B, H_kv, npp, P, d).permute(0, 2, 1, 3, 4).reshape(B * npp, H_kv, P, d)
        pool = torch.empty_like(logical)
        pool[perm] = logical
        return pool
    kp, vp = to_pages(k), to_pages(v)
    table = perm.view(B, npp).to(torch.int32).contiguous()
    lens = torch.full((B,), N_k, dtype=torch.int32, device="cuda")
    fa.decode_split_paged(q, kp, vp, table, lens, S, o_part=o_part, lse_part=l_part)
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for i in range(reps):
        torch.amax(flush)
        evp[i][0].record(stream)
        fa.decode_split_paged(q, kp, vp, table, lens, S, o_part=o_part, lse_part=l_part)
        evp[i][1].record(stream)
    torch.cuda.synchronize()
    paged_ms = sum(e[0].elapsed_time(e[1]) for e in evp) / reps
    # the paged split + combine, and fa_decode_paged (both in one launch), timed the same way
    for i in range(reps):
        torch.amax(flush)
        evp[i][0].record(stream)
        fa.decode_split_paged(q, kp, vp, table, lens, S, o_part=o_part, lse_part=l_part)
        fa.combine(o_part, l_part, out=o, lse=lse)
        evp[i][1].record(stream)
    torch.cuda.synchronize()
    paged_both_ms = sum(e[0].elapsed_time(e[1]) for e in evp) / reps
    fa.decode_paged(q, kp, vp, table, lens, S, counters=counters, o_part=o_part, lse_part=l_part, out=o, lse=lse)
    for i in range(reps):
        torch.amax(flush)
        evp[i][0].record(stream)
        fa.decode_paged(q, kp, vp, table, lens, S, counters=counters, o_part=o_part, lse_part=l_part, out=o, lse=lse)
        evp[i][1].record(stream)
    torch.cuda.synchronize()
    paged_fused_ms = sum(e[0].elapsed_time(e[1]) for e in evp) / reps
    del kp, vp
    ms_rep = sum(split) / reps
    gbs = kv_bytes / (b2b_ms * 1e-3) / 1e9
    return {"N_k": N_k, "num_splits": S, "split_us": b2b_ms * 1e3,
            "split_timing": "back-to-back launches over %d rotated cache copies (%d launches, one event pair)"
                            % (n_copies, n_b2b),
            "split_us_per_rep": ms_rep * 1e3, "split_us_per_rep_median": split[reps // 2] * 1e3,
            "split_per_rep_GBs": kv_bytes / (ms_rep * 1e-3) / 1e9,
            "paged16_split_us": paged_ms * 1e3, "paged16_timing": "per repetition after a read sweep", "paged16_split_GBs": kv_bytes / (paged_ms * 1e-3) / 1e9,
            "paged16_end_to_end_us": paged_both_ms * 1e3, "paged16_one_launch_us": paged_fused_ms * 1e3,
            "unsplit_fwd_us": unsplit_ms * 1e3, "unsplit_fwd_GBs": kv_bytes / (unsplit_ms * 1e-3) / 1e9,
            "combine_us": sum(comb) / reps * 1e3, "end_to_end_us": sum(both) / reps * 1e3,
            "end_to_end_b2b_us": both_b2b_ms * 1e3, "fused_b2b_us": fused_b2b_ms * 1e3,
            "fused_GBs": kv_bytes / (fused_b2b_ms * 1e-3) / 1e9,
            "split_GBs": gbs, "split_pct_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS,
            "end_to_end_GBs": kv_bytes / (sum(both) / reps * 1e-3) / 1e9, "kv_bytes": kv_bytes}


def leg_copy(torch, reps=5, mib=1024):
    """A plain device copy of known size (calibrates the HBM byte counters)."""
    a = torch.empty(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"copy_bytes_each_way": a.numel() * 4, "reps": reps}


def cpu_baseline(target_s=12.0):
    """The fp64 oracle on whole (batch, head) slices of the headline workload, one slice at a
    time until about target_s (every slice of the causal workload carries the same work)."""
    import numpy as np

    import oracle

    w = HEADLINE
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    Q, K, V = fwd_inputs(w["seed"], B, H, w["H_kv"], N, d)
    orc = oracle.Oracle()
    threads = oracle.host_threads()
    slice_flops = fwd_flops(1, 1, N, N, d, w["causal"])
    n, elapsed = 0, 0.0
    while n < B * H and (n == 0 or elapsed / n * (n + 1) <= target_s):
        rows = np.arange(n * N, (n + 1) * N, dtype=np.int64)
        t0 = time.perf_counter()
        orc.attention(Q, K, V, causal=w["causal"], rows=rows, nthreads=threads)
        elapsed += time.perf_counter() - t0
        n += 1
    return {"value": slice_flops * n / elapsed / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": "%d of %d (batch, head) slices of the long causal workload (N=8192, d=128), every row, "
                      "fp64, %.1f s" % (n, B * H, elapsed),
            "seconds": elapsed}


def traffic_from_counters(dominant_kernel_substr):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if the kernel is unchanged."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, "no counter summary"
    for name, k in c.get("kernels", {}).items():
        if dominant_kernel_substr in name:
            if k.get("source_hash") != kernel_source_hash(name):
                return None, "kernel changed since the counters were taken"
            return k.get("hbm_bytes_per_launch"), "profiles/hbm_counters.json (%s)" % name
    return None, "dominant kernel not in the counter summary"


def shader_counters(dominant_kernel_substr):
    """MFMA busy and LDS bank conflicts per launch from the committed shader-counter summary,
    if the kernel is unchanged (None otherwise)."""
    try:
        with open(SQ_COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    for name, k in c.get("kernels", {}).items():
        if dominant_kernel_substr in name:
            if k.get("source_hash") != kernel_source_hash(name):
                return None
            return dict(k, source="profiles/sq_counters.json (%s)" % name)
    return None


# ---------------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--legs", default="fwd,fwd_other,decode,bwd,fp8,poly,cpu",
                    help="comma list of fwd (the headline step), fwd_other (the batched-prefill and grouped-query "
                         "forward workloads), decode, bwd, fp8, poly (the forward with polynomial exponentials), "
                         "cpu, copy")
    ap.add_argument("--all", action="store_true", help="add fwd_other to --legs")
    ap.add_argument("--decode-reps", type=int, default=30)
    ap.add_argument("--decode-nk", default="4096,65536", help="comma list of decode cache lengths")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU's share is the "
              "single-GPU kernel at its real shape; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_59_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.library()
    torch.cuda.set_device(0)
    legs = set(args.legs.split(","))
    w = HEADLINE
    T_r = -(-w["N"] // 128)
    head_grid = ((T_r + 1) // 2 if w["causal"] else T_r) * w["B"] * w["H"] * 256  # work-items of one launch
    head_kernel = "fwd_kernel<%d, %s>" % (w["d"], "true" if w["causal"] else "false")
    out = {"metric": METRIC, "value": None, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w["name"] + (", causal" if w["causal"] else ""), "global_batch": w["B"],
                      "seq_len": w["N"], "heads": w["H"], "kv_heads": w["H_kv"], "head_dim": w["d"],
                      "causal": w["causal"], "parallelism": "single GPU"}}

    if "copy" in legs:
        log("copy leg", leg_copy(torch))

    if "fwd" in legs:
        log("forward leg: >= 30 ms settle + %d warmup + %d timed steps" % (args.warmup, args.steps))
        r = leg_forward(fa, torch, args.steps, args.warmup, w["name"], w["seed"], w["B"], w["H"], w["H_kv"],
                        w["N"], w["d"], w["causal"])
        out["value"] = round(r["tflops"], 2)
        out["ms_per_step"] = round(r["step_ms"], 4)
        out["pct_bf16_peak"] = round(100.0 * r["tflops"] / PEAK_BF16_TFLOPS, 2)
        out["config"]["kernel_avg_us"] = round(r["step_ms"] * 1e3, 2)
        out["config"]["wall_ms_per_step"] = round(r["wall_ms_per_step"], 4)
        traffic, src = traffic_from_counters("%s grid=%d" % (head_kernel, head_grid))
        out["roofline"] = {"kernel": "%s (%s)" % (head_kernel, w["name"]), "bound": "mfma",
                           "achieved": round(r["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                           "traffic_source": src, "avg_launch_us": round(r["step_ms"] * 1e3, 2),
                           "algorithmic_flops_per_launch": r["flops"],
                           "algorithmic_bytes_per_launch": r["bytes"],
                           "traffic_over_algorithmic": (round(traffic / r["bytes"], 3) if traffic else None),
                           "counters": shader_counters("%s grid=%d" % (head_kernel, head_grid))}
        log("forward", out["roofline"])

    if "fwd_other" in legs or args.all:
        others = [("batched prefill B=16 H=16 N=1024 d=64 non-causal", 2, 16, 16, 16, 1024, 64, False),
                  ("batched prefill B=16 H=16 N=1024 d=64 causal", 2, 16, 16, 16, 1024, 64, True),
                  ("GQA ragged causal B=4 H=32 H_kv=8 N=4095 d=128", 4, 4, 32, 8, 4095, 128, True),
                  ("batched prefill B=16 H=16 N=1024 d=128 non-causal", 2, 16, 16, 16, 1024, 128, False)]
        out["forward_workloads"] = []
        for name, seed, B, H, H_kv, N, d, causal in others:
            log("forward", name)
            out["forward_workloads"].append({k: (round(v, 2) if isinstance(v, float) else v) for k, v in
                                             leg_forward_other(fa, torch, 50, name, seed, B, H, H_kv, N, d,
                                                               causal).items()})
            torch.cuda.empty_cache()

    if "poly" in legs:
        # fa_fwd_poly_exp2: a quarter, half or all of the softmax exponentials on the FMA units
        out["fwd_poly_exp2"] = []
        for name, seed, B, H, H_kv, N, d, causal in (
                ("batched prefill B=16 H=16 N=1024 d=64 non-causal", 2, 16, 16, 16, 1024, 64, False),
                ("long causal B=2 H=16 N=8192 d=128", 3, 2, 16, 16, 8192, 128, True)):
            base = leg_forward_other(fa, torch, 50, name, seed, B, H, H_kv, N, d, causal)
            rec = {"workload": name, "exact_exp2_us": round(base["us"], 2)}
            for qu in (1, 2, 4):
                r = leg_forward_other(fa, torch, 50, name, seed, B, H, H_kv, N, d, causal, poly_exp2=qu)
                rec["poly_%d_of_4_us" % qu] = round(r["us"], 2)
                rec["poly_%d_of_4_vs_exact" % qu] = round(r["us"] / base["us"], 3)
            log("poly exp2", rec)
            out["fwd_poly_exp2"].append(rec)
            torch.cuda.empty_cache()

    if "decode" in legs:
        dec = {}
        for N_k, seed in ((4096, 5), (65536, 6)):
            if str(N_k) not in args.decode_nk.split(","):
                continue
            log("decode leg N_k=%d" % N_k)
            dec["N_k=%d" % N_k] = {k: (round(v, 2) if isinstance(v, float) else v)
                                   for k, v in leg_decode(fa, torch, args.decode_reps, N_k, seed).items()}
            log("decode", dec["N_k=%d" % N_k])
            torch.cuda.empty_cache()
        out["decode"] = dec

    if "bwd" in legs:
        log("backward leg")
        out["backward"] = leg_backward(fa, torch, 30)
        log("backward", out["backward"])
        torch.cuda.empty_cache()

    if "fp8" in legs:
        log("fp8 leg")
        out["fp8"] = leg_fp8(fa, torch, 30)
        log("fp8", out["fp8"])
        torch.cuda.empty_cache()

    if "cpu" in legs:
        log("cpu baseline (oracle, ~%.0f s)" % args.cpu_seconds)
        cb = cpu_baseline(args.cpu_seconds)
        out["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cb.items()}

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
