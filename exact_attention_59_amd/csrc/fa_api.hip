// fa_api.hip -- the C ABI declared in include/fa.h: argument validation (before any
// HIP call), dispatch to the gfx950 kernels, and the host-side helpers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool debug_enabled() {
    static const bool on = [] {
        const char* v = getenv("FA_DEBUG");
        return v && v[0] && v[0] != '0';
    }();
    return on;
}

int finish(hipError_t err, const char* what) {
    if (err != hipSuccess) {
        if (debug_enabled()) fprintf(stderr, "[fa] %s launch failed: %s\n", what, hipGetErrorString(err));
        return FA_ERR_HIP;
    }
    return FA_OK;
}

// Largest element count of one tensor we accept (offsets are 64-bit inside the kernels;
// grid sizes are checked separately).
constexpr long long kMaxElems = 1LL << 62;

int compute_units() {
    static std::once_flag once;
    static int cus = 256;
    std::call_once(once, [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        (void)hipGetLastError();  // a machine without a GPU leaves an error behind; clear it
    });
    return cus;
}

}  // namespace

FA_EXPORT const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (a size <= 0, H not a multiple of H_kv, or num_splits outside [1, N_k])";
        case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dimension must be 64 or 128, or a size exceeds the limits)";
        case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case FA_ERR_ARG: return "invalid argument (scale not finite and positive, or a flag not 0/1)";
        case FA_ERR_HIP: return "the HIP runtime reported an error while enqueueing";
        case FA_ERR_CAPACITY: return "the problem needs more than fa_decode_static's static scratch array holds (16 MiB: counters, LSE_part and O_part)";
        default: return "unknown status";
    }
}

FA_EXPORT int fa_fwd_tile_shape(int d, int* block_rows, int* block_cols) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (block_rows) *block_rows = fa::fwd_block_rows(d);
    if (block_cols) *block_cols = fa::fwd_block_cols(d);
    return FA_OK;
}

// Mirrors the kernel's loop bounds: query tile i walks key tiles 0 .. n_i - 1, where
// n_i stops at the last key visible to the tile's last real row.
FA_EXPORT long long fa_fwd_tile_count(int N_q, int N_k, int d, int causal) {
    if (N_q <= 0 || N_k <= 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1)) return -1;
    const long long BR = fa::fwd_block_rows(d), BC = fa::fwd_block_cols(d);
    const long long T_r = (N_q + BR - 1) / BR, T_c = (N_k + BC - 1) / BC;
    if (!causal) return T_r * T_c;
    long long total = 0;
    for (long long i = 0; i < T_r; ++i) {
        const long long last_row = (i * BR + BR < N_q ? i * BR + BR : N_q) - 1;
        const long long kl = last_row + (N_k - N_q);
        if (kl >= 0) total += (kl / BC + 1 < T_c) ? kl / BC + 1 : T_c;
    }
    return total;
}

// Checks shared by the two forward entry points; *blocks gets the launch's workgroup count.
static int check_fwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE, int B, int H,
                     int H_kv, int N_q, int N_k, int d, int causal, float scale, long long* blocks_out) {
    if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N_q * d >= kMaxElems || (long long)B * H_kv * N_k * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long blocks = (long long)((N_q + fa::fwd_block_rows(d) - 1) / fa::fwd_block_rows(d)) * B * H;
    if (blocks > 0x7fffffffLL || (long long)B * H > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) || misaligned(LSE)) return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    *blocks_out = blocks;
    return FA_OK;
}

FA_EXPORT int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int H_kv,
                     int N_q, int N_k, int d, int causal, float scale, void* stream) {
    long long blocks = 0;
    const int st = check_fwd(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, &blocks);
    if (st != FA_OK) return st;
    if (debug_enabled())
        fprintf(stderr, "[fa] fwd B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d causal=%d blocks=%lld\n", B, H, H_kv, N_q,
                N_k, d, causal, blocks);
    return finish(fa::launch_fwd(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal == 1, scale,
                                 static_cast<hipStream_t>(stream)),
                  "fa_fwd");
}

FA_EXPORT int fa_fwd_poly_exp2(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                               int H_kv, int N_q, int N_k, int d, int causal, float scale, int poly_quarters,
                               void* stream) {
    long long blocks = 0;
    const int st = check_fwd(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, &blocks);
    if (st != FA_OK) return st;
    if (poly_quarters != 1 && poly_quarters != 2 && poly_quarters != 4) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] fwd_poly_exp2 B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d causal=%d quarters=%d\n", B, H,
                H_kv, N_q, N_k, d, causal, poly_quarters);
    return finish(fa::launch_fwd_poly(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal == 1, scale, poly_quarters,
                                      static_cast<hipStream_t>(stream)),
                  "fa_fwd_poly_exp2");
}

FA_EXPORT int fa_exp2_poly(const float* x, float* y, long long n, void* stream) {
    if (!x || !y) return FA_ERR_NULL;
    if (n < 0) return FA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(y) & 3u)) return FA_ERR_ALIGN;
    if (n == 0) return FA_OK;
    return finish(fa::launch_exp2_poly(x, y, n, static_cast<hipStream_t>(stream)), "fa_exp2_poly");
}

FA_EXPORT int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                     void* dQ, void* dK, void* dV, float* workspace, int B, int H, int H_kv, int N_q, int N_k, int d,
                     int causal, float scale, void* stream) {
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !workspace) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N_q * d >= kMaxElems || (long long)B * H_kv * N_k * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long q_blocks = (long long)((N_q + fa::kBwdBlockRows - 1) / fa::kBwdBlockRows) * B * H;
    const long long k_blocks = (long long)((N_k + fa::kBwdBlockKeys - 1) / fa::kBwdBlockKeys) * B * H_kv;
    if (q_blocks > 0x7fffffffLL || k_blocks > 0x7fffffffLL || (long long)B * H * N_q / 16 > 0x7fffffffLL)
        return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) || misaligned(dO) || misaligned(LSE) ||
        misaligned(dQ) || misaligned(dK) || misaligned(dV) || misaligned(workspace))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] bwd B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d causal=%d\n", B, H, H_kv, N_q, N_k, d, causal);
    return finish(fa::launch_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, H_kv, N_q, N_k, d, causal == 1,
                                 scale, static_cast<hipStream_t>(stream)),
                  "fa_bwd");
}

FA_EXPORT size_t fa_bwd_workspace_bytes(int B, int H, int N_q) {
    if (B <= 0 || H <= 0 || N_q <= 0) return 0;
    return (size_t)B * H * N_q * sizeof(float);
}

FA_EXPORT int fa_fp8_block_rows(int* q_rows, int* kv_rows) {
    if (q_rows) *q_rows = fa::kFp8QRows;
    if (kv_rows) *kv_rows = fa::kFp8KRows;
    return FA_OK;
}

FA_EXPORT int fa_fp8_quantize(const void* Q, const void* K, const void* V, int incoherent, uint64_t sign_lo,
                              uint64_t sign_hi, void* Q8, void* K8, void* Vt8, float* q_scale, float* k_scale,
                              float* v_scale, int B, int H, int H_kv, int N_q, int N_k, int d, void* stream) {
    if (!Q || !K || !V || !Q8 || !K8 || !Vt8 || !q_scale || !k_scale || !v_scale) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N_q * d >= kMaxElems || (long long)B * H_kv * (N_k + fa::kFp8KRows) * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long tq = (N_q + fa::kFp8QRows - 1) / fa::kFp8QRows, tk = (N_k + fa::kFp8KRows - 1) / fa::kFp8KRows;
    if ((long long)B * H * tq + 2LL * B * H_kv * tk > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(Q8) || misaligned(K8) || misaligned(Vt8) ||
        (reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(v_scale) & 3u))
        return FA_ERR_ALIGN;
    if (incoherent != 0 && incoherent != 1) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] fp8_quantize B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d incoherent=%d\n", B, H, H_kv, N_q, N_k,
                d, incoherent);
    return finish(fa::launch_fp8_quantize(Q, K, V, incoherent, sign_lo, sign_hi, Q8, K8, Vt8, q_scale, k_scale,
                                          v_scale, B, H, H_kv, N_q, N_k, d, static_cast<hipStream_t>(stream)),
                  "fa_fp8_quantize");
}

FA_EXPORT int fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
                         const float* v_scale, void* O, float* LSE, int B, int H, int H_kv, int N_q, int N_k, int d,
                         int causal, float scale, void* stream) {
    if (!Q8 || !K8 || !Vt8 || !q_scale || !k_scale || !v_scale || !O || !LSE) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * N_q * d >= kMaxElems || (long long)B * H_kv * (N_k + fa::kFp8KRows) * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long blocks = (long long)((N_q + fa::kFp8QRows - 1) / fa::kFp8QRows) * B * H;
    if (blocks > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q8) || misaligned(K8) || misaligned(Vt8) || misaligned(O) || misaligned(LSE) ||
        (reinterpret_cast<uintptr_t>(q_scale) & 3u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(v_scale) & 3u))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] fwd_fp8 B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d causal=%d\n", B, H, H_kv, N_q, N_k, d, causal);
    return finish(fa::launch_fwd_fp8(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, H_kv, N_q, N_k, d,
                                     causal == 1, scale, static_cast<hipStream_t>(stream)),
                  "fa_fwd_fp8");
}

FA_EXPORT int fa_decode_split(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                              int B, int H, int H_kv, int N_k, int d, int num_splits, float scale,
                              void* stream) {
    if (!Q || !K || !V || !O_part || !LSE_part) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (num_splits < 1 || num_splits > N_k) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (H / H_kv > 4 * fa::kDecHeadsPerBlock) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H_kv * N_k * d >= kMaxElems || (long long)B * H * num_splits * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long n_qc = (H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock;
    if ((long long)num_splits * n_qc * B * H_kv > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O_part) || misaligned(LSE_part))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] decode_split B=%d H=%d H_kv=%d N_k=%d d=%d S=%d\n", B, H, H_kv, N_k, d, num_splits);
    return finish(fa::launch_decode_split(Q, K, V, O_part, LSE_part, B, H, H_kv, N_k, d, num_splits, scale,
                                          static_cast<hipStream_t>(stream)),
                  "fa_decode_split");
}

// Checks shared by the two paged entry points; sets *page_log2 on success.
static int check_paged(const void* Q, const void* K_pages, const void* V_pages, const int* block_table,
                       const int* seq_lens, const float* O_part, const float* LSE_part, int B, int H, int H_kv,
                       int page_size, int max_pages, int num_pages, int d, int num_splits, float scale,
                       int* page_log2) {
    if (!Q || !K_pages || !V_pages || !block_table || !seq_lens || !O_part || !LSE_part) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || page_size <= 0 || max_pages <= 0 || num_pages <= 0 || d <= 0)
        return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    const long long max_tokens = (long long)max_pages * page_size;
    if (num_splits < 1 || num_splits > max_tokens) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (H / H_kv > 4 * fa::kDecHeadsPerBlock) return FA_ERR_UNSUPPORTED;
    int lg = 0;
    while ((1 << lg) < page_size && lg < 30) ++lg;
    if ((1 << lg) != page_size || page_size < 16 || page_size > 4096) return FA_ERR_UNSUPPORTED;
    if (max_tokens > 0x7fffffffLL || (long long)B * max_pages > 0x7fffffffLL ||
        (long long)num_pages * H_kv * page_size * d >= kMaxElems || (long long)B * H * num_splits * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long n_qc = (H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock;
    if ((long long)num_splits * n_qc * B * H_kv > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K_pages) || misaligned(V_pages) || misaligned(O_part) || misaligned(LSE_part) ||
        (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    *page_log2 = lg;
    return FA_OK;
}

FA_EXPORT int fa_decode_split_paged(const void* Q, const void* K_pages, const void* V_pages,
                                    const int* block_table, const int* seq_lens, float* O_part,
                                    float* LSE_part, int B, int H, int H_kv, int page_size, int max_pages,
                                    int num_pages, int d, int num_splits, float scale, void* stream) {
    int page_log2 = 0;
    const int rc = check_paged(Q, K_pages, V_pages, block_table, seq_lens, O_part, LSE_part, B, H, H_kv, page_size,
                               max_pages, num_pages, d, num_splits, scale, &page_log2);
    if (rc != FA_OK) return rc;
    if (debug_enabled())
        fprintf(stderr, "[fa] decode_split_paged B=%d H=%d H_kv=%d P=%d max_pages=%d num_pages=%d d=%d S=%d\n", B, H,
                H_kv, page_size, max_pages, num_pages, d, num_splits);
    return finish(fa::launch_decode_split_paged(Q, K_pages, V_pages, block_table, seq_lens, O_part, LSE_part, B, H,
                                                H_kv, page_log2, max_pages, num_pages, d, num_splits, scale,
                                                static_cast<hipStream_t>(stream)),
                  "fa_decode_split_paged");
}

FA_EXPORT int fa_decode_paged(const void* Q, const void* K_pages, const void* V_pages, const int* block_table,
                              const int* seq_lens, float* O_part, float* LSE_part, int* counters, void* O,
                              float* LSE, int B, int H, int H_kv, int page_size, int max_pages, int num_pages,
                              int d, int num_splits, float scale, void* stream) {
    if (!counters || !O) return FA_ERR_NULL;
    int page_log2 = 0;
    const int rc = check_paged(Q, K_pages, V_pages, block_table, seq_lens, O_part, LSE_part, B, H, H_kv, page_size,
                               max_pages, num_pages, d, num_splits, scale, &page_log2);
    if (rc != FA_OK) return rc;
    if (misaligned(O) || (LSE && misaligned(LSE)) || (reinterpret_cast<uintptr_t>(counters) & 3u))
        return FA_ERR_ALIGN;
    if (debug_enabled())
        fprintf(stderr, "[fa] decode_paged (fused) B=%d H=%d H_kv=%d P=%d max_pages=%d num_pages=%d d=%d S=%d\n", B,
                H, H_kv, page_size, max_pages, num_pages, d, num_splits);
    return finish(fa::launch_decode_paged_fused(Q, K_pages, V_pages, block_table, seq_lens, O_part, LSE_part,
                                                counters, O, LSE, B, H, H_kv, page_log2, max_pages, num_pages, d,
                                                num_splits, scale, static_cast<hipStream_t>(stream)),
                  "fa_decode_paged");
}

FA_EXPORT int fa_combine(const float* O_part, const float* LSE_part, void* O, float* LSE, int B, int H, int d,
                         int num_splits, void* stream) {
    if (!O_part || !LSE_part || !O) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || d <= 0 || num_splits < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * num_splits * d >= kMaxElems || (long long)B * H > 0x7fffffffLL)
        return FA_ERR_UNSUPPORTED;
    if (misaligned(O_part) || misaligned(LSE_part) || misaligned(O) || (LSE && misaligned(LSE)))
        return FA_ERR_ALIGN;
    if (debug_enabled()) fprintf(stderr, "[fa] combine B=%d H=%d d=%d S=%d\n", B, H, d, num_splits);
    return finish(fa::launch_combine(O_part, LSE_part, O, LSE, B, H, d, num_splits,
                                     static_cast<hipStream_t>(stream)),
                  "fa_combine");
}

// Split count: aim for about two resident workgroups per compute unit in one wave of
// workgroups, but keep every segment at least 256 keys long (Lecture 11 section 6.4).
FA_EXPORT int fa_decode_num_splits(int B, int H_kv, int N_k, int d) {
    if (B <= 0 || H_kv <= 0 || N_k <= 0 || d <= 0) return 0;
    const long long heads = (long long)B * H_kv;
    const long long target = 2LL * compute_units();
    long long s = (target + heads - 1) / heads;
    const long long max_by_len = N_k / 256 > 0 ? N_k / 256 : 1;
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    if (s > N_k) s = N_k;
    return (int)s;
}

FA_EXPORT int fa_decode(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                        int* counters, void* O, float* LSE, int B, int H, int H_kv, int N_k, int d,
                        int num_splits, float scale, void* stream) {
    if (!Q || !K || !V || !O_part || !LSE_part || !counters || !O) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (num_splits < 1 || num_splits > N_k) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (H / H_kv > 4 * fa::kDecHeadsPerBlock) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H_kv * N_k * d >= kMaxElems || (long long)B * H * num_splits * d >= kMaxElems)
        return FA_ERR_UNSUPPORTED;
    const long long n_qc = (H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock;
    if ((long long)num_splits * n_qc * B * H_kv > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O_part) || misaligned(LSE_part) ||
        misaligned(O) || (LSE && misaligned(LSE)) || (reinterpret_cast<uintptr_t>(counters) & 3u))
        return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] decode (fused) B=%d H=%d H_kv=%d N_k=%d d=%d S=%d\n", B, H, H_kv, N_k, d, num_splits);
    return finish(fa::launch_decode_fused(Q, K, V, O_part, LSE_part, counters, O, LSE, B, H, H_kv, N_k, d,
                                          num_splits, scale, static_cast<hipStream_t>(stream)),
                  "fa_decode");
}

FA_EXPORT int fa_decode_static(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                               int H_kv, int N_k, int d, int num_splits, float scale, void* stream) {
    if (!Q || !K || !V || !O) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_k <= 0 || d <= 0) return FA_ERR_SHAPE;
    if (H % H_kv) return FA_ERR_SHAPE;
    if (num_splits < 1 || num_splits > N_k) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (H / H_kv > 4 * fa::kDecHeadsPerBlock) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H_kv * N_k * d >= kMaxElems) return FA_ERR_UNSUPPORTED;
    const long long n_qc = (H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock;
    if ((long long)num_splits * n_qc * B * H_kv > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    // capacity of the static scratch array: the counters and both partial arrays
    if ((long long)B * H_kv * n_qc * (long long)sizeof(int) > (long long)fa::kStaticCounterBytes ||
        (long long)B * H * num_splits * (d + 1) > (long long)(fa::kStaticScratchBytes / sizeof(float)) ||
        fa::decode_static_bytes(B, H, d, num_splits) > fa::kStaticScratchBytes)
        return FA_ERR_CAPACITY;
    if (misaligned(Q) || misaligned(K) || misaligned(V) || misaligned(O) || (LSE && misaligned(LSE))) return FA_ERR_ALIGN;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
    if (debug_enabled())
        fprintf(stderr, "[fa] decode (static scratch) B=%d H=%d H_kv=%d N_k=%d d=%d S=%d\n", B, H, H_kv, N_k, d,
                num_splits);
    return finish(fa::launch_decode_static(Q, K, V, O, LSE, B, H, H_kv, N_k, d, num_splits, scale,
                                           static_cast<hipStream_t>(stream)),
                  "fa_decode_static");
}

FA_EXPORT int fa_decode_counters_reset(int* counters, int B, int H, int H_kv, void* stream) {
    if (!counters) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv) return FA_ERR_SHAPE;
    const long long n = (long long)B * H_kv * ((H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock);
    if (n > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(counters) & 3u) return FA_ERR_ALIGN;
    return finish(fa::launch_counters_reset(counters, (int)n, static_cast<hipStream_t>(stream)),
                  "fa_decode_counters_reset");
}

FA_EXPORT int fa_decode_counters_check(const int* counters, int B, int H, int H_kv, int* nonzero, void* stream) {
    if (!counters || !nonzero) return FA_ERR_NULL;
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv) return FA_ERR_SHAPE;
    const long long n = (long long)B * H_kv * ((H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock);
    if (n > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(counters) & 3u) || (reinterpret_cast<uintptr_t>(nonzero) & 3u))
        return FA_ERR_ALIGN;
    return finish(fa::launch_counters_check(counters, (int)n, nonzero, static_cast<hipStream_t>(stream)),
                  "fa_decode_counters_check");
}

FA_EXPORT size_t fa_decode_counter_bytes(int B, int H, int H_kv) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv) return 0;
    const size_t n_qc = (size_t)(H / H_kv + fa::kDecHeadsPerBlock - 1) / fa::kDecHeadsPerBlock;
    return (size_t)B * H_kv * n_qc * sizeof(int);
}

FA_EXPORT size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
    if (B <= 0 || H <= 0 || d <= 0 || num_splits <= 0) return 0;
    const size_t rows = (size_t)B * H * num_splits;
    return rows * (size_t)d * sizeof(float) + rows * sizeof(float);
}
