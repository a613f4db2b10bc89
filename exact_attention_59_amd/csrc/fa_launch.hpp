// fa_launch.hpp -- library-internal launchers (C++ linkage, hidden); fa_api.hip calls them
// after validating arguments.  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Forward tile shape for head dimension d: waves per workgroup (each owns 32 query rows),
// query rows per workgroup, and keys per tile.
constexpr int fwd_waves(int /*d*/) { return 4; }
constexpr int fwd_block_rows(int d) { return 32 * fwd_waves(d); }
constexpr int fwd_block_cols(int /*d*/) { return 64; }

// Backward tile shapes: the dQ kernel's query rows per workgroup and keys per tile; the
// dK/dV kernel's keys per workgroup and queries per tile.
constexpr int kBwdBlockRows = 128;
constexpr int bwd_dq_block_cols(int d) { return d == 128 ? 32 : 64; }
constexpr int kBwdBlockKeys = 128;
constexpr int kBwdBlockQueries = 32;

// FP8 path: rows per quantisation block of Q (= the forward's query tile) and of K / V
// (= the forward's key tile).
constexpr int kFp8QRows = 128;
constexpr int kFp8KRows = 64;

// Decode: keys per wave iteration and query heads per workgroup.
constexpr int kDecKeysPerWave = 32;
constexpr int kDecHeadsPerBlock = 16;

hipError_t launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                      int H_kv, int N_q, int N_k, int d, bool causal, float scale, hipStream_t stream);

// The forward with poly_quarters (1, 2 or 4) of every four softmax exponentials taken by the
// FMA-unit polynomial exp2_poly instead of v_exp_f32 (any other value: launch_fwd).
hipError_t launch_fwd_poly(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                           int H_kv, int N_q, int N_k, int d, bool causal, float scale, int poly_quarters,
                           hipStream_t stream);
// y[i] = exp2_poly(x[i]) for i < n (the forward's polynomial, for its error tests).
hipError_t launch_exp2_poly(const float* x, float* y, long long n, hipStream_t stream);

// Backward: dQ (its kernel also writes D = rowsum(dO * O) into `workspace`, B*H*N_q floats),
// then dK and dV.
hipError_t launch_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                      void* dQ, void* dK, void* dV, float* workspace, int B, int H, int H_kv, int N_q, int N_k, int d,
                      bool causal, float scale, hipStream_t stream);

hipError_t launch_fp8_quantize(const void* Q, const void* K, const void* V, int transform, uint64_t sign_lo,
                               uint64_t sign_hi, void* Q8, void* K8, void* Vt8, float* q_scale, float* k_scale,
                               float* v_scale, int B, int H, int H_kv, int N_q, int N_k, int d, hipStream_t stream);

hipError_t launch_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
                          const float* v_scale, void* O, float* LSE, int B, int H, int H_kv, int N_q, int N_k, int d,
                          bool causal, float scale, hipStream_t stream);

hipError_t launch_decode_split(const void* Q, const void* K, const void* V, float* O_part,
                               float* LSE_part, int B, int H, int H_kv, int N_k, int d, int num_splits,
                               float scale, hipStream_t stream);

hipError_t launch_decode_split_paged(const void* Q, const void* K_pages, const void* V_pages,
                                     const int* block_table, const int* seq_lens, float* O_part,
                                     float* LSE_part, int B, int H, int H_kv, int page_log2, int max_pages,
                                     int num_pages, int d, int num_splits, float scale, hipStream_t stream);

// Split and combine in one launch (the split kernel's last workgroup per group merges).
hipError_t launch_decode_paged_fused(const void* Q, const void* K_pages, const void* V_pages,
                                     const int* block_table, const int* seq_lens, float* O_part,
                                     float* LSE_part, int* counters, void* O, float* LSE, int B, int H, int H_kv,
                                     int page_log2, int max_pages, int num_pages, int d, int num_splits,
                                     float scale, hipStream_t stream);
hipError_t launch_decode_fused(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                               int* counters, void* O, float* LSE, int B, int H, int H_kv, int N_k, int d,
                               int num_splits, float scale, hipStream_t stream);

// Group counters of the one-launch decode: zero them, or count the non-zero ones into *nonzero.
hipError_t launch_counters_reset(int* counters, int n, hipStream_t stream);
hipError_t launch_counters_check(const int* counters, int n, int* nonzero, hipStream_t stream);

// fa_decode_static: fa_decode with its workspace and counters in a file-scope device array
// of kStaticScratchBytes (no allocation); the first call on a device clears its counters.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr size_t kStaticCounterBytes = (size_t)64 << 10;
size_t decode_static_bytes(int B, int H, int d, int num_splits);  // counters + LSE_part + O_part
hipError_t launch_decode_static(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int H_kv, int N_k, int d, int num_splits, float scale, hipStream_t stream);

hipError_t launch_combine(const float* O_part, const float* LSE_part, void* O, float* LSE, int B, int H,
                          int d, int num_splits, hipStream_t stream);

}  // namespace fa
