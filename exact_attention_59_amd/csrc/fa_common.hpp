// fa_common.hpp -- device-side building blocks shared by the gfx950 attention kernels:
// vector types, the two bf16 MFMA shapes used, lane reductions, bf16 packing.
//
// MFMA register layouts relied on (CDNA3/CDNA4 matrix-core conventions, 64-lane wave):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//     B: lane l holds B[8*(l/32) + e][l % 32]
//     D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l % 16][8*(l/16) + e]
//     B: lane l holds B[8*(l/16) + e][l % 16]
//     D: lane l, register r holds D[4*(l/16) + r][l % 16]
// The contraction index only has to be numbered the same way in A and B, so the
// kernels are free to permute it (they do, to make loads contiguous).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands OCP e4m3 and unit block scales
// (E8M0 exponent 127 = 2^0): D[32x32] += A[32x64] * B[64x32] in fp32.  Each lane holds 32
// e4m3 bytes of A (row l % 32) and of B (column l % 32); byte e of lane l's A pairs with
// byte e of lane l' = (n + 32 * (l / 32))'s B -- the 64-deep contraction runs over the
// slots (l / 32, e), numbered alike in both operands (established by an on-GPU probe).
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Round two floats to OCP e4m3 (nearest-even; NaN beyond 464) into bytes 0-1 (HI = false)
// or 2-3 (HI = true) of `old`, keeping its other half (v_cvt_pk_fp8_f32).
template <bool HI>
__device__ __forceinline__ int pack_fp8x2(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Workgroup id -> (head index, rank within the head).  Consecutive ids are dispatched
// round-robin over the 8 XCDs, each with its own L2.  Heads are numbered so that the `group`
// consecutive heads that read one K/V head (grouped-query attention; group = 1 otherwise)
// form a unit.  When the number of units is a multiple of 8, every workgroup of a unit goes
// to the same XCD (id % 8 == unit % 8) and, within an XCD, ids walk head by head through
// the unit, so the workgroups that read the same K/V tiles are resident together and share
// them in that L2.  Otherwise, when the head count is a multiple of 8, heads are spread the
// same way one by one; else ids go rank-major over all heads.
__device__ __forceinline__ void map_block_xcd(int bid, int n_ranks, int n_heads, int group, int& head, int& rank) {
    const int n_units = n_heads / group;
    if ((n_units & 7) == 0 || (n_heads & 7) == 0) {
        const int g = (n_units & 7) == 0 ? group : 1;
        const int xcd = bid & 7, li = bid >> 3;
        const int hl = li / n_ranks;  // the XCD's hl-th head
        rank = li - hl * n_ranks;
        const int unit = xcd + 8 * (hl / g);
        head = unit * g + (hl - (hl / g) * g);
    } else {
        rank = bid / n_heads;
        head = bid - rank * n_heads;
    }
}

// 2^x on the transcendental unit (v_exp_f32); exact at x = 0, 0 at -inf.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// 2^x on the FMA units (FA4's softmax trick: part of the exponentials leave the
// transcendental unit; CUDA Kernel interview course, FlashAttention v4 card).  Reduction
// x = n + f with n = floor(x) and f = x - n in [0, 1] (the subtraction is exact, except that a
// tiny negative x rounds f to 1), the cubic p(f) = 1 + f (c1 + c2 f + c3 f^2)
// whose fp32 coefficients minimise max |p(f) / 2^f - 1| on [0, 1] (Remez exchange; printed by
// exact_attention_59_amd/fit_exp2_poly.py), then ldexp by n.  Relative error <= 8.6e-5 for
// x >= -126, and exact at integers (p(0) = 1); arguments at or below -200, and -inf, give
// exactly 0 (ldexp underflows), those in (-200, -126) a value below 2^-126.  Eight VALU
// instructions against one transcendental one.
constexpr float kExp2C1 = 0x1.63e658p-1f, kExp2C2 = 0x1.d2378ap-3f, kExp2C3 = 0x1.3baaa6p-4f;
__device__ __forceinline__ float exp2_poly(float x) {
    x = fmaxf(x, -200.f);
    const float fl = floorf(x);
    const float f = x - fl;
    const int n = (int)fl;
    const float p = fmaf(fmaf(fmaf(kExp2C3, f, kExp2C2), f, kExp2C1), f, 1.f);
    return __builtin_ldexpf(p, n);
}

__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, kWave)); }
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, kWave); }

// Combine a value across the two 32-lane halves of the wave (v_permlane32_swap:
// lanes 32..63 of one copy trade places with lanes 0..31 of the other).
__device__ __forceinline__ float half_swap_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum of the two halves' values, added in the same order in every lane.
__device__ __forceinline__ float half_swap_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same across lanes l and l ^ 16 (v_permlane16_swap: the odd 16-lane rows of one copy
// trade places with the even rows of the other), then across the two 32-lane halves: a
// reduction over the 4 lanes l % 16 + 16 k, with no LDS round trip.  Every lane of a group
// adds the same operands in the same order.
__device__ __forceinline__ float quad_row_max(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return half_swap_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_row_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return half_swap_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// Round two floats to bf16 (RNE, v_cvt_pk_bf16_f32) and pack them, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Copy a value through an opaque v_mov, once, outside a loop.  The copy is produced by a
// VALU instruction, so the compiler's wait-count bookkeeping no longer ties it to the
// global load that filled the source registers (otherwise the loop may wait on in-flight
// prefetch loads before every use of the value).
__device__ __forceinline__ u32x4 vgpr_copy(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("v_mov_b32 %0, %1" : "=v"(r[i]) : "v"(v[i]));
    return r;
}

// ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane i supplies the address of
// 4 consecutive 16-bit elements (row i/4 of a 4-row block, columns 4*(i%4)..+3) and
// receives element i of every row: result[e] = row e, column i.  `p` must point into LDS.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// bf16 (raw bits) -> float, exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Order LDS traffic of one wave: every lane's earlier LDS accesses complete before
// any later one is issued, and the compiler may not move LDS accesses across it.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Copy 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at LDS byte address lds_base + 16 * l.  Issued as inline assembly so
// that the compiler's wait-count bookkeeping does not see it: the compiler counts such a
// copy as both a vector-memory and an LDS access, which would turn every LDS-read wait in
// the loop into a full wait.  Completion is awaited explicitly with wait_vmem(), and the
// workgroup barrier after that orders it before any read of the buffer.
__device__ __forceinline__ void copy_to_lds16(const void* g, uint32_t lds_base) {
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}
// The same copy with a wave-uniform base address (SGPR pair) and a 32-bit per-lane byte
// offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void copy_to_lds16_sbase(const void* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_base) : "memory");
}

// Output epilogue of the kernels that keep one output row per lane: the wave's accumulators
// hold the transposed tile of its 32 rows, acc[db][4*gq + e] being element d = 32*db + 8*gq +
// 4*hh + e of row l32 (lane = 32*hh + l32).  The values are scaled by f, rounded to bf16 (RNE),
// staged in `stage` (32 * D elements of LDS that no other wave touches before the caller's next
// barrier) and stored as whole rows, 16 bytes a lane: row r goes to out + r * D when r < rows.
// Staged layout: the 16-byte chunk k of row r sits at chunk k ^ (r % chunks per row), its two
// 8-byte halves exchanged when bit 3 of r is set.  An 8-byte LDS write is served 16 lanes at a
// time over 32 four-byte banks (measured on gfx950 with the bank-conflict counter), so the 16
// rows of such a group fill 16 distinct 8-byte slots; the whole-row reads are conflict-free.
template <int D>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[D / 32], float f, uint16_t* stage,
                                                  uint16_t* __restrict__ out, int rows) {
    constexpr int CH = D / 8;      // 16-byte chunks per row
    constexpr int ROWS = 512 / D;  // rows per 64-lane read of 16 bytes a lane
    // A fresh lane index, so that no lane-derived value of the caller's loop is kept live
    // across it to be reused here.
    int el;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(el));
    const int er = el & 31, eh = el >> 5, sw = er & (CH - 1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier LDS reads of the slice are done
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<u32x2*>(stage + er * D + 8 * ((4 * db + gq) ^ sw) + 4 * (eh ^ ((er >> 3) & 1))) =
                u32x2{pack_bf16x2(acc[db][4 * gq + 0] * f, acc[db][4 * gq + 1] * f),
                      pack_bf16x2(acc[db][4 * gq + 2] * f, acc[db][4 * gq + 3] * f)};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes land before its reads
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
        const int r = ROWS * i + el / CH, ch = el % CH;
        u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * D + 8 * (ch ^ (r & (CH - 1))));
        if ((ROWS * i) & 8) v = u32x4{v[2], v[3], v[0], v[1]};  // bit 3 of r (ROWS >= 4)
        if (r < rows) *reinterpret_cast<u32x4*>(out + (int64_t)r * D + 8 * ch) = v;
    }
}

// Output epilogue of the kernels that keep one output column per lane: acc[db][r] holds row
// 8*(r/4) + 4*hh + r%4 of the wave's 32 rows at column d = 32*db + l32.  The values are scaled
// by f, rounded to bf16 (RNE), written to `stage` (32 * D elements of LDS that no other wave
// touches before the caller's next barrier) two bytes a lane, and stored as whole rows, 16
// bytes a lane: row r goes to out + r * D when r < rows.  Staged layout: the 16-byte chunk k of
// row r sits at chunk k ^ (4 * (r / 4) mod chunks per row), so that the two half-waves' rows
// of one write (r and r + 4) fall on different banks; the whole-row reads see every chunk of
// a row once.
template <int D>
__device__ __forceinline__ void store_cols_staged(const f32x16 (&acc)[D / 32], float f, uint16_t* stage,
                                                  uint16_t* __restrict__ out, int rows) {
    constexpr int CH = D / 8;      // 16-byte chunks per row
    constexpr int ROWS = 512 / D;  // rows per 64-lane read of 16 bytes a lane
    int el;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(el));
    const int l32 = el & 31, hh = el >> 5;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier LDS reads of the slice are done
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
        const int sw = 4 * ((row >> 2) & (CH / 4 - 1));
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            stage[row * D + 8 * ((4 * db + (l32 >> 3)) ^ sw) + (l32 & 7)] =
                (uint16_t)(pack_bf16x2(acc[db][r] * f, 0.f) & 0xffffu);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes land before its reads
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
        const int r = ROWS * i + el / CH, ch = el % CH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * D + 8 * (ch ^ (4 * ((r >> 2) & (CH / 4 - 1)))));
        if (r < rows) *reinterpret_cast<u32x4*>(out + (int64_t)r * D + 8 * ch) = v;
    }
}

// s_waitcnt vmcnt(0): this wave's global->LDS copies have landed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

}  // namespace fa
