// fa_fp8.hip -- FP8 (OCP e4m3) attention forward for gfx950: block quantisation with
// incoherent processing, then the FlashAttention-2 forward on fp8 matrix cores.
//
// What is computed (the FlashAttention v3 card of the CUDA Kernel interview course, "FP8
// path", and Lecture 11 section 4.4's list: per-block scales, and a random orthogonal
// transform applied first so that outlier channels are spread out):
//   fp8_quant_kernel: Q and K rows are multiplied by diag(s) H (random signs s, the
//     unnormalised Sylvester-Hadamard matrix H, H H^T = d I) and quantised to e4m3 with one
//     scale per block of rows (128 query rows, 64 keys); V is quantised with one scale per
//     64 keys, untransformed, and stored transposed per tile.  Per block: amax = max |x|,
//     code = e4m3(x * (448 / amax)) in fp32 with nearest-even rounding, scale = amax / 448
//     (times 1/d for transformed queries, so that dequantised q . k is the original score).
//   fwd_fp8_kernel: exact attention of the dequantised tensors, computed as the bf16 forward
//     does (one workgroup per 128 query rows, 64-key tiles staged in LDS, online softmax with
//     a stale max, deferred normalisation), with S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_scale_f32_32x32x64_f8f6f4 and P rounded to e4m3.
//
// Scales never multiply a matrix element inside the loop: the query block's and the key
// tile's scales multiply the softmax's score factor (one scalar per tile), and the value
// tile's scale s_v enters the exponent -- p8 = 2^(t - m + log2(s_v / s_v,max)) is what is
// rounded to e4m3, l adds p8 * (s_v,max / s_v) once per tile, and O = s_v,max * acc / l.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr float kFp8Max = 448.0f;
constexpr float kRescaleSlackFp8 = 8.0f;  // p <= 2^8 = 256 stays below e4m3's 448

// Position p = 32*h + e of a transposed value tile row holds key
//   kappa(p) = 32*(e/16) + 8*((e%16)/4) + 4*h + e%4
// of the tile: the key that byte e of half h of the P^T operand holds (the lane's scores
// in the 32x32 accumulator layout, two 32-key blocks), so the V^T operand of the same
// contraction slot is 32 consecutive bytes of the row.
__device__ __forceinline__ int vt_key(int p) {
    const int h = p >> 5, e = p & 31;
    return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3);
}

// Value of lane (lane xor M), M in {1, 2, 4, 8}, by DPP lane moves inside 16-lane rows (no LDS
// traffic, unlike a general shuffle): xor 1 and 2 are quad permutations [1,0,3,2] and
// [2,3,0,1]; xor 4 mirrors each 8-lane half (lane 8r + i takes 8r + 7 - i) and then reverses
// each quad, which together take lane 8r + 4a + b from 8r + 4(1 - a) + b; xor 8 rotates the
// 16-lane row by 8.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "DPP lane exchange inside a 16-lane row");
    const int x = __float_as_int(v);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
    if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
    if constexpr (M == 4) {
        const int y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror
        return __int_as_float(__builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, false));  // quad [3,2,1,0]
    }
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));  // row_ror:8
}

// ---------------------------------------------------------------------------- quantisation
// One workgroup of 256 threads per block of rows (a query block of kFp8QRows rows or a
// key/value tile of kFp8KRows keys).  D/8 consecutive lanes hold one row, 8 elements each
// (element 8*sub + e); the transform's stages 1, 2, 4 are inside a lane, the wider ones
// exchange with the lane whose sub differs in one bit.  Every element goes through the same
// fp32 additions, in the same order, as the plain stage-by-stage transform.
template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V, uint64_t sign_lo,
                                                        uint64_t sign_hi, int transform, uint8_t* __restrict__ Q8,
                                                        uint8_t* __restrict__ K8, uint8_t* __restrict__ Vt8,
                                                        float* __restrict__ q_scale, float* __restrict__ k_scale,
                                                        float* __restrict__ v_scale, int BH, int BHkv, int N_q, int N_k,
                                                        int TQ, int TK) {
    constexpr int LPR = D / 8;        // lanes per row
    constexpr int RPP = 256 / LPR;    // rows per pass
    constexpr int MAXP = kFp8QRows / RPP;
    __shared__ __attribute__((aligned(16))) uint8_t codes_s[kFp8KRows * D];  // value tile, row-major
    __shared__ float red[4];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int sub = tid % LPR, rr = tid / LPR;
    int kind, head, t;  // kind 0 = Q, 1 = K, 2 = V
    {
        const int bid = blockIdx.x, nq = BH * TQ, nk = BHkv * TK;
        if (bid < nq) {
            kind = 0; head = bid / TQ; t = bid - head * TQ;
        } else if (bid < nq + nk) {
            kind = 1; head = (bid - nq) / TK; t = bid - nq - head * TK;
        } else {
            kind = 2; head = (bid - nq - nk) / TK; t = bid - nq - nk - head * TK;
        }
    }
    const int N = kind == 0 ? N_q : N_k;
    const int BLK = kind == 0 ? kFp8QRows : kFp8KRows;
    const uint16_t* src = (kind == 0 ? Q : kind == 1 ? K : V) + (int64_t)head * N * D;
    const int r0 = t * BLK;
    const int rows = min(BLK, N - r0);
    const bool xform = transform && kind != 2;

    // Signs of this lane's 8 channels.
    uint32_t neg = 0;
    if (xform) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * sub + e;
            const uint64_t bit = j < 64 ? (sign_lo >> j) & 1u : (sign_hi >> (j - 64)) & 1u;
            neg |= (uint32_t)bit << e;
        }
    }

    // Every load of the block is issued before the first is used (rows past the end read the
    // block's last row, no branch; their values are zeroed below), so that the passes do not
    // each wait for memory in turn.
    u32x4 raw_all[MAXP];
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p * RPP >= BLK) break;  // uniform
        const int row = min(p * RPP + rr, rows - 1);
        raw_all[p] = *reinterpret_cast<const u32x4*>(src + (int64_t)(r0 + row) * D + 8 * sub);
    }
    float x[MAXP][8];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p * RPP >= BLK) break;  // uniform
        const int row = p * RPP + rr;
        const bool active = row < rows;
        const u32x4 raw = active ? raw_all[p] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[p][2 * e] = bf16_bits_to_f32(raw[e] & 0xffffu);
            x[p][2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16);
        }
        if (xform) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((neg >> e) & 1u) x[p][e] = -x[p][e];
#pragma unroll
            for (int len = 1; len < 8; len <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((e & len) == 0) {
                        const float a = x[p][e], b = x[p][e + len];
                        x[p][e] = a + b;
                        x[p][e + len] = a - b;
                    }
#pragma unroll
            for (int ls = 1; ls < LPR; ls <<= 1) {  // stage len = 8 * ls
                // upper lane: o - x, lower lane: x + o, as one fma with x's sign chosen per lane
                // (x * -1 is exact, so the single rounding is that of the subtraction)
                const float sgn = (sub & ls) != 0 ? -1.f : 1.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = x[p][e];
                    const float o = ls == 1 ? lane_xor<1>(v) : ls == 2 ? lane_xor<2>(v) : ls == 4 ? lane_xor<4>(v)
                                                                                          : lane_xor<8>(v);
                    x[p][e] = fmaf(v, sgn, o);
                }
            }
        }
        if (active)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[p][e]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    if (lane == 0) red[w] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float rcp = amax > 0.f ? kFp8Max / amax : 0.f;
    if (tid == 0) {
        float sc = amax > 0.f ? amax / kFp8Max : 0.f;
        if (kind == 0 && transform) sc *= 1.0f / D;
        float* dst = kind == 0 ? q_scale : kind == 1 ? k_scale : v_scale;
        dst[(int64_t)head * (kind == 0 ? TQ : TK) + t] = sc;
    }

#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p * RPP >= BLK) break;
        const int row = p * RPP + rr;
        if (row >= rows) continue;
        int lo = pack_fp8x2<false>(x[p][0] * rcp, x[p][1] * rcp, 0);
        lo = pack_fp8x2<true>(x[p][2] * rcp, x[p][3] * rcp, lo);
        int hi = pack_fp8x2<false>(x[p][4] * rcp, x[p][5] * rcp, 0);
        hi = pack_fp8x2<true>(x[p][6] * rcp, x[p][7] * rcp, hi);
        if (kind == 2) {
            *reinterpret_cast<u32x2*>(codes_s + row * D + 8 * sub) = u32x2{(uint32_t)lo, (uint32_t)hi};
        } else {
            uint8_t* dst = (kind == 0 ? Q8 : K8) + ((int64_t)head * N + r0 + row) * D + 8 * sub;
            *reinterpret_cast<u32x2*>(dst) = u32x2{(uint32_t)lo, (uint32_t)hi};
        }
    }
    if (kind != 2) return;  // uniform per workgroup
    __syncthreads();
    // Transposed, key-permuted tile: D rows (channels) x 64 positions; 16 bytes per thread.
    // The lanes of a wave take consecutive channels of one 16-position group, so every LDS
    // read instruction reads one key row (64 consecutive bytes, no bank conflicts).
    uint8_t* tile = Vt8 + ((int64_t)head * TK + t) * (D * kFp8KRows);
#pragma unroll
    for (int q = tid; q < D * 4; q += 256) {
        const int j = q % D, p0 = 16 * (q / D);
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int key = vt_key(p0 + 4 * k + b);
                const uint32_t byte = key < rows ? codes_s[key * D + j] : 0u;
                v |= byte << (8 * b);
            }
            wv[k] = v;
        }
        *reinterpret_cast<u32x4*>(tile + j * kFp8KRows + p0) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
}

// ---------------------------------------------------------------------------- forward
// K tile in LDS: 64 rows of D bytes, 16-byte chunks swizzled so that 16 consecutive rows
// reading one logical chunk hit 16 distinct bank groups (two rows per 256 bytes at D=128,
// four at D=64).  V^T tile: D rows of 64 bytes, four rows per 256 bytes.
template <int D>
__device__ __forceinline__ int swz_k8(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
__device__ __forceinline__ int swz_v8(int r) { return (r >> 2) & 3; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                                                         const uint8_t* __restrict__ Vt8,
                                                         const float* __restrict__ q_scale,
                                                         const float* __restrict__ k_scale,
                                                         const float* __restrict__ v_scale, uint16_t* __restrict__ O,
                                                         float* __restrict__ LSE, int H, int H_kv, int N_q, int N_k,
                                                         int T_r, int BH, float c) {
    constexpr int BR = kFp8QRows, BC = kFp8KRows;
    constexpr int TILE = BC * D;                 // bytes of a K tile and of a V^T tile
    constexpr int CPW = TILE / 1024 / 4;         // 1 KB copies per wave per tile
    constexpr int KCH = D / 16;                  // 16-byte chunks per K row
    static_assert(CPW >= 1, "tile must split into 1 KB copies over 4 waves");
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE];
    asm volatile("" ::"s"(O), "s"(LSE));

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int n_ranks = CAUSAL ? (T_r + 1) / 2 : T_r;
    int bh, rank;
    map_block_xcd(blockIdx.x, n_ranks, BH, H / H_kv, bh, rank);
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / H_kv);
    const int bg = b * H_kv + g;
    const int T_c = (N_k + BC - 1) / BC;
    const int off = N_k - N_q;
    const uint8_t* kh = K8 + (int64_t)bg * N_k * D;
    const uint8_t* vh = Vt8 + (int64_t)bg * T_c * TILE;
    const float* ksh = k_scale + (int64_t)bg * T_c;
    const float* vsh = v_scale + (int64_t)bg * T_c;

    // s_v,max over the head's value tiles (wave-wide max, the same in every wave).
    float sv_max = 0.f;
    for (int i = lane; i < T_c; i += 64) sv_max = fmaxf(sv_max, vsh[i]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sv_max = fmaxf(sv_max, __shfl_xor(sv_max, m, kWave));
    const float inv_sv_max = sv_max > 0.f ? 1.f / sv_max : 0.f;

    // Copy helpers: copy u of this wave fills 1 KB block (w * CPW + u) of a tile.  A whole tile
    // is copied from a wave-uniform base (scalar registers, advanced by 1 KB per copy) plus fixed
    // per-lane byte offsets; the ragged last K tile clamps rows per lane.  V^T tiles are padded
    // to whole tiles by the quantiser, and their swizzle repeats within every copy's rows, so
    // one offset serves all of V's copies.
    uint32_t koff[CPW];
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
        const int row = (w * CPW + u) * (1024 / D) + lane / KCH;
        koff[u] = (uint32_t)((lane / KCH) * D + 16 * ((lane % KCH) ^ swz_k8<D>(row)));
    }
    const uint32_t voff = (uint32_t)((lane / 4) * BC + 16 * ((lane % 4) ^ swz_v8(w * CPW * 16 + lane / 4)));
    auto dma_k = [&](int j, uint8_t* dst) {
        if ((j + 1) * BC <= N_k) {
            const uint8_t* tile = kh + (int64_t)j * BC * D;
#pragma unroll
            for (int u = 0; u < CPW; ++u)
                copy_to_lds16_sbase(tile + (w * CPW + u) * 1024, koff[u], lds_addr(dst + (w * CPW + u) * 1024));
            return;
        }
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const int blk = w * CPW + u;
            const int row = blk * (1024 / D) + lane / KCH;
            const int ch = (lane % KCH) ^ swz_k8<D>(row);
            const uint8_t* gp = kh + (int64_t)min(j * BC + row, N_k - 1) * D + 16 * ch;
            copy_to_lds16(gp, lds_addr(dst + blk * 1024));
        }
    };
    auto dma_v = [&](int j, uint8_t* dst) {
        const uint8_t* tile = vh + (int64_t)j * TILE;
#pragma unroll
        for (int u = 0; u < CPW; ++u)
            copy_to_lds16_sbase(tile + (w * CPW + u) * 1024, voff, lds_addr(dst + (w * CPW + u) * 1024));
    };
    // A-operand reads: 32 bytes of row `row` at logical chunks c0, c0 + 1.
    auto read32 = [&](const uint8_t* base, int row, int rowbytes, int c0, int sw) -> i32x8 {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + row * rowbytes + 16 * (c0 ^ sw));
        const u32x4 b2 = *reinterpret_cast<const u32x4*>(base + row * rowbytes + 16 * ((c0 + 1) ^ sw));
        return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b2[0], (int)b2[1], (int)b2[2], (int)b2[3]};
    };

    auto run_tile = [&](const int q_tile) {
        const int q0w = q_tile * BR + w * 32, q_row = q0w + l32;
        int n_tiles = T_c, n_w = T_c;
        {
            const int last_row = min(q_tile * BR + BR, N_q) - 1;
            const int last_row_w = min(q0w + 32, N_q) - 1;
            if (CAUSAL) {
                const int kl = last_row + off, klw = last_row_w + off;
                n_tiles = kl < 0 ? 0 : min(T_c, kl / BC + 1);
                n_w = klw < 0 ? 0 : min(T_c, klw / BC + 1);
            }
            if (last_row_w < q0w) n_w = 0;
        }
        const float sq = q_scale[(int64_t)bh * T_r + q_tile];
        // Q^T operand: lane holds Q8[q_row][64*ks + 32*hh + e], e < 32.  The loads are issued
        // here (rows past N_q read row N_q - 1, no branch) and the values taken through the
        // opaque copy only after the first tile copies are issued too (zeros past N_q).
        u32x4 q_raw[2 * (D / 64)];
        {
            const uint8_t* qp = Q8 + ((int64_t)bh * N_q + min(q_row, N_q - 1)) * D + 32 * hh;
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks) {
                q_raw[2 * ks] = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
                q_raw[2 * ks + 1] = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
            }
        }
        i32x8 qf[D / 64];
        auto take_q = [&] {
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks) {
                const u32x4 a = vgpr_copy(q_raw[2 * ks]);
                const u32x4 b2 = vgpr_copy(q_raw[2 * ks + 1]);
                const bool ok = q_row < N_q;
                qf[ks] = i32x8{ok ? (int)a[0] : 0, ok ? (int)a[1] : 0, ok ? (int)a[2] : 0, ok ? (int)a[3] : 0,
                               ok ? (int)b2[0] : 0, ok ? (int)b2[1] : 0, ok ? (int)b2[2] : 0, ok ? (int)b2[3] : 0};
            }
        };
        const int sk_row = swz_k8<D>(l32);  // same for rows l32 and 32 + l32
        const int sv_row = swz_v8(l32);

        f32x16 acc[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
        float m2 = -INFINITY, lsum = 0.f;

        auto step = [&](auto parity, int j) {
            constexpr bool odd = decltype(parity)::value;
            const uint8_t* kr = odd ? k_lds1 : k_lds0;
            const uint8_t* vr = odd ? v_lds1 : v_lds0;
            uint8_t* kf = odd ? k_lds0 : k_lds1;
            uint8_t* vf = odd ? v_lds0 : v_lds1;
            if (j + 1 < n_tiles) {
                dma_k(j + 1, kf);
                dma_v(j + 1, vf);
            }
            if (j < n_w) {
                f32x16 s[2];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    s[mb] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < D / 64; ++ks)
                        s[mb] = mfma32_fp8(read32(kr, 32 * mb + l32, D, 4 * ks + 2 * hh, sk_row), qf[ks], s[mb]);
                }
                const float sk = ksh[j], sv = vsh[j];
                // score factor (kept positive, so that a masked -inf stays -inf)
                const float cs = fmaxf(c * sq * sk, 1.17549435e-38f);
                // per-tile weights from reciprocals (v_rcp_f32, about 1 ulp) instead of divisions
                const float lv = sv > 0.f ? log2_hw(sv * inv_sv_max) : 0.f;
                const float wv = sv > 0.f ? sv_max * __builtin_amdgcn_rcpf(sv) : 1.f;
                const int key0 = j * BC;
                if (key0 + BC > N_k || (CAUSAL && key0 + BC - 1 > q0w + off)) {
                    const int lim = (CAUSAL ? min(N_k - 1, q_row + off) : N_k - 1) - key0 - 4 * hh;
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (32 * mb + 8 * (r >> 2) + (r & 3) > lim) s[mb][r] = -INFINITY;
                }
                float mx = -INFINITY;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
                mx = half_swap_max(mx);
                const float t_max = mx * cs;
                const bool need = t_max > m2 + kRescaleSlackFp8;
                if (__any(need)) {
                    const float alpha = need ? exp2_hw(m2 - t_max) : 1.f;
                    lsum *= alpha;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
                    m2 = need ? t_max : m2;
                }
                const float bias = (m2 == -INFINITY ? 0.f : m2) - lv;
                float ps = 0.f;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = exp2_hw(fmaf(s[mb][r], cs, -bias));
                        s[mb][r] = p;
                        ps += p;
                    }
                lsum += ps * wv;
                // P^T operand: byte e = 16*mb + r of the lane's 32 holds s[mb][r].
                i32x8 pb;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int mb = k >> 2, r0 = 4 * (k & 3);
                    const int lo = pack_fp8x2<false>(s[mb][r0], s[mb][r0 + 1], 0);
                    pb[k] = pack_fp8x2<true>(s[mb][r0 + 2], s[mb][r0 + 3], lo);
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    acc[db] = mfma32_fp8(read32(vr, 32 * db + l32, BC, 2 * hh, sv_row), pb, acc[db]);
            }
            wait_vmem();
            __syncthreads();
        };

        if (n_tiles > 0) {
            dma_k(0, k_lds0);
            dma_v(0, v_lds0);
            take_q();
            wait_vmem();
            __syncthreads();
        }
        for (int j = 0; j < n_tiles; j += 2) {
            step(std::integral_constant<bool, false>{}, j);
            if (j + 1 < n_tiles) step(std::integral_constant<bool, true>{}, j + 1);
        }

        // Epilogue: the wave stages its rows in one of the four tile buffers (idle: every read of
        // the loop completed before its last barrier, and no copy is in flight) and stores them
        // as whole rows.
        lsum = half_swap_sum(lsum);
        static_assert(TILE >= 32 * D * 2, "a tile buffer holds a wave's 32 output rows");
        uint8_t* const stage = w == 0 ? k_lds0 : w == 1 ? k_lds1 : w == 2 ? v_lds0 : v_lds1;
        store_rows_staged<D>(acc, lsum > 0.f ? sv_max / lsum : 0.f, reinterpret_cast<uint16_t*>(stage),
                             O + ((int64_t)bh * N_q + q0w) * D, N_q - q0w);
        if (hh == 0 && q_row < N_q)
            LSE[(int64_t)bh * N_q + q_row] = lsum > 0.f ? (m2 + log2_hw(lsum)) * kLn2 : -INFINITY;
    };

    run_tile(CAUSAL ? T_r - 1 - rank : rank);
    if (CAUSAL && rank != T_r - 1 - rank) {
        __syncthreads();
        run_tile(rank);
    }
}

template <int D>
hipError_t launch_fp8_quantize_t(const void* Q, const void* K, const void* V, int transform, uint64_t sign_lo,
                                 uint64_t sign_hi, void* Q8, void* K8, void* Vt8, float* q_scale, float* k_scale,
                                 float* v_scale, int B, int H, int H_kv, int N_q, int N_k, hipStream_t stream) {
    const int TQ = (N_q + kFp8QRows - 1) / kFp8QRows, TK = (N_k + kFp8KRows - 1) / kFp8KRows;
    const long long blocks = (long long)B * H * TQ + 2LL * B * H_kv * TK;
    hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), sign_lo, sign_hi, transform, static_cast<uint8_t*>(Q8),
                       static_cast<uint8_t*>(K8), static_cast<uint8_t*>(Vt8), q_scale, k_scale, v_scale, B * H,
                       B * H_kv, N_q, N_k, TQ, TK);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8_t(const void* Q8, const void* K8, const void* Vt8, const float* q_scale,
                            const float* k_scale, const float* v_scale, void* O, float* LSE, int B, int H, int H_kv,
                            int N_q, int N_k, float scale, hipStream_t stream) {
    const int T_r = (N_q + kFp8QRows - 1) / kFp8QRows;
    const float c = (float)((double)scale * 1.4426950408889634073599);
    const long long blocks = (long long)(CAUSAL ? (T_r + 1) / 2 : T_r) * B * H;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(Q8), static_cast<const uint8_t*>(K8),
                       static_cast<const uint8_t*>(Vt8), q_scale, k_scale, v_scale, static_cast<uint16_t*>(O), LSE,
                       H, H_kv, N_q, N_k, T_r, B * H, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const void* Q, const void* K, const void* V, int transform, uint64_t sign_lo,
                               uint64_t sign_hi, void* Q8, void* K8, void* Vt8, float* q_scale, float* k_scale,
                               float* v_scale, int B, int H, int H_kv, int N_q, int N_k, int d, hipStream_t stream) {
    if (d == 64)
        return launch_fp8_quantize_t<64>(Q, K, V, transform, sign_lo, sign_hi, Q8, K8, Vt8, q_scale, k_scale,
                                         v_scale, B, H, H_kv, N_q, N_k, stream);
    return launch_fp8_quantize_t<128>(Q, K, V, transform, sign_lo, sign_hi, Q8, K8, Vt8, q_scale, k_scale, v_scale,
                                      B, H, H_kv, N_q, N_k, stream);
}

hipError_t launch_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
                          const float* v_scale, void* O, float* LSE, int B, int H, int H_kv, int N_q, int N_k, int d,
                          bool causal, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_fwd_fp8_t<64, true>(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, H_kv, N_q,
                                                   N_k, scale, stream)
                      : launch_fwd_fp8_t<64, false>(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, H_kv, N_q,
                                                    N_k, scale, stream);
    return causal ? launch_fwd_fp8_t<128, true>(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, H_kv, N_q, N_k,
                                                scale, stream)
                  : launch_fwd_fp8_t<128, false>(Q8, K8, Vt8, q_scale, k_scale, v_scale, O, LSE, B, H, H_kv, N_q,
                                                 N_k, scale, stream);
}

}  // namespace fa
