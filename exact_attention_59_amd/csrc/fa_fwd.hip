// fa_fwd.hip -- FlashAttention-2 forward for gfx950 (bf16 in/out, fp32 state).
//
// What is computed (Lecture 11 sections 3.1-3.4, 4.1-4.2, 5.3; the FlashAttention v2
// card of the CUDA Kernel interview course): for each query row, O = softmax(scale *
// q K^T) V and LSE = m + ln l, streaming K/V tiles and carrying the online state
// (m, l, acc); normalisation is deferred to the end; S and P stay in registers.
//
// Work decomposition (FA2 order, split-Q):
//   - one workgroup of 4 waves per (batch, head, 128-row query tile); each wave owns
//     32 query rows, so no cross-wave reduction is ever needed;
//   - the workgroup walks the 64-key tiles K_j, V_j once; both are staged in LDS
//     (K row-major, V transposed) and shared by the 4 waves;
//   - under the causal mask the tile loop stops at the last tile any row of the
//     workgroup can see, and a wave skips tiles its own rows cannot see; only tiles
//     crossing the diagonal or the ragged end of K are masked element-wise;
//   - workgroup ids are ordered tile-rank-major so that, under the causal mask, the
//     longest query tiles start first, and workgroups sharing a K/V head land on the
//     same XCD (consecutive ids go round-robin over the 8 XCDs and B*H is a
//     multiple of 8 in the usual shapes).
//
// Register layout: the scores are computed transposed, S^T = K_j Q_i^T, with
// v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = head dim).  A lane then holds
// one query row (lane % 32) and 16 of every 32 keys, so the row max and row sum are
// lane-local plus a single exchange between the two 32-lane halves.  The fp32 P^T
// values, rounded to bf16, are already in the layout of the B operand of the second
// product O^T += V_j^T P^T; the key order inside that contraction is permuted to
// match, and V_j^T is read from LDS in the same order.  O^T keeps one query row per
// lane, so the rescale by alpha is a per-lane scalar multiply.
//
// Softmax in base 2: t = s * scale * log2(e); m is kept in t units;
// p = 2^(t - m), alpha = 2^(m_old - m_new); LSE = (m + log2 l) * ln 2.
// l sums the fp32 p (before rounding P to bf16).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdCfg {
    static constexpr int BR = kFwdBlockRows;  // query rows per workgroup
    static constexpr int BC = kFwdBlockCols;  // keys per tile
    static constexpr int THREADS = 256;
    static constexpr int KS = D + 8;   // LDS row stride (elements) of the K tile [BC][D]
    static constexpr int VS = BC + 8;  // LDS row stride (elements) of the V^T tile [D][BC]
    static constexpr int CHUNKS_PER_ROW = D / 8;                    // 16-byte chunks per K/V row
    static constexpr int K_CHUNKS = BC * CHUNKS_PER_ROW / THREADS;  // K chunks per thread
    static constexpr int V_KPT = BC * CHUNKS_PER_ROW / THREADS;     // V keys per thread (one chunk each)
    static constexpr int LDS_ELEMS = BC * KS + D * VS;
    static_assert(K_CHUNKS >= 1 && V_KPT >= 2 && V_KPT % 2 == 0, "tile too small for the thread count");
    static_assert(THREADS / CHUNKS_PER_ROW * V_KPT == BC, "V transpose mapping must cover the tile");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                     int H, int H_kv, int N_q, int N_k, int T_r, int BH,
                                                     float c) {
    using C = FwdCfg<D>;
    constexpr int BR = C::BR, BC = C::BC, KS = C::KS, VS = C::VS, CPR = C::CHUNKS_PER_ROW;
    __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
    uint16_t* Ks = smem;
    uint16_t* Vt = smem + BC * KS;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int bid = blockIdx.x;
    const int rank = bid / BH;
    const int bh = bid - rank * BH;
    const int q_tile = CAUSAL ? (T_r - 1 - rank) : rank;
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / H_kv);
    const int64_t q_base = (int64_t)bh * N_q * D;
    const int64_t kv_base = (int64_t)(b * H_kv + g) * N_k * D;
    const int off = N_k - N_q;  // bottom-right causal alignment
    const int T_c = (N_k + BC - 1) / BC;

    const int q0w = q_tile * BR + w * 32;  // first query row of this wave
    const int q_row = q0w + l32;           // this lane's query row

    // Tiles the workgroup walks and tiles this wave computes.
    int n_tiles = T_c, n_w = T_c;
    {
        const int last_row = min(q_tile * BR + BR, N_q) - 1;
        const int last_row_w = min(q0w + 32, N_q) - 1;
        if (CAUSAL) {
            const int kl = last_row + off, klw = last_row_w + off;
            n_tiles = kl < 0 ? 0 : min(T_c, kl / BC + 1);
            n_w = klw < 0 ? 0 : min(T_c, klw / BC + 1);
        }
        if (last_row_w < q0w) n_w = 0;  // wave entirely past the end of Q
    }

    // Q fragment (B operand of S^T = K Q^T): lane holds Q[q_row][16*ks + 8*hh + e].
    bf16x8 qf[D / 16];
    if (q_row < N_q) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(Q + q_base + (int64_t)q_row * D + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(qp[2 * ks]);
    } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }

    // Global -> register staging of one K/V tile (rows past N_k read as zero).
    u32x4 kreg[C::K_CHUNKS], vreg[C::V_KPT];
    const int v_dc = tid % CPR, v_kg = tid / CPR;
    auto load_tile = [&](int j) {
        const int key0 = j * BC;
#pragma unroll
        for (int r = 0; r < C::K_CHUNKS; ++r) {
            const int cidx = tid + C::THREADS * r;
            const int key = key0 + cidx / CPR, dc = cidx % CPR;
            const int key_c = min(key, N_k - 1);  // in-bounds address; the value is zeroed below
            kreg[r] = key < N_k ? *reinterpret_cast<const u32x4*>(K + kv_base + (int64_t)key_c * D + dc * 8)
                                : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < C::V_KPT; ++r) {
            const int key = key0 + v_kg * C::V_KPT + r;
            const int key_c = min(key, N_k - 1);
            vreg[r] = key < N_k ? *reinterpret_cast<const u32x4*>(V + kv_base + (int64_t)key_c * D + v_dc * 8)
                                : u32x4{0, 0, 0, 0};
        }
    };
    // Register -> LDS: K row-major; V transposed to Vt[d][key] (pairs of keys per 32-bit word).
    auto store_tile = [&]() {
#pragma unroll
        for (int r = 0; r < C::K_CHUNKS; ++r) {
            const int cidx = tid + C::THREADS * r;
            *reinterpret_cast<u32x4*>(Ks + (cidx / CPR) * KS + (cidx % CPR) * 8) = kreg[r];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t words[C::V_KPT / 2];
#pragma unroll
            for (int p = 0; p < C::V_KPT / 2; ++p) {
                const uint32_t a = vreg[2 * p][e >> 1], bb = vreg[2 * p + 1][e >> 1];
                words[p] = (e & 1) ? ((a >> 16) | (bb & 0xffff0000u)) : ((a & 0xffffu) | (bb << 16));
            }
            uint16_t* dst = Vt + (v_dc * 8 + e) * VS + v_kg * C::V_KPT;
            if constexpr (C::V_KPT == 4) {
                *reinterpret_cast<u32x2*>(dst) = u32x2{words[0], words[1]};
            } else if constexpr (C::V_KPT == 2) {
                *reinterpret_cast<uint32_t*>(dst) = words[0];
            } else {
#pragma unroll
                for (int p = 0; p < C::V_KPT / 2; ++p) reinterpret_cast<uint32_t*>(dst)[p] = words[p];
            }
        }
    };

    float m2 = -INFINITY;  // running max, in units of log2(e) * scale * score
    float lsum = 0.f;      // running sum of 2^(t - m2)
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    if (n_tiles > 0) load_tile(0);
    for (int j = 0; j < n_tiles; ++j) {
        __syncthreads();  // every wave is done with tile j-1
        store_tile();
        __syncthreads();  // tile j visible to every wave
        if (j + 1 < n_tiles) load_tile(j + 1);
        if (j >= n_w) continue;

        // S^T[key][query] = K_j Q^T   (two 32-key blocks)
        f32x16 s[BC / 32];
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb) {
            s[mb] = f32x16{};
            const uint16_t* kp = Ks + (32 * mb + l32) * KS + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                s[mb] = mfma32(*reinterpret_cast<const bf16x8*>(kp + 16 * ks), qf[ks], s[mb]);
        }

        // Element mask on ragged or diagonal tiles only.
        const int key0 = j * BC;
        const bool ragged = key0 + BC > N_k;
        const bool diag = CAUSAL && (key0 + BC - 1 > q0w + off);
        if (ragged || diag) {
            const int lim = CAUSAL ? min(N_k - 1, q_row + off) : N_k - 1;  // last visible key
#pragma unroll
            for (int mb = 0; mb < BC / 32; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key > lim) s[mb][r] = -INFINITY;
                }
        }

        // Online softmax update (row = this lane's query; the other half holds the other keys).
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
        mx = xor_max(mx, 32);
        const float m_new = fmaxf(m2, mx * c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_hw(m2 - m_use);
        float ps = 0.f;
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_hw(fmaf(s[mb][r], c, -m_use));
                s[mb][r] = p;
                ps += p;
            }
        ps = xor_sum(ps, 32);
        lsum = fmaf(lsum, alpha, ps);
        m2 = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;

        // P^T as B operand: 16-key step k2 uses registers 8*(k2&1) .. +7 of block k2/2,
        // i.e. keys 16*k2 + 8*(e/4) + 4*hh + e%4 for e = 0..7.
        bf16x8 pf[BC / 16];
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2) {
            const int mb = k2 >> 1, r0 = 8 * (k2 & 1);
            pf[k2] = as_bf16x8(u32x4{pack_bf16x2(s[mb][r0 + 0], s[mb][r0 + 1]),
                                     pack_bf16x2(s[mb][r0 + 2], s[mb][r0 + 3]),
                                     pack_bf16x2(s[mb][r0 + 4], s[mb][r0 + 5]),
                                     pack_bf16x2(s[mb][r0 + 6], s[mb][r0 + 7])});
        }

        // O^T[d][query] += V_j^T P^T, V^T read in the same permuted key order.
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint16_t* vp = Vt + (32 * db + l32) * VS + 16 * k2 + 4 * hh;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
                acc[db] = mfma32(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf[k2], acc[db]);
            }
    }

    // Epilogue: O = acc / l (once), LSE = (m + log2 l) ln 2.
    if (q_row < N_q) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        uint16_t* op = O + q_base + (int64_t)q_row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int d0 = 32 * db + 8 * gq + 4 * hh;
                *reinterpret_cast<u32x2*>(op + d0) =
                    u32x2{pack_bf16x2(acc[db][4 * gq + 0] * inv, acc[db][4 * gq + 1] * inv),
                          pack_bf16x2(acc[db][4 * gq + 2] * inv, acc[db][4 * gq + 3] * inv)};
            }
        if (hh == 0) LSE[(int64_t)bh * N_q + q_row] = lsum > 0.f ? (m2 + log2_hw(lsum)) * kLn2 : -INFINITY;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                        int H_kv, int N_q, int N_k, float scale, hipStream_t stream) {
    const int T_r = (N_q + kFwdBlockRows - 1) / kFwdBlockRows;
    const int BH = B * H;
    const float c = (float)((double)scale * 1.4426950408889634073599);
    const long long blocks = (long long)T_r * BH;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), static_cast<uint16_t*>(O), LSE, H, H_kv, N_q, N_k,
                       T_r, BH, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                      int H_kv, int N_q, int N_k, int d, bool causal, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_fwd_t<64, true>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream)
                      : launch_fwd_t<64, false>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream);
    return causal ? launch_fwd_t<128, true>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream)
                  : launch_fwd_t<128, false>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream);
}

}  // namespace fa
