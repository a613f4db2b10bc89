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
//   - the workgroup walks the 64-key tiles K_j, V_j once; both are staged row-major
//     in LDS (bank-conflict-free strides), double-buffered, and shared by the 4 waves;
//     one barrier per tile;
//   - software pipeline inside each wave: the MFMAs of tile j+1's scores are issued
//     next to tile j's softmax (they are independent), so the matrix cores work while
//     the vector ALUs compute exp; the rescale of acc is skipped unless the running
//     max grows by more than a fixed slack (exact: the max cancels in acc / l);
//   - under the causal mask the tile loop stops at the last tile any row of the
//     workgroup can see, and a wave skips tiles its own rows cannot see; only tiles
//     crossing the diagonal or the ragged end of K are masked element-wise;
//   - under the causal mask a workgroup takes two query tiles, i and T_r-1-i, so every
//     workgroup does the same work (no tail of long tiles); the order of the two is chosen
//     per head dimension for L2 reuse of K/V (end of the kernel);
//   - optionally (POLY > 0) part of the exponentials are computed by a cubic on the FMA
//     units instead of the transcendental instruction (the FA4 softmax trick);
//   - workgroup ids are mapped so that the workgroups of a head share an XCD (and its
//     L2) and are resident together;
//   - the output tile is staged through LDS so that every store writes whole rows.
//
// Register layout: the scores are computed transposed, S^T = K_j Q_i^T, with
// v_mfma_f32_32x32x16_bf16 (M = keys, N = queries, K = head dim).  A lane then holds
// one query row (lane % 32) and 16 of every 32 keys, so the row max and row sum are
// lane-local plus a single exchange between the two 32-lane halves.  The fp32 P^T
// values, rounded to bf16, are already in the layout of the B operand of the second
// product O^T += V_j^T P^T; the key order inside that contraction is permuted to
// match, and V_j^T is read from row-major LDS with gfx950's transposing LDS read.  O^T keeps one query row per
// lane, so the rescale by alpha is a per-lane scalar multiply.
//
// Softmax in base 2: t = s * scale * log2(e); m is kept in t units;
// p = 2^(t - m), alpha = 2^(m_old - m_new); LSE = (m + log2 l) * ln 2.
// l sums the fp32 p (before rounding P to bf16).
#include <algorithm>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

template <int D>
struct FwdCfg {
    static constexpr int NW = fwd_waves(D);       // waves per workgroup
    static constexpr int BR = fwd_block_rows(D);  // query rows per workgroup (32 per wave)
    static constexpr int BC = fwd_block_cols(D);  // keys per tile
    static constexpr int THREADS = 64 * NW;
    static constexpr int TILE = BC * D;       // elements of one K or V tile buffer (rows unpadded)
    // A 64-lane global->LDS copy moves 1 KB; the waves split a tile's copies evenly.
    static constexpr int DMA_PER_WAVE = BC * D * 2 / 1024 / NW;
    static_assert(BR == 32 * NW, "each wave owns 32 query rows");
    static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * NW * 1024 == BC * D * 2, "tile must split into 1 KB copies");
};

// LDS tiles are row-major without padding; the 16-byte chunks of row r are stored at
// chunk index c ^ swz(r) so that both read patterns are bank-conflict-free (64 banks):
//   K (QK A operand): 16 consecutive rows, one chunk each -> 16 distinct chunk slots;
//   V (transposing reads): 4 consecutive rows x 4 consecutive chunks (32 d-values) -> 16
//   distinct slots.  A row of d = 128 spans all 64 banks, a row of d = 64 half of them.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Lazy rescale threshold (log2 units).  The running max m is only moved when a tile's
// max exceeds it by more than this; until then p = 2^(t - m) <= 2^kRescaleSlack, which
// fp32 and bf16 hold exactly as well as p <= 1.  The result is the same exact softmax:
// whatever m is used, it cancels between the numerator acc and the denominator l.
constexpr float kRescaleSlack = 8.0f;

// Workgroups per CU: three at d = 64 (at most 168 VGPRs, 12 waves per CU), whose third
// wave per SIMD covers latency that two leave exposed; two at d = 128 (its MFMA tiles and
// accumulators need up to 256 VGPRs).
template <int D>
constexpr int kFwdBlocksPerCU = D == 64 ? 3 : 8 / fwd_waves(D);

// POLY (0..4): of every four exponentials of a lane's softmax, the first POLY are taken with
// exp2_poly on the FMA units and the rest with v_exp_f32 (0 = all on the transcendental unit).
template <int D, bool CAUSAL, int POLY = 0>
__global__ __launch_bounds__(FwdCfg<D>::THREADS, kFwdBlocksPerCU<D>) void fwd_kernel(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                     int H, int H_kv, int N_q, int N_k, int T_r, int BH,
                                                     float c) {
    using C = FwdCfg<D>;
    constexpr int BR = C::BR, BC = C::BC;
    // Separate arrays per buffer, so that copies into one buffer and reads of another are
    // known not to overlap.
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[C::TILE];

    // The output pointers are first needed after the loop; consume their scalar loads
    // here.  A scalar load still in flight would make every LDS wait in the loop a full
    // wait (scalar and LDS loads share one counter, and scalar ones complete out of order).
    asm volatile("" ::"s"(O), "s"(LSE));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    const int l32 = lane & 31, hh = lane >> 5;

    // Causal rows get longer with the query index, so a causal workgroup takes the pair of
    // query tiles (T_r-1-rank, rank): every workgroup then carries the same work.
    const int n_ranks = CAUSAL ? (T_r + 1) / 2 : T_r;
    int bh, rank;
    map_block_xcd(blockIdx.x, n_ranks, BH, H / H_kv, bh, rank);
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / H_kv);
    const int64_t q_base = (int64_t)bh * N_q * D;
    const int64_t kv_base = (int64_t)(b * H_kv + g) * N_k * D;
    const int off = N_k - N_q;  // bottom-right causal alignment
    const int T_c = (N_k + BC - 1) / BC;

  auto run_tile = [&](const int q_tile) {
    // The lane index is produced afresh for each query tile (an opaque v_mbcnt), so that the
    // per-lane offsets below are recomputed per tile instead of being kept, and spilled,
    // across the first tile's loop of a causal pair.
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    const int l32 = lane & 31, hh = lane >> 5;
    const int q0w = q_tile * BR + w * 32;  // first query row of this wave
    const int q_row = q0w + l32;           // this lane's query row

    // Tiles the workgroup walks (n_tiles) and tiles this wave computes (n_w <= n_tiles).
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

    // Q fragment (B operand of S^T = K Q^T): lane holds Q[q_row][16*ks + 8*hh + e].  The
    // loads are issued here (rows past N_q read row N_q - 1, no branch) and the values taken
    // through the opaque copy only after the first tile copies are issued too, so that the
    // wave waits for memory once in its prologue; rows past N_q get zeros.
    u32x4 q_raw[D / 16];
    {
        const u32x4* qp = reinterpret_cast<const u32x4*>(Q + q_base + (int64_t)min(q_row, N_q - 1) * D + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) q_raw[ks] = qp[2 * ks];
    }
    bf16x8 qf[D / 16];

    // ---- global -> LDS copies (no registers involved).  Copy t of this wave fills LDS
    // block (w * DMA_PER_WAVE + t), 1 KB; lane l's 16 bytes land at offset 16*l in it,
    // i.e. at row r, stored chunk sc; the lane reads logical chunk sc ^ swz(r) of row r.
    // Rows past N_k repeat row N_k - 1 (finite data whose scores are masked, P = 0).
    constexpr int ROWS_PER_COPY = 512 / D;
    const int dma_r0 = w * C::DMA_PER_WAVE * ROWS_PER_COPY + lane / (D / 8);
    const int dma_sc = lane % (D / 8);
    const uint32_t dma_lds_off = __builtin_amdgcn_readfirstlane(w * C::DMA_PER_WAVE * 1024);  // bytes
    // A whole tile is copied from a wave-uniform base address (scalar registers, advanced by
    // 1 KB per copy) plus fixed per-lane byte offsets, which keeps the address arithmetic off
    // the vector ALUs.  V's swizzle repeats within every copy's rows, so one offset serves
    // all of V's copies; K's differs per copy.  The ragged last tile clamps rows per lane.
    uint32_t dma_koff[C::DMA_PER_WAVE];
#pragma unroll
    for (int t = 0; t < C::DMA_PER_WAVE; ++t) {
        const int r = dma_r0 + t * ROWS_PER_COPY;
        dma_koff[t] = 2u * (uint32_t)(dma_r0 * D + 8 * (dma_sc ^ swz_k<D>(r)));
    }
    const uint32_t dma_voff = 2u * (uint32_t)(dma_r0 * D + 8 * (dma_sc ^ swz_v<D>(dma_r0)));
    auto dma_tile = [&](const uint16_t* __restrict__ src, int j, uint16_t* dst, bool is_v) {
        const int key0 = j * BC;
        const uint16_t* head = src + kv_base;
        if (key0 + BC <= N_k) {
            const uint16_t* tile = head + (int64_t)key0 * D;
#pragma unroll
            for (int t = 0; t < C::DMA_PER_WAVE; ++t)
                copy_to_lds16_sbase(tile + t * 512, is_v ? dma_voff : dma_koff[t],
                                    lds_addr(dst) + dma_lds_off + t * 1024);
            return;
        }
#pragma unroll
        for (int t = 0; t < C::DMA_PER_WAVE; ++t) {
            const int r = dma_r0 + t * ROWS_PER_COPY;
            const int c = dma_sc ^ (is_v ? swz_v<D>(r) : swz_k<D>(r));
            const uint16_t* g = head + (int64_t)min(key0 + r, N_k - 1) * D + 8 * c;
            copy_to_lds16(g, lds_addr(dst) + dma_lds_off + t * 1024);
        }
    };

    // ---- the two contractions
    // S^T[key][query] = K_j Q^T for the two 32-key blocks of the tile (chains interleaved).
    // Lane reads row 32*mb + l32, logical chunk 2*ks + hh; the swizzle of that row depends
    // on l32 only, so the per-ks offsets are fixed per lane.
    int k_off[D / 16];
    {
        const int sk = swz_k<D>(l32);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) k_off[ks] = l32 * D + 8 * ((2 * ks + hh) ^ sk);
    }
    // Fragments are read from LDS into registers at the top of a step, all at once, so
    // their latency overlaps the softmax instead of stalling each MFMA.
    using KFrag = bf16x8[D / 16][BC / 32];
    auto load_k = [&](const uint16_t* Ks, KFrag& kf) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int mb = 0; mb < BC / 32; ++mb)
                kf[ks][mb] = *reinterpret_cast<const bf16x8*>(Ks + k_off[ks] + 32 * mb * D);
    };
    auto qk = [&](const KFrag& kf, f32x16 (&s)[BC / 32]) {
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb) s[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int mb = 0; mb < BC / 32; ++mb) s[mb] = mfma32(kf[ks][mb], qf[ks], s[mb]);
    };
    // O^T[d][query] += V_j^T P^T.  P^T is the B operand: for 16-key step k2, half hh of
    // the wave holds keys 16*k2 + 4*hh + (0..3) and 16*k2 + 8 + 4*hh + (0..3).  The A
    // operand V_j^T comes from row-major V in LDS through ds_read_b64_tr_b16: in each
    // 16-lane group, lane i addresses row i/4, columns 4*(i%4)..+3 of a 4-key x 16-d
    // block and receives column i (4 consecutive keys at one d).  Groups 0/1 (2/3) cover
    // d = 32*db + 0..15 / 16..31 for half 0 (1); two reads give the 8 keys of the slot.
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    // With the swizzle, lane (i = lane % 16) reads row 16*k2 + 8*x + 4*hh + i/4, stored
    // chunk (4*db + cg) ^ swz_v(row) where cg = 2*((lane/16)%2) + (i%4)/2, plus 4*(i%2)
    // elements; swz_v of those rows depends on i only.
    int v_off[D / 32];
    {
        const int i = lane & 15;
        const int sv = swz_v<D>(4 * hh + (i >> 2)) >> 2;
        const int cg = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            v_off[db] = (4 * hh + (i >> 2)) * D + 32 * (db ^ sv) + 8 * cg + 4 * (i & 1);
    }
    // V^T fragments of 16-key steps k2 in [K2_0, K2_1).
    using VFrag = i16x8[BC / 16][D / 32];
    auto load_v = [&](const uint16_t* Vs, VFrag& vf, auto k2_0, auto k2_1) {
#pragma unroll
        for (int k2 = decltype(k2_0)::value; k2 < decltype(k2_1)::value; ++k2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint16_t* p = Vs + v_off[db] + 16 * k2 * D;
                const i16x4 lo = lds_read_tr16(p);
                const i16x4 hi = lds_read_tr16(p + 8 * D);
                vf[k2][db] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    };
    auto pv = [&](const VFrag& vf, const bf16x8 (&pf)[BC / 16]) {
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                acc[db] = mfma32(__builtin_bit_cast(bf16x8, vf[k2][db]), pf[k2], acc[db]);
    };

    // ---- online softmax state of this lane's query row (both 32-lane halves hold it)
    float m2 = -INFINITY;  // running (possibly stale) max, in units of log2(e) * scale * score
    float lsum = 0.f;      // this half's share of sum 2^(t - m2); the halves are added at the end

    // Mask (ragged or diagonal tiles only), row max, and the rare rescale.  Returns the
    // max to subtract in the exponent.
    auto softmax_prepare = [&](f32x16 (&s)[BC / 32], int j) -> float {
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
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
        mx = half_swap_max(mx);
        const float t_max = mx * c;
        const bool need = t_max > m2 + kRescaleSlack;  // false for -inf rows
        if (__any(need)) {
            // Lanes that keep their max use alpha = 1 (their m may still be -inf, and
            // -inf - -inf must not reach exp2); a first max gives alpha = 2^-inf = 0.
            const float alpha = need ? exp2_hw(m2 - t_max) : 1.f;
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
            m2 = need ? t_max : m2;
        }
        return m2 == -INFINITY ? 0.f : m2;
    };
    // p = 2^(s*c - m), lane-local partial sum, P^T packed to bf16 as the B operand.
    auto softmax_finish = [&](f32x16 (&s)[BC / 32], float m_use, bf16x8 (&pf)[BC / 16]) {
        float ps = 0.f;
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float x = fmaf(s[mb][r], c, -m_use);
                const float p = (r & 3) < POLY ? exp2_poly(x) : exp2_hw(x);
                s[mb][r] = p;
                ps += p;
            }
        lsum += ps;
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2) {
            const int mb = k2 >> 1, r0 = 8 * (k2 & 1);
            pf[k2] = as_bf16x8(u32x4{pack_bf16x2(s[mb][r0 + 0], s[mb][r0 + 1]),
                                     pack_bf16x2(s[mb][r0 + 2], s[mb][r0 + 3]),
                                     pack_bf16x2(s[mb][r0 + 4], s[mb][r0 + 5]),
                                     pack_bf16x2(s[mb][r0 + 6], s[mb][r0 + 7])});
        }
    };

    // ---- pipeline: tile j+1's QK is issued while tile j's softmax runs.
    // LDS: K buffers hold K_{j+1} (read now) and K_{j+2} (being copied in); V buffers hold
    // V_j (read now) and V_{j+1} (being copied in).  One barrier per tile.  The loop is
    // unrolled by two so that every buffer choice is a compile-time constant.
    f32x16 sA[BC / 32], sB[BC / 32];
    if (n_tiles > 0) {
        dma_tile(K, 0, k_lds0, false);
        dma_tile(V, 0, v_lds0, true);
        if (n_tiles > 1) dma_tile(K, 1, k_lds1, false);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4 v = vgpr_copy(q_raw[ks]);
            qf[ks] = as_bf16x8(q_row < N_q ? v : u32x4{0, 0, 0, 0});
        }
        wait_vmem();
        __syncthreads();
        // Unconditional (a wave with no rows to compute ignores the result).
        KFrag kf;
        load_k(k_lds0, kf);
        qk(kf, sA);
        __syncthreads();
    }

    auto step = [&](auto parity, int j, f32x16 (&s_cur)[BC / 32], f32x16 (&s_next)[BC / 32]) {
        constexpr bool odd = decltype(parity)::value;
        uint16_t* const k_fill = odd ? k_lds1 : k_lds0;  // receives K_{j+2}
        uint16_t* const k_read = odd ? k_lds0 : k_lds1;  // holds K_{j+1}
        uint16_t* const v_fill = odd ? v_lds0 : v_lds1;  // receives V_{j+1}
        uint16_t* const v_read = odd ? v_lds1 : v_lds0;  // holds V_j
        if (j + 2 < n_tiles) dma_tile(K, j + 2, k_fill, false);
        if (j + 1 < n_tiles) dma_tile(V, j + 1, v_fill, true);
        if (j < n_w) {
            bf16x8 pf[BC / 16];
            KFrag kf;
            VFrag vf;
            if constexpr (D == 64) {
                // K_{j+1} fragments are read once the max is known and V_j^T fragments
                // before the exps, so that few fragments are live at once (the register
                // budget of three workgroups per CU) and V's read latency overlaps the exps.
                const float m_use = softmax_prepare(s_cur, j);
                load_k(k_read, kf);
                // Tile j+1's scores, issued unconditionally so that the MFMAs share a basic
                // block with the exps below and overlap them.  Past this wave's last tile the
                // buffer holds other finite data and the result is never used.
                qk(kf, s_next);
                load_v(v_read, vf, std::integral_constant<int, 0>{}, std::integral_constant<int, BC / 16>{});
                softmax_finish(s_cur, m_use, pf);
                pv(vf, pf);
            } else {
                const float m_use = softmax_prepare(s_cur, j);
                load_k(k_read, kf);
                qk(kf, s_next);
                softmax_finish(s_cur, m_use, pf);
                load_v(v_read, vf, std::integral_constant<int, 0>{}, std::integral_constant<int, BC / 16>{});
                pv(vf, pf);
            }
        }
        wait_vmem();
        __syncthreads();
    };
    for (int j = 0; j < n_tiles; j += 2) {
        step(std::integral_constant<bool, false>{}, j, sA, sB);
        if (j + 1 < n_tiles) step(std::integral_constant<bool, true>{}, j + 1, sB, sA);
    }

    // Epilogue: O = acc / l (once), LSE = (m + log2 l) ln 2.  The wave stages its rows in its
    // own slice of the K buffers, which are idle: every read of the loop completed before its
    // last barrier, and no copy is in flight.
    lsum = half_swap_sum(lsum);
    static_assert(C::NW == 4 && C::TILE >= 64 * D, "two waves' rows per K buffer");
    store_rows_staged<D>(acc, lsum > 0.f ? 1.f / lsum : 0.f, (w < 2 ? k_lds0 : k_lds1) + (w & 1) * 32 * D,
                         O + q_base + (int64_t)q0w * D, N_q - q0w);
    if (hh == 0 && q_row < N_q)
        LSE[(int64_t)bh * N_q + q_row] = lsum > 0.f ? (m2 + log2_hw(lsum)) * kLn2 : -INFINITY;
  };

    // Order of a causal pair.  At d = 64 the long tile goes first: the workgroups of a head
    // start their long sweeps together and share every K/V tile in L2, and only the short
    // tiles' sweeps re-read (1.15x the algorithmic bytes; short-first measured 1.33x).  At
    // d = 128 the short tile goes first (the grouped-query workload moves 1.06x its
    // algorithmic bytes instead of 1.19x, the long causal one 1.23x instead of 1.25x; time
    // unchanged).
    constexpr bool kShortFirst = D == 128;
    const int first = CAUSAL && !kShortFirst ? T_r - 1 - rank : rank;
    run_tile(first);
    if (CAUSAL && rank != T_r - 1 - rank) {
        __syncthreads();  // the first tile's last LDS reads are done before the next prologue
        run_tile(first == rank ? T_r - 1 - rank : rank);
    }
}

template <int D, bool CAUSAL, int POLY = 0>
hipError_t launch_fwd_t(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                        int H_kv, int N_q, int N_k, float scale, hipStream_t stream) {
    constexpr int BR = FwdCfg<D>::BR;
    const int T_r = (N_q + BR - 1) / BR;
    const int BH = B * H;
    const float c = (float)((double)scale * 1.4426950408889634073599);
    const long long blocks = (long long)(CAUSAL ? (T_r + 1) / 2 : T_r) * BH;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, POLY>), dim3((unsigned)blocks), dim3(FwdCfg<D>::THREADS), 0, stream,
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

template <int POLY>
hipError_t launch_fwd_poly_t(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                             int H_kv, int N_q, int N_k, int d, bool causal, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_fwd_t<64, true, POLY>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream)
                      : launch_fwd_t<64, false, POLY>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream);
    return causal ? launch_fwd_t<128, true, POLY>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream)
                  : launch_fwd_t<128, false, POLY>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, scale, stream);
}

hipError_t launch_fwd_poly(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                           int H_kv, int N_q, int N_k, int d, bool causal, float scale, int poly_quarters,
                           hipStream_t stream) {
    switch (poly_quarters) {
        case 1: return launch_fwd_poly_t<1>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, stream);
        case 2: return launch_fwd_poly_t<2>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, stream);
        case 4: return launch_fwd_poly_t<4>(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, stream);
        default: return launch_fwd(Q, K, V, O, LSE, B, H, H_kv, N_q, N_k, d, causal, scale, stream);
    }
}

namespace {
__global__ __launch_bounds__(256) void exp2_poly_kernel(const float* __restrict__ x, float* __restrict__ y,
                                                        long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        y[i] = exp2_poly(x[i]);
}
}  // namespace

hipError_t launch_exp2_poly(const float* x, float* y, long long n, hipStream_t stream) {
    const long long blocks = std::min<long long>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(exp2_poly_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n);
    return hipGetLastError();
}

}  // namespace fa
