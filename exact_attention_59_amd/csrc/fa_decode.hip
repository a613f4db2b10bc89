// fa_decode.hip -- flash-decoding for gfx950: split-KV kernel and log-sum-exp combine.
//
// What is computed (Lecture 11 sections 6.1-6.4): one query token per sequence.  The
// cached keys are cut into S contiguous segments (views, no copy); a workgroup per
// (sequence, key/value head, segment) runs the online softmax over its segment and
// writes the segment's normalised output o_s and lse_s; the combine kernel merges the
// segments exactly: lse = log sum_s e^(lse_s), o = sum_s e^(lse_s - lse) o_s.
//
// Split kernel design (HBM-bound: every K/V byte is read exactly once):
//   - the H/H_kv query heads sharing a key/value head are packed as the N columns of
//     one MFMA tile (up to 16 per workgroup), so K and V are read once per group
//     (Lecture 11 section 6.2, GQA packing into the M dimension of the tile);
//   - the 4 waves of a workgroup take interleaved 32-key blocks of the segment and
//     keep independent online states; they are merged once at the end through LDS.
//     Waves never wait for each other inside the key loop;
//   - each wave keeps two blocks in flight beyond the one it computes (a two-slot
//     register ring, refilled as soon as a slot's data is consumed);
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16: a lane holds one query (lane % 16)
//     and 8 of every 32 keys; K goes straight from global memory into A-operand
//     registers, each load instruction reading whole 64-byte lines of 16 key rows;
//   - O^T += V^T P^T: V is written row-major (XOR-swizzled chunks) to the wave's own
//     LDS block and read back with the transposing LDS read in the key order of P^T.
#include <mutex>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

// ---- fa_decode_static: the one-launch decode with its partials and group counters in a
// file-scope device array instead of caller workspaces (for callers that cannot allocate).
// Layout: [counters: kStaticCounterBytes][LSE_part][O_part], each region 256-byte aligned.
// Each device holds its own copy for the life of the process; every call on a device uses
// that device's copy, so calls that overlap on one device race.  Host code uses the
// device address from hipGetSymbolAddress (static_scratch below), never this name.
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

namespace {

template <int D>
struct DecCfg {
    static constexpr int KB = kDecKeysPerWave;    // keys per block
    static constexpr int NQ = kDecHeadsPerBlock;  // query heads per workgroup (MFMA N)
    static constexpr int NW = 4;
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int KSTEPS = D / 32;         // contraction steps of S^T (32 d each)
    static constexpr int K_LOADS = 2 * KSTEPS;    // 16-byte K loads per lane per block
    static constexpr int V_LOADS = KB * CPR / 64; // 16-byte V loads per lane per block
    static constexpr int V_ELEMS = KB * D;        // one wave's LDS V block
    static constexpr int NQP = NQ + 4;            // padded query stride of the merge buffer
    static constexpr int MERGE_FLOATS = 2 * NW * NQ + NW * D * NQP;
    static constexpr int SMEM_BYTES =
        (NW * V_ELEMS * 2 > MERGE_FLOATS * 4) ? NW * V_ELEMS * 2 : MERGE_FLOATS * 4;
    static_assert(V_LOADS * 64 == KB * CPR, "V block must split evenly over the lanes");
};

// Chunk swizzle of the LDS V block: the transposing reads of one pass take 8 rows x 32
// contiguous bytes; XOR-ing the chunk index with an even per-row value keeps each 32-byte
// pair together and puts the 8 rows on distinct banks.
template <int D>
__device__ __forceinline__ int dec_swz(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }

// Paged key/value cache (PAGED = true): K and V are pools of pages [num_pages][H_kv][P][D]
// (P = 2^page_log2 >= 16 tokens of one head contiguous in a page); token t of sequence b
// lives in page block_table[b][t / P] at row t % P; seq_lens[b] tokens are valid.  A
// 32-key block starts at a multiple of 16 tokens, so each of its two 16-key halves lies in
// one page.  Lengths and table entries are clamped to the pool, so a bad table cannot
// address memory outside it.
struct PagedKV {
    const int* block_table;  // [B][max_pages]
    const int* seq_lens;     // [B]
    int page_log2, max_pages, num_pages;
};

// Split and combine in one launch (FUSE = true): a counter per (sequence, K/V head, head
// chunk) counts the workgroups that have written their segment's partials; the one that
// brings it to S merges the segments into O and LSE and sets the counter back to zero.
struct FusedOut {
    int* counters;  // [B][H_kv][n_qc], zero on entry
    uint16_t* O;    // [B][H][d] bf16
    float* LSE;     // [B][H] fp32, or null
};

// s_waitcnt operand that waits for every outstanding vector memory access (vmcnt = 0) and
// leaves the export and LDS/scalar counters at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool PAGED, bool FUSE>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(const uint16_t* __restrict__ Q,
                                                              const uint16_t* __restrict__ K,
                                                              const uint16_t* __restrict__ V,
                                                              float* __restrict__ O_part,
                                                              float* __restrict__ LSE_part, int H,
                                                              int H_kv, int N_k, int S, int L, int n_qc,
                                                              float c, PagedKV pg, FusedOut fz) {
    using C = DecCfg<D>;
    constexpr int KB = C::KB, NQ = C::NQ, NW = C::NW, CPR = C::CPR;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int n16 = lane & 15, hq = lane >> 4;

    int bid = blockIdx.x;
    const int s = bid % S;
    bid /= S;
    const int qc = bid % n_qc;
    const int bg = bid / n_qc;  // b * H_kv + g
    const int group = H / H_kv;
    const int b = bg / H_kv, g = bg - b * H_kv;

    // Keys [k_beg, k_end) of this sequence form segment s.  Paged: per-sequence length, and
    // segment lengths rounded up to whole 32-key blocks (so blocks start on 16-token rows).
    int len = N_k, seg = L;
    if constexpr (PAGED) {
        len = min(max(pg.seq_lens[b], 0), pg.max_pages << pg.page_log2);
        seg = ((len + S - 1) / S + KB - 1) / KB * KB;
    }
    const int k_beg = min(s * seg, len), k_end = min(k_beg + seg, len);
    const int nblk = (k_end - k_beg + KB - 1) / KB;
    const uint16_t* Kh = K + (int64_t)bg * N_k * D;  // contiguous layout
    const uint16_t* Vh = V + (int64_t)bg * N_k * D;

    // Query head of this lane's MFMA column.
    const int qh = qc * NQ + n16;  // index inside the group
    const bool q_valid = qh < group;
    const int h = g * group + qh;

    // Q fragment (B operand): lane holds Q[h][32*t + 8*hq + e] for step t.  The loads are
    // issued here and their values taken (through the opaque copy) only once the first
    // K/V blocks' loads are in flight as well, so that no wave waits on Q alone.
    // Columns past the group read the group's last head (finite values; their outputs are
    // never stored), so that the loads are unconditional like the K/V loads below.
    u32x4 q_raw[C::KSTEPS];
    {
        const int h_ld = q_valid ? h : g * group + group - 1;
        const u32x4* qp = reinterpret_cast<const u32x4*>(Q + ((int64_t)b * H + h_ld) * D + 8 * hq);
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) q_raw[t] = qp[4 * t];
    }
    bf16x8 qf[C::KSTEPS];

    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem) + w * C::V_ELEMS;

    // ---- block loads.  K: lane (n16, hq) holds row 16*mb + n16, d = 32*t + 8*hq + 0..7
    // (the 4 lanes of a row cover one 64-byte line per instruction).  V: lane holds row
    // v_kg*V_LOADS + r, chunk v_dc (V_LOADS divides 16: a lane's rows share a 16-key half).
    // Rows past the segment read the segment's last row again (a clamped in-bounds address,
    // finite data): their scores are masked to -inf, so they get P = 0 and add nothing.
    // The loads are unconditional (no zero fill), so that no wave waits on one block's
    // loads before the next block's are requested.
    const int v_dc = lane % CPR, v_kg = lane / CPR;
    static_assert(16 % C::V_LOADS == 0, "a lane's V rows stay in one 16-key half");

    // Paged cache: the block-table entries of this wave's first 32 * kPageWin blocks are read
    // once, into registers: the wave's block k (bi = w + NW * k) takes lanes 2k and 2k + 1 of
    // window k / 32, the pages of its keys key0 and key0 + 16.  Blocks take them with
    // v_readlane, so the loop reads no memory for them: a table read there would be a vector
    // load, awaited with the in-order vector-memory counter together with the other ring
    // slot's K/V loads.  Later blocks read the table directly.
    constexpr int kPageWin = 4;
    int pwin[kPageWin] = {0, 0, 0, 0};
    if constexpr (PAGED) {
        const int* bt = pg.block_table + (int64_t)b * pg.max_pages;
#pragma unroll
        for (int win = 0; win < kPageWin; ++win) {
            const int key0 = k_beg + (w + NW * (32 * win + (lane >> 1))) * KB;
            const int idx = ((lane & 1) ? key0 + 16 : key0) >> pg.page_log2;
            pwin[win] = bt[min(max(idx, 0), pg.max_pages - 1)];  // entries past the wave's blocks unused
        }
    }

    auto load_block = [&](int bi, u32x4 (&kr)[C::K_LOADS], u32x4 (&vr)[C::V_LOADS]) {
        const int key0 = k_beg + bi * KB;
        const bool full = key0 + KB <= k_end;
        // Row key0 + 16*half of K and V (half = 0, 1).
        const uint16_t *kh0, *kh1, *vh0, *vh1;
        if constexpr (PAGED) {
            const int P = 1 << pg.page_log2;
            const int k = (bi - w) / NW;  // this wave's k-th block (uniform)
            int e0, e1;
            if (k < 32 * kPageWin) {
                const int win = k >> 5, l0 = 2 * (k & 31);
                const int v = win == 0 ? pwin[0] : win == 1 ? pwin[1] : win == 2 ? pwin[2] : pwin[3];
                e0 = __builtin_amdgcn_readlane(v, l0);
                e1 = __builtin_amdgcn_readlane(v, l0 + 1);
            } else {
                // (taken wave-uniform, so that both paths meet in scalar registers and the
                // window path carries no wait for these loads)
                const int* bt = pg.block_table + (int64_t)b * pg.max_pages;
                e0 = __builtin_amdgcn_readfirstlane(bt[key0 >> pg.page_log2]);
                e1 = __builtin_amdgcn_readfirstlane(bt[min((key0 + 16) >> pg.page_log2, pg.max_pages - 1)]);
            }
            const int p0 = min(max(e0, 0), pg.num_pages - 1);
            const int p1 = min(max(e1, 0), pg.num_pages - 1);
            const int64_t o0 = (((int64_t)p0 * H_kv + g) * P + (key0 & (P - 1))) * D;
            const int64_t o1 = (((int64_t)p1 * H_kv + g) * P + ((key0 + 16) & (P - 1))) * D;
            kh0 = K + o0;
            kh1 = K + o1;
            vh0 = V + o0;
            vh1 = V + o1;
        } else {
            kh0 = Kh + (int64_t)key0 * D;
            kh1 = kh0 + 16 * D;
            vh0 = Vh + (int64_t)key0 * D;
            vh1 = vh0 + 16 * D;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int key = key0 + 16 * mb + n16;
            const int rel = (full ? key : min(key, k_end - 1)) - key0;  // in-bounds row
            const u32x4* kp = reinterpret_cast<const u32x4*>((rel >= 16 ? kh1 : kh0) + (rel & 15) * D + 8 * hq);
#pragma unroll
            for (int t = 0; t < C::KSTEPS; ++t) kr[mb * C::KSTEPS + t] = kp[4 * t];
        }
#pragma unroll
        for (int r = 0; r < C::V_LOADS; ++r) {
            const int key = key0 + v_kg * C::V_LOADS + r;
            const int rel = (full ? key : min(key, k_end - 1)) - key0;
            vr[r] = *reinterpret_cast<const u32x4*>((rel >= 16 ? vh1 : vh0) + (rel & 15) * D + v_dc * 8);
        }
    };

    // Transposing-read offsets for the PV A operand (V^T, M = 16 d, K = 32 keys): lane
    // (i = n16) of group hq reads row 16*x + 4*hq + i/4, d = 16*db + 4*(i%4) .. +3.
    int v_off[D / 16];
    {
        const int row = 4 * hq + (n16 >> 2);  // rows 16*x + row share the swizzle of row
        const int sw = dec_swz<D>(row);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const int chunk = 2 * db + ((n16 & 3) >> 1);
            v_off[db] = row * D + 8 * (chunk ^ sw) + 4 * (n16 & 1);
        }
    }

    float m2 = -INFINITY, lsum = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] = f32x4{};

    // Block bi's keys at or past `lim` (the segment's end) are masked.
    auto compute = [&](int bi, int lim, const u32x4 (&kr)[C::K_LOADS], const u32x4 (&vr)[C::V_LOADS],
                       auto&& refill) {
        // V block -> this wave's LDS (row-major, swizzled chunks)
#pragma unroll
        for (int r = 0; r < C::V_LOADS; ++r) {
            const int row = v_kg * C::V_LOADS + r;
            *reinterpret_cast<u32x4*>(Vs + row * D + 8 * (v_dc ^ dec_swz<D>(row))) = vr[r];
        }
        // S^T[key][query] for two 16-key blocks
        f32x4 sc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sc[mb] = f32x4{};
#pragma unroll
            for (int t = 0; t < C::KSTEPS; ++t) sc[mb] = mfma16(as_bf16x8(kr[mb * C::KSTEPS + t]), qf[t], sc[mb]);
        }
        refill();  // this block's K registers are consumed; V is in LDS
        wave_lds_fence();
        // mask keys past the segment (only the last block can be short) or the whole block
        const int key0 = k_beg + bi * KB;
        if (key0 + KB > lim) {
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (key0 + 16 * mb + 4 * hq + r >= lim) sc[mb][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[mb][r]);
        mx = quad_row_max(mx);
        const float t_max = mx * c;
        if (t_max > m2) {  // per lane: the decode state is tiny, rescale whenever the max grows
            const float alpha = exp2_hw(m2 - t_max);  // 0 when m2 = -inf
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) acc[db] *= alpha;
            m2 = t_max;
        }
        const float m_use = m2 == -INFINITY ? 0.f : m2;
        float ps = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2_hw(fmaf(sc[mb][r], c, -m_use));
                sc[mb][r] = p;
                ps += p;
            }
        lsum += quad_row_sum(ps);
        // P^T as B operand: slot e <-> key 16*(e/4) + 4*hq + e%4.
        const bf16x8 pf = as_bf16x8(u32x4{pack_bf16x2(sc[0][0], sc[0][1]), pack_bf16x2(sc[0][2], sc[0][3]),
                                          pack_bf16x2(sc[1][0], sc[1][1]), pack_bf16x2(sc[1][2], sc[1][3])});
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const i16x4 lo = lds_read_tr16(Vs + v_off[db]);
            const i16x4 hi = lds_read_tr16(Vs + v_off[db] + 16 * D);
            acc[db] = mfma16(__builtin_bit_cast(bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}),
                             pf, acc[db]);
        }
        wave_lds_fence();  // every lane's reads of the V block are done before it is rewritten
    };

    // Two-slot register ring: while block i is computed, blocks i+NW and i+2*NW (this
    // wave's next two) are in flight.  Q's values are taken once the first two blocks'
    // loads are issued as well.
    u32x4 k0[C::K_LOADS], v0[C::V_LOADS], k1[C::K_LOADS], v1[C::V_LOADS];
    if (w < nblk) load_block(w, k0, v0);
    if (w + NW < nblk) load_block(w + NW, k1, v1);
#pragma unroll
    for (int t = 0; t < C::KSTEPS; ++t) qf[t] = as_bf16x8(vgpr_copy(q_raw[t]));
    for (int bi = w; bi < nblk; bi += 2 * NW) {
        compute(bi, k_end, k0, v0, [&] { if (bi + 2 * NW < nblk) load_block(bi + 2 * NW, k0, v0); });
        if (bi + NW < nblk)
            compute(bi + NW, k_end, k1, v1, [&] { if (bi + 3 * NW < nblk) load_block(bi + 3 * NW, k1, v1); });
    }

    // Merge the 4 wave states through LDS (reusing the V blocks).  The accumulators are laid
    // out d-major with a padded query stride, [NW][D][NQ + 4]: one store instruction (lanes
    // n16 = 0..15, hq = 0..3 at d = 16 db + 4 hq + r) and one load instruction below (16
    // columns d0 x 4 queries) each touch 64 distinct banks.
    __syncthreads();
    float* mm = reinterpret_cast<float*>(smem);  // [NW][NQ]
    float* ll = mm + NW * NQ;                    // [NW][NQ]
    float* aa = ll + NW * NQ;                    // [NW][D][NQP]
    constexpr int NQP = C::NQP;
    if (hq == 0) {
        mm[w * NQ + n16] = m2;
        ll[w * NQ + n16] = lsum;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) aa[(w * D + 16 * db + 4 * hq + r) * NQP + n16] = acc[db][r];
    __syncthreads();

    // 256 threads x (D/16) outputs: thread -> query n = tid / 16 and columns d0 + 16 k
    // (d0 = tid % 16, k < D/16): the 16 threads of a row interleave, so that one store
    // instruction writes 64 contiguous bytes per row (the one-launch path writes through
    // the L2, where each store instruction goes to memory as it is).
    constexpr int DPT = D / 16;
    constexpr int CS = 16;
    const int n = tid >> 4, d0 = tid & 15;
    const int qh_out = qc * NQ + n;
    if (qh_out < group) {
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, mm[v * NQ + n]);
        const int64_t row = ((int64_t)b * H + (g * group + qh_out)) * S + s;
        float o[DPT];
        float lse;
        if (M == -INFINITY) {
#pragma unroll
            for (int k = 0; k < DPT; ++k) o[k] = 0.f;
            lse = -INFINITY;
        } else {
            float wt[NW], l = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const float mv = mm[v * NQ + n];
                wt[v] = mv == -INFINITY ? 0.f : exp2_hw(mv - M);
                l = fmaf(wt[v], ll[v * NQ + n], l);
            }
            const float inv = 1.f / l;
#pragma unroll
            for (int k = 0; k < DPT; ++k) {
                float x = 0.f;
#pragma unroll
                for (int v = 0; v < NW; ++v) x = fmaf(wt[v], aa[(v * D + d0 + CS * k) * NQP + n], x);
                o[k] = x * inv;
            }
            lse = (M + log2_hw(l)) * kLn2;
        }
        if constexpr (FUSE) {
            // Agent-scope atomic stores write through this XCD's L2, so another XCD's
            // workgroup can read them once they have completed (see the count below).
#pragma unroll
            for (int k = 0; k < DPT; ++k)
                __hip_atomic_store(O_part + row * D + d0 + CS * k, o[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((tid & 15) == 0) __hip_atomic_store(LSE_part + row, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
#pragma unroll
            for (int k = 0; k < DPT; ++k) O_part[row * D + d0 + CS * k] = o[k];
            if ((tid & 15) == 0) LSE_part[row] = lse;
        }
    }

    if constexpr (FUSE) {
        // Flash-decoding in one launch: the last workgroup of this (sequence, K/V head, head
        // chunk) merges the S segments (the log-sum-exp merge of combine_kernel, taken online
        // over chunks of segments).  Ordering without a release fence, which at agent scope
        // writes back the XCD's whole L2 and cost ~24 us per launch here: the partials above
        // are agent-scope atomic stores, which write through the non-coherent L2; every
        // thread waits for its own stores to complete (vmcnt = 0) before the barrier, so when
        // thread 0 counts, all of this workgroup's partials are in memory.  The merging
        // workgroup reads them with agent-scope atomic loads, which do not hit a stale L2
        // line.
        __shared__ int is_last;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(fz.counters + (int64_t)bg * n_qc + qc, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            is_last = old == S - 1;
        }
        __syncthreads();
        if (is_last) {
            constexpr float kLog2e = 1.4426950408889634f;
            if (qh_out < group) {
                const int64_t hrow = (int64_t)b * H + (g * group + qh_out);
                const float* lp = LSE_part + hrow * S;
                const float* op = O_part + hrow * S * D + d0;
                // One pass over the segments, CH at a time with all of a chunk's loads in
                // flight: running maximum M, l = sum_s e^(lse_s - M), acc = sum_s e^(lse_s - M) o_s,
                // rescaled when M grows; lse = M + ln l and O = acc / l at the end.
                constexpr int CH = 16;
                float M = -INFINITY, l = 0.f, acc[DPT];
#pragma unroll
                for (int k = 0; k < DPT; ++k) acc[k] = 0.f;
                for (int t0 = 0; t0 < S; t0 += CH) {
                    float ls[CH], x[CH][DPT];
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const int t = min(t0 + j, S - 1);  // past the end: a repeat, weighted 0 below
                        ls[j] = ld_agent(lp + t);
#pragma unroll
                        for (int k = 0; k < DPT; ++k) x[j][k] = ld_agent(op + (int64_t)t * D + CS * k);
                    }
                    float Mc = M;
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        if (t0 + j >= S) ls[j] = -INFINITY;
                        Mc = fmaxf(Mc, ls[j]);
                    }
                    if (Mc == -INFINITY) continue;  // only empty segments so far
                    const float r = exp2_hw((M - Mc) * kLog2e);  // 0 while M = -inf
                    l *= r;
#pragma unroll
                    for (int k = 0; k < DPT; ++k) acc[k] *= r;
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const float w = exp2_hw((ls[j] - Mc) * kLog2e);  // 0 for empty segments
                        l += w;
#pragma unroll
                        for (int k = 0; k < DPT; ++k) acc[k] = fmaf(w, x[j][k], acc[k]);
                    }
                    M = Mc;
                }
                float o[DPT];
                float lse = -INFINITY;
                if (M != -INFINITY) {
                    const float inv = 1.f / l;
#pragma unroll
                    for (int k = 0; k < DPT; ++k) o[k] = acc[k] * inv;
                    lse = M + log2_hw(l) * kLn2;
                } else {
#pragma unroll
                    for (int k = 0; k < DPT; ++k) o[k] = 0.f;
                }
                uint16_t* dst = fz.O + hrow * D + d0;
#pragma unroll
                for (int k = 0; k < DPT; ++k) dst[CS * k] = (uint16_t)(pack_bf16x2(o[k], 0.f) & 0xffffu);
                if (fz.LSE && (tid & 15) == 0) fz.LSE[hrow] = lse;
            }
            if (tid == 0)  // ready for the next call
                __hip_atomic_store(fz.counters + (int64_t)bg * n_qc + qc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// One wave per (b, h): lse = M + ln l and O = acc / l, with M = max_s lse_s,
// l = sum_s e^(lse_s - M) and acc = sum_s e^(lse_s - M) o_s, taken online over chunks of CH
// segments: a chunk's LSE values and partial rows are all requested before any is used (one
// memory round trip per chunk, the kernel's whole cost at small S), then the running M, l
// and acc are rescaled if the chunk raises M.  Lane l holds columns DPL*l .. DPL*l + DPL-1.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ O_part,
                                                      const float* __restrict__ LSE_part,
                                                      uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                      int BH, int S) {
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int DPL = D / 64;  // outputs per lane
    constexpr int CH = 16;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= BH) return;
    const float* lp = LSE_part + (int64_t)row * S;
    const float* op = O_part + (int64_t)row * S * D + lane * DPL;
    float M = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int t0 = 0; t0 < S; t0 += CH) {
        float ls[CH], x[CH][DPL];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int t = min(t0 + j, S - 1);  // past the end: a repeat, weighted 0 below
            ls[j] = lp[t];
            if constexpr (DPL == 2) {
                const float2 v = *reinterpret_cast<const float2*>(op + (int64_t)t * D);
                x[j][0] = v.x;
                x[j][1] = v.y;
            } else {
                x[j][0] = op[(int64_t)t * D];
            }
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (t0 + j >= S) ls[j] = -INFINITY;
            Mc = fmaxf(Mc, ls[j]);
        }
        if (Mc == -INFINITY) continue;  // only empty segments so far
        const float r = exp2_hw((M - Mc) * kLog2e);  // 0 while M = -inf
        l *= r;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] *= r;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float w = exp2_hw((ls[j] - Mc) * kLog2e);  // 0 for empty segments
            l += w;
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, x[j][k], acc[k]);
        }
        M = Mc;
    }
    float o[DPL];
    float lse = -INFINITY;
    if (M != -INFINITY) {
        const float inv = 1.f / l;
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = acc[k] * inv;
        lse = M + log2_hw(l) * kLn2;
    } else {
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[k] = 0.f;
    }
    uint16_t* dst = O + (int64_t)row * D + lane * DPL;
    if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o[0], o[1]);
    } else {
        const uint32_t pk = pack_bf16x2(o[0], 0.f);
        *dst = (uint16_t)(pk & 0xffffu);
    }
    if (LSE && lane == 0) LSE[row] = lse;
}

template <int D, bool PAGED, bool FUSE = false>
hipError_t launch_decode_t(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                           int B, int H, int H_kv, int N_k, int S, float scale, const PagedKV& pg,
                           hipStream_t stream, const FusedOut& fz = FusedOut{nullptr, nullptr, nullptr}) {
    const int group = H / H_kv;
    const int n_qc = (group + kDecHeadsPerBlock - 1) / kDecHeadsPerBlock;
    const int L = (N_k + S - 1) / S;
    const float c = (float)((double)scale * 1.4426950408889634073599);
    const long long blocks = (long long)S * n_qc * B * H_kv;
    hipLaunchKernelGGL((decode_split_kernel<D, PAGED, FUSE>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), O_part, LSE_part, H, H_kv, N_k, S, L, n_qc, c, pg, fz);
    return hipGetLastError();
}

template <int D>
hipError_t launch_combine_t(const float* O_part, const float* LSE_part, void* O, float* LSE, int B, int H,
                            int S, hipStream_t stream) {
    const int BH = B * H;
    hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream, O_part,
                       LSE_part, static_cast<uint16_t*>(O), LSE, BH, S);
    return hipGetLastError();
}

__global__ void zero_ints_kernel(int* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Number of non-zero ints among p[0 .. n) into *out (one workgroup).
__global__ __launch_bounds__(256) void count_nonzero_kernel(const int* p, int n, int* out) {
    __shared__ int total;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    int c = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) c += p[i] != 0;
    atomicAdd(&total, c);
    __syncthreads();
    if (threadIdx.x == 0) *out = total;
}

constexpr int kMaxDevices = 64;

// Device address of this device's scratch array, looked up once per device (with that
// device current).  `fresh` is set on the first call on a device: its counters must be
// cleared before first use.
hipError_t static_scratch(unsigned char** out, bool* fresh) {
    static std::mutex mu;
    static unsigned char* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    *fresh = false;
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptr[dev] = static_cast<unsigned char*>(p);
        *fresh = true;
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t decode_static_bytes(int B, int H, int d, int num_splits) {
    const size_t rows = (size_t)B * H * num_splits;
    const size_t lse = (rows * sizeof(float) + 255) / 256 * 256;
    return kStaticCounterBytes + lse + rows * (size_t)d * sizeof(float);
}

hipError_t launch_decode_static(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int H_kv, int N_k, int d, int num_splits, float scale, hipStream_t stream) {
    unsigned char* base = nullptr;
    bool fresh = false;
    hipError_t e = static_scratch(&base, &fresh);
    if (e != hipSuccess) return e;
    int* counters = reinterpret_cast<int*>(base);
    if (fresh) {  // the group counters start at zero; every completed call leaves them zero
        hipLaunchKernelGGL(zero_ints_kernel, dim3(16), dim3(256), 0, stream, counters,
                           (int)(kStaticCounterBytes / sizeof(int)));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t rows = (size_t)B * H * num_splits;
    float* lse_part = reinterpret_cast<float*>(base + kStaticCounterBytes);
    float* o_part = reinterpret_cast<float*>(base + kStaticCounterBytes + (rows * sizeof(float) + 255) / 256 * 256);
    return launch_decode_fused(Q, K, V, o_part, lse_part, counters, O, LSE, B, H, H_kv, N_k, d, num_splits, scale,
                               stream);
}

hipError_t launch_counters_reset(int* counters, int n, hipStream_t stream) {
    hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)min((n + 255) / 256, 64)), dim3(256), 0, stream, counters, n);
    return hipGetLastError();
}

hipError_t launch_counters_check(const int* counters, int n, int* nonzero, hipStream_t stream) {
    hipLaunchKernelGGL(count_nonzero_kernel, dim3(1), dim3(256), 0, stream, counters, n, nonzero);
    return hipGetLastError();
}

hipError_t launch_decode_split(const void* Q, const void* K, const void* V, float* O_part,
                               float* LSE_part, int B, int H, int H_kv, int N_k, int d, int num_splits,
                               float scale, hipStream_t stream) {
    const PagedKV none{nullptr, nullptr, 0, 0, 0};
    if (d == 64)
        return launch_decode_t<64, false>(Q, K, V, O_part, LSE_part, B, H, H_kv, N_k, num_splits, scale, none,
                                          stream);
    return launch_decode_t<128, false>(Q, K, V, O_part, LSE_part, B, H, H_kv, N_k, num_splits, scale, none,
                                       stream);
}

hipError_t launch_decode_split_paged(const void* Q, const void* K_pages, const void* V_pages,
                                     const int* block_table, const int* seq_lens, float* O_part,
                                     float* LSE_part, int B, int H, int H_kv, int page_log2, int max_pages,
                                     int num_pages, int d, int num_splits, float scale, hipStream_t stream) {
    const PagedKV pg{block_table, seq_lens, page_log2, max_pages, num_pages};
    // N_k = 0: the contiguous layout is not used
    if (d == 64)
        return launch_decode_t<64, true>(Q, K_pages, V_pages, O_part, LSE_part, B, H, H_kv, 0, num_splits, scale,
                                         pg, stream);
    return launch_decode_t<128, true>(Q, K_pages, V_pages, O_part, LSE_part, B, H, H_kv, 0, num_splits, scale,
                                      pg, stream);
}

hipError_t launch_decode_paged_fused(const void* Q, const void* K_pages, const void* V_pages,
                                     const int* block_table, const int* seq_lens, float* O_part,
                                     float* LSE_part, int* counters, void* O, float* LSE, int B, int H, int H_kv,
                                     int page_log2, int max_pages, int num_pages, int d, int num_splits,
                                     float scale, hipStream_t stream) {
    const PagedKV pg{block_table, seq_lens, page_log2, max_pages, num_pages};
    const FusedOut fz{counters, static_cast<uint16_t*>(O), LSE};
    if (d == 64)
        return launch_decode_t<64, true, true>(Q, K_pages, V_pages, O_part, LSE_part, B, H, H_kv, 0, num_splits,
                                               scale, pg, stream, fz);
    return launch_decode_t<128, true, true>(Q, K_pages, V_pages, O_part, LSE_part, B, H, H_kv, 0, num_splits,
                                            scale, pg, stream, fz);
}

hipError_t launch_decode_fused(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                               int* counters, void* O, float* LSE, int B, int H, int H_kv, int N_k, int d,
                               int num_splits, float scale, hipStream_t stream) {
    const PagedKV none{nullptr, nullptr, 0, 0, 0};
    const FusedOut fz{counters, static_cast<uint16_t*>(O), LSE};
    if (d == 64)
        return launch_decode_t<64, false, true>(Q, K, V, O_part, LSE_part, B, H, H_kv, N_k, num_splits, scale,
                                                none, stream, fz);
    return launch_decode_t<128, false, true>(Q, K, V, O_part, LSE_part, B, H, H_kv, N_k, num_splits, scale, none,
                                             stream, fz);
}

hipError_t launch_combine(const float* O_part, const float* LSE_part, void* O, float* LSE, int B, int H,
                          int d, int num_splits, hipStream_t stream) {
    if (d == 64) return launch_combine_t<64>(O_part, LSE_part, O, LSE, B, H, num_splits, stream);
    return launch_combine_t<128>(O_part, LSE_part, O, LSE, B, H, num_splits, stream);
}

}  // namespace fa
