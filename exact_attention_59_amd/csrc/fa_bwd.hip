// fa_bwd.hip -- FlashAttention backward for gfx950 (bf16 in/out, fp32 accumulation).
//
// What is computed (Lecture 11 section 5.1): the gradients of sum(dO * O) with respect to
// Q, K and V, given dO and the forward's O and LSE.  P is recomputed on chip from the
// saved log-sum-exp (P = exp(S - LSE), one exp per score) instead of being stored:
//   D_i = dO_i . O_i                  (Exercise 6's identity; bwd_dq_kernel, per row)
//   dV  = P^T dO,   dP = dO V^T,   dS = P * (dP - D)
//   dK  = scale * dS^T Q              (bwd_dkdv_kernel: one workgroup per 128 keys)
//   dQ  = scale * dS K                (bwd_dq_kernel: one workgroup per 128 query rows)
// Each main kernel recomputes S and dP for its own outputs (seven matrix products instead of
// the section's five), so every gradient row is written by exactly one workgroup: no
// atomics, and the result does not depend on scheduling.
//
// Layouts follow the forward kernel: products on v_mfma_f32_32x32x16_bf16, LDS tiles
// row-major with XOR-swizzled 16-byte chunks.  Q and dO tiles (and K in the dQ kernel) are
// read both as rows (an MFMA operand along d) and as columns (ds_read_b64_tr_b16, an
// operand along the sequence); one swizzle keeps both kinds of read bank-conflict-free, so
// each tile is staged once.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

// Chunk swizzle serving both reads.  A row read (ds_read_b128) has 16 consecutive rows
// fetch the same logical chunk: their physical chunks must cover every bank once, which
// needs swz to be one-to-one on the row bits that select a bank group (r mod 16 at d=128,
// where a row spans all 64 banks; r/2 mod 8 at d=64, where two rows do).  A transposing
// read has 32 lanes fetch 4 rows x 4 consecutive chunks: bits 2-3 of swz must separate
// the 4 rows (at d=64 rows r and r+1 already sit in different bank halves, so bit 2 must
// separate r and r+2).  The low two bits of swz, taken from r/4, only permute chunks
// within an aligned group of 4 and keep the first property.
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

constexpr float kLog2e = 1.4426950408889634f;

// Copy rows [r0, r0 + ROWS) of a row-major [n_rows][D] bf16 matrix into an LDS tile (rows
// at or past n_rows repeat row n_rows - 1: finite data whose products are masked).  Each
// 64-lane copy moves 1 KB = 512 / D rows; the NW waves of a workgroup share the copies.
template <int D, int ROWS, int NW = 4>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ src, int r0, int n_rows, uint16_t* dst,
                                           int w, int lane) {
    constexpr int RPC = 512 / D;
    constexpr int NCOPY = ROWS / RPC;
#pragma unroll
    for (int u = 0; u < (NCOPY + NW - 1) / NW; ++u) {
        const int t = w + NW * u;
        if (NCOPY % NW == 0 || t < NCOPY) {  // wave-uniform
            const int r = t * RPC + lane / (D / 8);
            const int c = (lane % (D / 8)) ^ swz<D>(r);
            const uint16_t* g = src + (int64_t)min(r0 + r, n_rows - 1) * D + 8 * c;
            copy_to_lds16(g, lds_addr(dst + t * 512));
        }
    }
}

// Per-lane read offsets shared by both main kernels (elements within one LDS tile):
//   row_off[ks]: an operand along d -- row l32, logical chunk 2*ks + hh;
//   tr_lo[db], tr_hi[db]: the two transposing reads of a 32-d x 16-row slice (see the
//     forward kernel's P V product): lane (i = lane % 16) addresses row 4*hh + i/4 (and 8
//     rows further for tr_hi), logical chunk 4*db + cg, half 4*(i%2).  A later 16-row
//     slice adds 16*D: swz depends on r mod 16 only.
template <int D>
struct Offsets {
    int row[D / 16];
    int tr_lo[D / 32];
    int tr_hi[D / 32];
};

template <int D>
__device__ __forceinline__ Offsets<D> operand_offsets(int lane) {
    Offsets<D> o;
    const int l32 = lane & 31, hh = lane >> 5;
    const int sr = swz<D>(l32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) o.row[ks] = l32 * D + 8 * ((2 * ks + hh) ^ sr);
    const int i = lane & 15;
    const int R = 4 * hh + (i >> 2);
    const int cg = 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        o.tr_lo[db] = R * D + 8 * ((4 * db + cg) ^ swz<D>(R)) + 4 * (i & 1);
        o.tr_hi[db] = (R + 8) * D + 8 * ((4 * db + cg) ^ swz<D>(R + 8)) + 4 * (i & 1);
    }
    return o;
}

// 8 sequence positions x 1 d for the operand slot of 16-step k2 (two transposing reads):
// element e comes from row 16*k2 + 4*hh + e (e < 4) or 16*k2 + 8 + 4*hh + e - 4.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, const Offsets<D>& o, int db, int k2) {
    const i16x4 lo = lds_read_tr16(tile + o.tr_lo[db] + 16 * k2 * D);
    const i16x4 hi = lds_read_tr16(tile + o.tr_hi[db] + 16 * k2 * D);
    return __builtin_bit_cast(bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// The B operand fragments of a row (q . k along d): lane holds row[16*ks + 8*hh + e].
// Loading takes two calls, so that several rows' loads (and a prologue's tile copies) are in
// flight before the wave waits for any of them: issue_row_loads reads a row that must be
// readable (callers clamp the index; no branch), take_row_frags takes the values through
// the opaque copy once they are needed and zeroes those of a row that is not valid.
template <int D>
__device__ __forceinline__ void issue_row_loads(const uint16_t* row, int hh, u32x4 (&raw)[D / 16]) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + 8 * hh);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) raw[ks] = p[2 * ks];
}
template <int D>
__device__ __forceinline__ void take_row_frags(const u32x4 (&raw)[D / 16], bool valid, bf16x8 (&f)[D / 16]) {
    asm volatile("" ::: "memory");  // the loads issued so far stay ahead of the first wait
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 v = vgpr_copy(raw[ks]);
        f[ks] = as_bf16x8(valid ? v : u32x4{0, 0, 0, 0});
    }
}

// ---------------------------------------------------------------------------- dQ
// One workgroup of 4 waves per (b, h, 128 query rows); wave w owns 32 rows, lane = row.
// Its prologue also forms D_i = dO_i . O_i of its rows and writes it for the dK/dV kernel.
// Per key tile: S^T = K Q^T and dP^T = V dO^T (A = K, V rows), P^T = 2^(c S^T - L2),
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (A = K^T through transposing reads of the same
// K tile).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE, float* __restrict__ Dv,
                                                        uint16_t* __restrict__ dQ, int H, int H_kv, int N_q, int N_k,
                                                        int T_r, int BH, float c, float scale) {
    constexpr int BR = kBwdBlockRows, BC = bwd_dq_block_cols(D), TILE = BC * D;
    __shared__ __attribute__((aligned(1024))) uint16_t k_s0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t k_s1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s1[TILE];
    asm volatile("" ::"s"(dQ));  // consume the scalar load before the loop (see the forward kernel)

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    int bh, rank;
    // Under the causal mask a workgroup takes the pair of query tiles (T_r-1-rank, rank), so
    // that every workgroup carries the same work (no tail of long tiles).
    const int n_ranks = CAUSAL ? (T_r + 1) / 2 : T_r;
    map_block_xcd(blockIdx.x, n_ranks, BH, H / H_kv, bh, rank);
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / H_kv);
    const int64_t q_base = (int64_t)bh * N_q * D;
    const int64_t kv_base = (int64_t)(b * H_kv + g) * N_k * D;
    const int off = N_k - N_q;
    const int T_c = (N_k + BC - 1) / BC;

  auto run = [&](const int q_tile) {
    const int q0w = q_tile * BR + w * 32, q_row = q0w + l32;
    int n_tiles = T_c, n_w = T_c;  // tiles the workgroup stages / this wave computes
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

    // Row constants: L2 = LSE * log2(e) (+inf for a row without a visible key or past N_q,
    // which makes its P zero), and D.
    // All loads are issued (rows clamped to N_q - 1) before any value is taken.
    const int q_ld = min(q_row, N_q - 1);
    const float lse_raw = LSE[(int64_t)bh * N_q + q_ld];
    u32x4 q_raw[D / 16], do_raw[D / 16], o_raw[D / 16];
    issue_row_loads<D>(Q + q_base + (int64_t)q_ld * D, hh, q_raw);
    issue_row_loads<D>(dO + q_base + (int64_t)q_ld * D, hh, do_raw);
    issue_row_loads<D>(O + q_base + (int64_t)q_ld * D, hh, o_raw);
    bf16x8 qf[D / 16], dof[D / 16];
    take_row_frags<D>(q_raw, q_row < N_q, qf);
    take_row_frags<D>(do_raw, q_row < N_q, dof);
    const float l2 = q_row < N_q ? (lse_raw == -INFINITY ? INFINITY : lse_raw * kLog2e) : INFINITY;
    // D = dO . O of this row (Exercise 6's identity): each half of the wave holds half of the
    // row's elements of dO (dof) and of O; the halves are added.  Written for the dK/dV kernel.
    float dd = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = vgpr_copy(o_raw[ks]);
        const u32x4 gv = __builtin_bit_cast(u32x4, dof[ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dd = fmaf(bf16_bits_to_f32(a[e] & 0xffffu), bf16_bits_to_f32(gv[e] & 0xffffu), dd);
            dd = fmaf(bf16_bits_to_f32(a[e] >> 16), bf16_bits_to_f32(gv[e] >> 16), dd);
        }
    }
    dd = half_swap_sum(dd);  // rows past N_q: dof is zero, so dd = 0
    if (hh == 0 && q_row < N_q) Dv[(int64_t)bh * N_q + q_row] = dd;
    const Offsets<D> o = operand_offsets<D>(lane);

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    auto stage = [&](int j, uint16_t* ks, uint16_t* vs) {
        stage_tile<D, BC>(K + kv_base, j * BC, N_k, ks, w, lane);
        stage_tile<D, BC>(V + kv_base, j * BC, N_k, vs, w, lane);
    };
    auto compute = [&](int j, const uint16_t* ks, const uint16_t* vs) {
        f32x16 st[BC / 32], dpt[BC / 32];
#pragma unroll
        for (int mb = 0; mb < BC / 32; ++mb) st[mb] = dpt[mb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int mb = 0; mb < BC / 32; ++mb) {
                st[mb] = mfma32(*reinterpret_cast<const bf16x8*>(ks + o.row[kk] + 32 * mb * D), qf[kk], st[mb]);
                dpt[mb] = mfma32(*reinterpret_cast<const bf16x8*>(vs + o.row[kk] + 32 * mb * D), dof[kk], dpt[mb]);
            }
        // register r of block mb holds key key0 + 32*mb + 8*(r/4) + 4*hh + r%4
        const int key0 = j * BC;
        const bool edge = key0 + BC > N_k || (CAUSAL && key0 + BC - 1 > q0w + off);
        const int lim = (CAUSAL ? min(N_k - 1, q_row + off) : N_k - 1) - key0 - 4 * hh;  // last visible key
        bf16x8 dsf[BC / 16];
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2) {
            const int mb = k2 >> 1, r0 = 8 * (k2 & 1);
            float ds[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = r0 + e;
                float p = exp2_hw(fmaf(st[mb][r], c, -l2));
                if (edge && 32 * mb + 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
                ds[e] = p * (dpt[mb][r] - dd);
            }
            dsf[k2] = as_bf16x8(u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                                      pack_bf16x2(ds[6], ds[7])});
        }
#pragma unroll
        for (int k2 = 0; k2 < BC / 16; ++k2)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(tr_frag<D>(ks, o, db, k2), dsf[k2], acc[db]);
    };

    if (n_tiles > 0) {
        stage(0, k_s0, v_s0);
        wait_vmem();
        __syncthreads();
    }
    for (int j = 0; j < n_tiles; j += 2) {
        if (j + 1 < n_tiles) stage(j + 1, k_s1, v_s1);
        if (j < n_w) compute(j, k_s0, v_s0);
        wait_vmem();
        __syncthreads();
        if (j + 1 >= n_tiles) break;
        if (j + 2 < n_tiles) stage(j + 2, k_s0, v_s0);
        if (j + 1 < n_w) compute(j + 1, k_s1, v_s1);
        wait_vmem();
        __syncthreads();
    }

    // dQ = scale * acc (register r of acc[db] holds d = 32*db + 8*(r/4) + 4*hh + r%4), staged
    // in the wave's own tile buffer (idle: every read of the loop completed before its last
    // barrier, and no copy is in flight) and stored as whole rows.
    static_assert(TILE >= 32 * D, "a tile buffer holds a wave's 32 rows");
    store_rows_staged<D>(acc, scale, w == 0 ? k_s0 : w == 1 ? k_s1 : w == 2 ? v_s0 : v_s1,
                         dQ + q_base + (int64_t)q0w * D, N_q - q0w);
  };

    run(CAUSAL ? T_r - 1 - rank : rank);
    if (CAUSAL && rank != T_r - 1 - rank) {
        __syncthreads();  // the first tile's last LDS reads are done before the next prologue
        run(rank);
    }
}

// ---------------------------------------------------------------------------- dK, dV
// One workgroup of 4 waves per (b, key/value head, 128 keys); wave w owns 32 keys, lane =
// key.  K and V rows of the wave sit in registers as B operands (used at d = 64; at d = 128
// they and the two accumulators do not fit one wave: see bwd_dkdv_pair_kernel).  The
// workgroup walks the queries of every query head of the group, staging 64 query rows of Q
// and dO per barrier and computing them as two 32-row halves (one barrier and one round of
// copies per 64 rows instead of per 32).  Per half: S = Q K^T and dP = dO V^T (A = Q, dO
// rows), P = 2^(c S - L2), dS = P (dP - D); then dV += P^T dO and dK += dS^T Q, with P^T and
// dS^T already in A-operand layout (the query index of the contraction permuted to match)
// and dO, Q as B operands through transposing reads of the same tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ LSE, const float* __restrict__ Dv,
                                                          uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H,
                                                          int H_kv, int N_q, int N_k, int T_k, int BG, float c,
                                                          float scale) {
    constexpr int BK = kBwdBlockKeys, BQ = kBwdBlockQueries, SUB = 2, SQ = SUB * BQ, QT = SQ * D;
    __shared__ __attribute__((aligned(1024))) uint16_t q_s0[QT];
    __shared__ __attribute__((aligned(1024))) uint16_t q_s1[QT];
    __shared__ __attribute__((aligned(1024))) uint16_t o_s0[QT];  // dO
    __shared__ __attribute__((aligned(1024))) uint16_t o_s1[QT];
    __shared__ __attribute__((aligned(16))) float ld_s[2][2 * SQ];  // [buffer][L2 of the tile's rows, then D]
    asm volatile("" ::"s"(dK), "s"(dV));

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    // Under the causal mask a workgroup takes the pair of key tiles (kr, T_k-1-kr): early keys
    // are seen by many query tiles, late ones by few, and the pair evens the work out.
    int bg, kr;
    const int n_ranks = CAUSAL ? (T_k + 1) / 2 : T_k;
    map_block_xcd(blockIdx.x, n_ranks, BG, 1, bg, kr);
    const int b = bg / H_kv, g = bg - b * H_kv;
    const int group = H / H_kv;
    const int64_t kv_base = (int64_t)bg * N_k * D;
    const int off = N_k - N_q;
  auto run = [&](const int kt) {
    const int k0w = kt * BK + w * 32, key = k0w + l32;

    // Query tiles that can see a key of this workgroup (query q sees key k iff k <= q + off).
    const int n_qt = (N_q + SQ - 1) / SQ;
    const int qt0 = CAUSAL ? min(n_qt, max(0, kt * BK - off) / SQ) : 0;
    const int per_head = n_qt - qt0;
    const int n_steps = group * per_head;

    const Offsets<D> o = operand_offsets<D>(lane);
    bf16x8 kf[D / 16], vf[D / 16];
    u32x4 k_raw[D / 16], v_raw[D / 16];
    issue_row_loads<D>(K + kv_base + (int64_t)min(key, N_k - 1) * D, hh, k_raw);
    issue_row_loads<D>(V + kv_base + (int64_t)min(key, N_k - 1) * D, hh, v_raw);

    f32x16 accK[D / 32], accV[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) accK[db] = accV[db] = f32x16{};

    // Step s -> query head and tile.
    auto head_of = [&](int s) { return g * group + s / per_head; };
    auto q0_of = [&](int s) { return (qt0 + s % per_head) * SQ; };
    auto stage = [&](int s, uint16_t* qs, uint16_t* os) {
        const int64_t base = ((int64_t)b * H + head_of(s)) * N_q * D;
        const int q0 = q0_of(s);
        stage_tile<D, SQ>(Q + base, q0, N_q, qs, w, lane);
        stage_tile<D, SQ>(dO + base, q0, N_q, os, w, lane);
    };
    // Row constants of a tile (waves w < SUB: lanes 0..31 L2 of rows q0 + 32*w + lane, lanes
    // 32..63 D), loaded at the start of a step and stored to LDS at its end.  The load is
    // unconditional (row clamped to N_q - 1, source picked per lane) and the value is fixed
    // up only where it is stored: a per-lane choice between loads makes the wave wait for
    // the load -- and so for the tile copies issued just before it -- before the step's work.
    auto load_ld = [&](int s) -> float {
        const int64_t rb = ((int64_t)b * H + head_of(s)) * N_q;
        const int q = min(q0_of(s) + 32 * w + l32, N_q - 1);
        return (hh == 0 ? LSE : Dv)[rb + q];
    };
    auto fix_ld = [&](int s, float v) -> float {
        if (q0_of(s) + 32 * w + l32 >= N_q) return hh == 0 ? INFINITY : 0.f;  // rows past N_q: P = 0
        return hh == 0 ? (v == -INFINITY ? INFINITY : v * kLog2e) : v;
    };
    auto compute_sub = [&](int q0, const uint16_t* qs, const uint16_t* os, const float* l2p, const float* ddp) {
        if (CAUSAL && q0 + BQ - 1 + off < k0w) return;  // no row of the tile sees a key of this wave
        f32x16 st = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            st = mfma32(*reinterpret_cast<const bf16x8*>(qs + o.row[kk]), kf[kk], st);
            dp = mfma32(*reinterpret_cast<const bf16x8*>(os + o.row[kk]), vf[kk], dp);
        }
        __builtin_amdgcn_sched_barrier(0);
        // register r holds query q0 + 8*(r/4) + 4*hh + r%4, key = lane's key
        const bool edge = CAUSAL && k0w + 31 > q0 + off;  // some (row, key) pair is masked
        bf16x8 pa[2], dsa[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float p[8], ds[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 8 * t + e;
                const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
                p[e] = exp2_hw(fmaf(st[r], c, -l2p[qr]));
                if (edge && key > q0 + qr + off) p[e] = 0.f;
                ds[e] = p[e] * (dp[r] - ddp[qr]);
            }
            pa[t] = as_bf16x8(u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                    pack_bf16x2(p[6], p[7])});
            dsa[t] = as_bf16x8(u32x4{pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                                     pack_bf16x2(ds[6], ds[7])});
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                accV[db] = mfma32(pa[t], tr_frag<D>(os, o, db, t), accV[db]);
                accK[db] = mfma32(dsa[t], tr_frag<D>(qs, o, db, t), accK[db]);
            }
    };
    auto compute = [&](int s, const uint16_t* qs, const uint16_t* os, const float* lds_ld) {
#pragma unroll
        for (int h = 0; h < SUB; ++h)
            compute_sub(q0_of(s) + BQ * h, qs + BQ * h * D, os + BQ * h * D, lds_ld + BQ * h, lds_ld + SQ + BQ * h);
    };
    const int ld_slot = (lane >> 5) * SQ + 32 * w + (lane & 31);  // waves 0..SUB-1 load row constants

    float ld0 = 0.f;
    if (n_steps > 0) {
        stage(0, q_s0, o_s0);
        if (w < SUB) ld0 = load_ld(0);
    }
    take_row_frags<D>(k_raw, key < N_k, kf);
    take_row_frags<D>(v_raw, key < N_k, vf);
    if (n_steps > 0 && w < SUB) ld_s[0][ld_slot] = fix_ld(0, ld0);
    wait_vmem();
    __syncthreads();
    for (int s = 0; s < n_steps; s += 2) {
        float nxt = 0.f;
        if (s + 1 < n_steps) {
            stage(s + 1, q_s1, o_s1);
            if (w < SUB) nxt = load_ld(s + 1);
        }
        __builtin_amdgcn_sched_barrier(0);  // the fix-up of nxt stays after the step's work
        compute(s, q_s0, o_s0, ld_s[0]);
        if (w < SUB && s + 1 < n_steps) ld_s[1][ld_slot] = fix_ld(s + 1, nxt);
        wait_vmem();
        __syncthreads();
        if (s + 1 >= n_steps) break;
        if (s + 2 < n_steps) {
            stage(s + 2, q_s0, o_s0);
            if (w < SUB) nxt = load_ld(s + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        compute(s + 1, q_s1, o_s1, ld_s[1]);
        if (w < SUB && s + 2 < n_steps) ld_s[0][ld_slot] = fix_ld(s + 2, nxt);
        wait_vmem();
        __syncthreads();
    }

    // dK = scale * accK, dV = accV (register r of lane holds key k0w + 8*(r/4) + 4*hh + r%4 at
    // d = 32*db + l32), staged in the wave's own Q/dO buffer (idle: every read of the loop
    // completed before its last barrier, and no copy is in flight) and stored as whole rows.
    static_assert(QT >= 2 * 32 * D, "a Q/dO buffer holds a wave's dK and dV rows");
    uint16_t* const slice = w == 0 ? q_s0 : w == 1 ? q_s1 : w == 2 ? o_s0 : o_s1;
    store_cols_staged<D>(accK, scale, slice, dK + kv_base + (int64_t)k0w * D, N_k - k0w);
    store_cols_staged<D>(accV, 1.f, slice + 32 * D, dV + kv_base + (int64_t)k0w * D, N_k - k0w);
  };

    run(kr);
    if (CAUSAL && kr != T_k - 1 - kr) {
        __syncthreads();  // the first tile's last LDS reads are done before the next prologue
        run(T_k - 1 - kr);
    }
}

// ---------------------------------------------------------------------------- dK, dV (wave pairs)
// One workgroup of 8 waves per (b, key/value head, 128 keys).  Waves w and w + 4 (which
// share a SIMD) own the same 32 keys, lane = key, and split the work of each 32-query
// tile: wave w ("P wave", K rows in registers) computes S = Q K^T, P = 2^(c S - L2), hands
// P to its partner through LDS and accumulates dV += P^T dO; wave w + 4 ("dS wave", V rows
// in registers) computes dP = dO V^T, takes P, forms dS = P (dP - D) and accumulates
// dK += dS^T Q.  Each wave holds one operand set and one 32 x D accumulator, and one
// wave's exp / dS arithmetic overlaps its partner's matrix products.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int H, int H_kv, int N_q, int N_k, int T_k, int BG,
    float c, float scale) {
    // A step stages SQ = 2 * BQ query rows and computes them as two BQ-row halves: one
    // exchange barrier and one copy round per 64 rows.
    constexpr int BK = kBwdBlockKeys, BQ = kBwdBlockQueries, SUB = 2, SQ = SUB * BQ, QT = SQ * D;
    __shared__ __attribute__((aligned(1024))) uint16_t q_s0[QT];
    __shared__ __attribute__((aligned(1024))) uint16_t q_s1[QT];
    __shared__ __attribute__((aligned(1024))) uint16_t o_s0[QT];  // dO
    __shared__ __attribute__((aligned(1024))) uint16_t o_s1[QT];
    __shared__ __attribute__((aligned(16))) float p_x[SUB][4][4][64][4];  // [half][pair][chunk][lane][4]: P, fp32
    __shared__ __attribute__((aligned(16))) float ld_s[2][2 * SQ];        // [buffer][L2 of the tile's rows, then D]
    asm volatile("" ::"s"(dK), "s"(dV));

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pr = w & 3;
    const bool ds_wave = w >= 4;
    const int l32 = lane & 31, hh = lane >> 5;
    // Under the causal mask a workgroup takes the pair of key tiles (kr, T_k-1-kr): early keys
    // are seen by many query tiles, late ones by few, and the pair evens the work out.
    int bg, kr;
    const int n_ranks = CAUSAL ? (T_k + 1) / 2 : T_k;
    map_block_xcd(blockIdx.x, n_ranks, BG, 1, bg, kr);
    const int b = bg / H_kv, g = bg - b * H_kv;
    const int group = H / H_kv;
    const int64_t kv_base = (int64_t)bg * N_k * D;
    const int off = N_k - N_q;
  auto run = [&](const int kt) {
    const int k0w = kt * BK + pr * 32, key = k0w + l32;

    const int n_qt = (N_q + SQ - 1) / SQ;
    const int qt0 = CAUSAL ? min(n_qt, max(0, kt * BK - off) / SQ) : 0;
    const int per_head = n_qt - qt0;
    const int n_steps = group * per_head;

    const Offsets<D> o = operand_offsets<D>(lane);
    bf16x8 frag[D / 16];  // K rows (P wave) or V rows (dS wave)
    u32x4 f_raw[D / 16];
    issue_row_loads<D>((ds_wave ? V : K) + kv_base + (int64_t)min(key, N_k - 1) * D, hh, f_raw);

    f32x16 acc[D / 32];  // dV (P wave) or dK (dS wave)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

    auto head_of = [&](int s) { return g * group + s / per_head; };
    auto q0_of = [&](int s) { return (qt0 + s % per_head) * SQ; };
    auto stage = [&](int s, uint16_t* qs, uint16_t* os) {
        const int64_t base = ((int64_t)b * H + head_of(s)) * N_q * D;
        const int q0 = q0_of(s);
        stage_tile<D, SQ, 8>(Q + base, q0, N_q, qs, w, lane);
        stage_tile<D, SQ, 8>(dO + base, q0, N_q, os, w, lane);
    };
    // Row constants (waves w < SUB: lanes 0..31 L2 of rows q0 + 32*w + lane, lanes 32..63 D):
    // unconditional load, value fixed up where it is stored (as in bwd_dkdv_kernel).
    auto load_ld = [&](int s) -> float {
        const int64_t rb = ((int64_t)b * H + head_of(s)) * N_q;
        const int q = min(q0_of(s) + 32 * w + l32, N_q - 1);
        return (hh == 0 ? LSE : Dv)[rb + q];
    };
    auto fix_ld = [&](int s, float v) -> float {
        if (q0_of(s) + 32 * w + l32 >= N_q) return hh == 0 ? INFINITY : 0.f;  // rows past N_q: P = 0
        return hh == 0 ? (v == -INFINITY ? INFINITY : v * kLog2e) : v;
    };
    const int ld_slot = hh * SQ + 32 * w + l32;  // waves 0..SUB-1 load row constants
    // P exchange of half h: chunk j at px[h][64 * j]
    float4* px[SUB];
#pragma unroll
    for (int h = 0; h < SUB; ++h) px[h] = reinterpret_cast<float4*>(&p_x[h][pr][0][lane][0]);

    // One step (two BQ-row halves): both waves of a pair take part in the exchange barrier.
    auto step = [&](int s, const uint16_t* qs, const uint16_t* os, const float* lds_ld) {
        const int q0 = q0_of(s);
        f32x16 x[SUB];
        bf16x8 a_op[SUB][2];
        bool act[SUB];
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            const int q0h = q0 + BQ * h;
            act[h] = !(CAUSAL && q0h + BQ - 1 + off < k0w);  // some row of the half sees a key of the pair
            x[h] = f32x16{};
            if (act[h]) {
                const uint16_t* rows = (ds_wave ? os : qs) + BQ * h * D;
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
                    x[h] = mfma32(*reinterpret_cast<const bf16x8*>(rows + o.row[kk]), frag[kk], x[h]);
                if (!ds_wave) {
                    // register r holds query q0h + 8*(r/4) + 4*hh + r%4
                    const bool edge = CAUSAL && k0w + 31 > q0h + off;
                    float p[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
                        p[r] = exp2_hw(fmaf(x[h][r], c, -lds_ld[BQ * h + qr]));
                        if (edge && key > q0h + qr + off) p[r] = 0.f;
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        px[h][64 * j] = make_float4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        a_op[h][t] = as_bf16x8(u32x4{pack_bf16x2(p[8 * t + 0], p[8 * t + 1]), pack_bf16x2(p[8 * t + 2], p[8 * t + 3]),
                                                     pack_bf16x2(p[8 * t + 4], p[8 * t + 5]), pack_bf16x2(p[8 * t + 6], p[8 * t + 7])});
                }
            }
        }
        __syncthreads();  // P of both halves is in LDS
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            if (!act[h]) continue;
            if (ds_wave) {
                float ds[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 pv = px[h][64 * j];
                    const float pj[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * j + e;
                        const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
                        ds[r] = pj[e] * (x[h][r] - lds_ld[SQ + BQ * h + qr]);
                    }
                }
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    a_op[h][t] = as_bf16x8(u32x4{pack_bf16x2(ds[8 * t + 0], ds[8 * t + 1]), pack_bf16x2(ds[8 * t + 2], ds[8 * t + 3]),
                                                 pack_bf16x2(ds[8 * t + 4], ds[8 * t + 5]), pack_bf16x2(ds[8 * t + 6], ds[8 * t + 7])});
            }
            const uint16_t* cols = (ds_wave ? qs : os) + BQ * h * D;  // dK += dS^T Q, dV += P^T dO
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) acc[db] = mfma32(a_op[h][t], tr_frag<D>(cols, o, db, t), acc[db]);
        }
    };

    float ld0 = 0.f;
    if (n_steps > 0) {
        stage(0, q_s0, o_s0);
        if (w < SUB) ld0 = load_ld(0);
    }
    take_row_frags<D>(f_raw, key < N_k, frag);
    if (n_steps > 0 && w < SUB) ld_s[0][ld_slot] = fix_ld(0, ld0);
    wait_vmem();
    __syncthreads();
    for (int s = 0; s < n_steps; s += 2) {
        float nxt = 0.f;
        if (s + 1 < n_steps) {
            stage(s + 1, q_s1, o_s1);
            if (w < SUB) nxt = load_ld(s + 1);
        }
        __builtin_amdgcn_sched_barrier(0);  // the fix-up of nxt stays after the step's work
        step(s, q_s0, o_s0, ld_s[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (w < SUB && s + 1 < n_steps) ld_s[1][ld_slot] = fix_ld(s + 1, nxt);
        wait_vmem();
        __syncthreads();
        if (s + 1 >= n_steps) break;
        if (s + 2 < n_steps) {
            stage(s + 2, q_s0, o_s0);
            if (w < SUB) nxt = load_ld(s + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        step(s + 1, q_s1, o_s1, ld_s[1]);
        __builtin_amdgcn_sched_barrier(0);
        if (w < SUB && s + 2 < n_steps) ld_s[0][ld_slot] = fix_ld(s + 2, nxt);
        wait_vmem();
        __syncthreads();
    }

    // register r of lane holds key k0w + 8*(r/4) + 4*hh + r%4 at d = 32*db + l32; staged in
    // half of a Q/dO buffer (idle: every read of the loop completed before its last barrier, and
    // no copy is in flight) and stored as whole rows.
    static_assert(QT >= 2 * 32 * D, "a Q/dO buffer holds two waves' rows");
    uint16_t* const slice = (w < 4 ? (w < 2 ? q_s0 : q_s1) : (w < 6 ? o_s0 : o_s1)) + (w & 1) * 32 * D;
    store_cols_staged<D>(acc, ds_wave ? scale : 1.f, slice, (ds_wave ? dK : dV) + kv_base + (int64_t)k0w * D,
                         N_k - k0w);
  };

    run(kr);
    if (CAUSAL && kr != T_k - 1 - kr) {
        __syncthreads();  // the first tile's last LDS reads are done before the next prologue
        run(T_k - 1 - kr);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                        void* dQ, void* dK, void* dV, float* Dv, int B, int H, int H_kv, int N_q, int N_k,
                        float scale, hipStream_t stream) {
    const float c = (float)((double)scale * 1.4426950408889634073599);
    const int T_r = (N_q + kBwdBlockRows - 1) / kBwdBlockRows;
    const int n_qr = CAUSAL ? (T_r + 1) / 2 : T_r;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)n_qr * B * H)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                       static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(O),
                       static_cast<const uint16_t*>(dO), LSE, Dv,
                       static_cast<uint16_t*>(dQ), H, H_kv, N_q, N_k, T_r, B * H, c, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int T_k = (N_k + kBwdBlockKeys - 1) / kBwdBlockKeys;
    const int n_kr = CAUSAL ? (T_k + 1) / 2 : T_k;
    // d = 128: the wave-pair kernel (one wave cannot hold both accumulators and both
    // operand sets); d = 64: the single-wave kernel (measured 4% faster, same results).
    if constexpr (D == 128)
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)n_kr * B * H_kv)), dim3(512), 0,
                           stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                           static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(dO), LSE, Dv,
                           static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV), H, H_kv, N_q, N_k, T_k, B * H_kv, c,
                           scale);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)n_kr * B * H_kv)), dim3(256), 0,
                           stream, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                           static_cast<const uint16_t*>(V), static_cast<const uint16_t*>(dO), LSE, Dv,
                           static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV), H, H_kv, N_q, N_k, T_k, B * H_kv, c,
                           scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                      void* dQ, void* dK, void* dV, float* workspace, int B, int H, int H_kv, int N_q, int N_k, int d,
                      bool causal, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_bwd_t<64, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, H_kv, N_q, N_k,
                                               scale, stream)
                      : launch_bwd_t<64, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, H_kv, N_q, N_k,
                                                scale, stream);
    return causal ? launch_bwd_t<128, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, H_kv, N_q, N_k,
                                            scale, stream)
                  : launch_bwd_t<128, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, H_kv, N_q, N_k,
                                             scale, stream);
}

}  // namespace fa
