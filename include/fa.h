/*
 * fa.h -- C ABI of libfa.so: exact attention on AMD Instinct MI355X (gfx950).
 *
 * Compute entry points:
 *   fa_fwd           FlashAttention-2 forward: O = softmax(scale * Q K^T) V and the
 *                    per-row log-sum-exp, computed tile by tile with the online
 *                    softmax state (m, l, acc); S and P never reach device memory.
 *   fa_fwd_poly_exp2 the forward with part of the softmax exponentials taken by a
 *                    polynomial on the FMA units (FA4's exp2 trick).
 *   fa_bwd           FlashAttention backward: dQ, dK, dV from dO, recomputing P on
 *                    chip from the saved log-sum-exp.
 *   fa_decode_split  flash-decoding, step 2: one query token per sequence, keys cut
 *                    into num_splits contiguous segments, per-segment normalised
 *                    output o_s and lse_s.
 *   fa_decode_split_paged  the split step over a paged key/value cache
 *                    (block table, per-sequence lengths).
 *   fa_combine       flash-decoding, step 3: exact merge of the segments by
 *                    log-sum-exp.
 *   fa_decode        flash-decoding in one launch (split, then the merge by the
 *                    last workgroup of each group).
 *   fa_fp8_quantize  FP8 path, step 1: random-sign Hadamard transform of Q and K
 *                    and e4m3 block quantisation of Q, K, V.
 *   fa_fwd_fp8       FP8 path, step 2: the forward on fp8 matrix cores.
 * Sources: Lecture 11, "Kernel Optimization Techniques: FlashAttention,
 * flash-decoding and megakernel", sections 2-6; the FlashAttention v1 and v2
 * cards of the "CUDA Kernel interview course" page.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers (hipMalloc'd or equivalent), except where a
 *     parameter says otherwise.  The caller allocates and frees every buffer;
 *     the library allocates nothing and keeps no state besides a cached
 *     compute-unit count.
 *   - bf16 tensors are raw 16-bit bfloat16 storage (1 sign, 8 exponent, 7
 *     mantissa bits), passed as void*.  All tensors are dense, row-major, with
 *     the innermost dimension contiguous, and start on a 16-byte boundary.
 *     Outputs must not overlap inputs.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Calls are asynchronous: they enqueue work and return.  A launch failure
 *     reported by the HIP runtime returns FA_ERR_HIP; faults during execution
 *     surface at the caller's next synchronisation of the stream.
 *   - Arguments are validated before any HIP call.  On any error status the
 *     outputs are left untouched and nothing is enqueued.
 *   - Entry points are thread-safe and re-entrant.
 *   - Scores are scale * (q . k); LSE is the natural logarithm of the sum of
 *     exp(score) over the visible keys.  A row with no visible key gets O = 0
 *     and LSE = -inf.  NaN or Inf inputs propagate; they are not detected.
 *   - Query head h reads key/value head h / (H / H_kv) (contiguous groups).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,       /* a size is <= 0, H % H_kv != 0, or num_splits out of range */
    FA_ERR_UNSUPPORTED = 3, /* head dimension d not in {64, 128}, or a size beyond the limits below */
    FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
    FA_ERR_ARG = 5,         /* scale not finite and positive, or a 0/1 flag out of range */
    FA_ERR_HIP = 6,         /* the HIP runtime reported an error when enqueueing */
    FA_ERR_CAPACITY = 7     /* fa_decode_static: the problem does not fit its static scratch array */
} fa_status;

/*
 * Exact attention forward (FlashAttention-2 order: one workgroup per query tile,
 * K/V tiles streamed through LDS; Lecture 11 sections 4.1-4.2 and 5.3; the v2
 * card's work partitioning).
 *   Q   [B][H][N_q][d]    bf16, read
 *   K   [B][H_kv][N_k][d] bf16, read
 *   V   [B][H_kv][N_k][d] bf16, read
 *   O   [B][H][N_q][d]    bf16, written (round-to-nearest-even)
 *   LSE [B][H][N_q]       fp32, written (natural log)
 *   causal: 0 = no mask; 1 = bottom-right aligned causal mask, query i sees key j
 *           iff j <= i + N_k - N_q (the lower triangle when N_q == N_k).
 *   scale: multiplies q . k (usually 1/sqrt(d)); must be finite and > 0 (the row max
 *          is taken on unscaled scores).
 * Limits: d in {64, 128}; B*H*N_q*d and B*H_kv*N_k*d below 2^62.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int H_kv,
           int N_q, int N_k, int d, int causal, float scale, void* stream);

/*
 * The forward of fa_fwd with a software exponential for part of the softmax (the
 * FA4 softmax trick of computing some exponentials with a polynomial on the FMA units
 * instead of the transcendental unit; CUDA Kernel interview course, FlashAttention v4
 * card).  Of every four exponentials a lane takes, the first poly_quarters (1, 2 or 4)
 * use p(x) = 2^n * (1 + f (c1 + c2 f + c3 f^2)), x = n + f, n = floor(x), with a
 * minimax cubic of relative error <= 8.6e-5 (exact at integer x); the rest use
 * v_exp_f32.  Each probability then carries a relative error <= 8.6e-5, so LSE moves by
 * at most about 8.6e-5 and O by at most about 2 * 8.6e-5 * max|V| from fa_fwd's result.
 * Arguments, layouts and limits as for fa_fwd; poly_quarters outside {1, 2, 4} gives
 * FA_ERR_ARG.  On gfx950 the transcendental instruction costs less than the
 * polynomial's eight FMA-unit instructions, so this path is slower than fa_fwd; it is
 * offered for the error analysis and for hardware where the balance differs.
 */
int fa_fwd_poly_exp2(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int H_kv,
                     int N_q, int N_k, int d, int causal, float scale, int poly_quarters, void* stream);

/*
 * The polynomial exponential of fa_fwd_poly_exp2 on its own: y[i] = 2^x[i] for
 * 0 <= i < n, as the forward computes it (relative error <= 8.6e-5 for x >= -126;
 * x <= -200 and -inf give 0).  x and y are device arrays of n floats, 4-byte aligned;
 * n = 0 enqueues nothing.  For tests of the error bound.
 */
int fa_exp2_poly(const float* x, float* y, long long n, void* stream);

/*
 * Exact attention backward (Lecture 11 section 5.1): for the forward above with the
 * same Q, K, V, causal and scale, and the upstream gradient dO, computes
 *   D_i = dO_i . O_i,  P_ij = exp(scale * q_i . k_j - LSE_i) over the visible keys,
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
 * P is recomputed from LSE (section 5.1's one-exp recovery); S, P and dS never reach
 * device memory.  With grouped heads, dK and dV of key/value head g sum over the query
 * heads that read it.  Every gradient row is written by exactly one workgroup: no
 * atomics, and the result is the same on every call.
 *   Q, K, V, causal, scale  as for fa_fwd
 *   O   [B][H][N_q][d]    bf16, read (the forward's output)
 *   dO  [B][H][N_q][d]    bf16, read
 *   LSE [B][H][N_q]       fp32, read (the forward's; -inf marks a row with no visible key)
 *   dQ  [B][H][N_q][d]    bf16, written
 *   dK  [B][H_kv][N_k][d] bf16, written (zero for a key no query sees)
 *   dV  [B][H_kv][N_k][d] bf16, written
 *   workspace  fa_bwd_workspace_bytes(B, H, N_q) bytes of device memory, 16-byte
 *              aligned, owned by the caller; it receives D (fp32) and may be reused
 *              once the call's work on `stream` has finished.
 * Limits: as for fa_fwd.  The two kernels (dQ, which also writes D, then dK/dV) run
 * in order on `stream`.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
           void* dQ, void* dK, void* dV, float* workspace, int B, int H, int H_kv, int N_q, int N_k, int d,
           int causal, float scale, void* stream);

/* Bytes of workspace fa_bwd needs: 4 * B * H * N_q (0 if a size is <= 0). */
size_t fa_bwd_workspace_bytes(int B, int H, int N_q);

/*
 * FP8 (OCP e4m3) forward, in two calls.  What the pages fix (the FlashAttention v3 card of
 * the CUDA Kernel interview course, "FP8 path"; Lecture 11 section 4.4): one scale per
 * block, and a random orthogonal transform applied first so that outlier channels are
 * spread over all channels.  Readings taken where they are silent:
 *   - e4m3 = OCP e4m3fn (bias 7, largest finite 448, subnormals to 2^-9), nearest-even;
 *   - the transform is x -> (s o x) H with H the unnormalised Sylvester-Hadamard matrix
 *     (H H^T = d I) and s the signs given by the 128-bit mask (bit j of sign_hi:sign_lo set
 *     means channel j is negated); it is applied to Q and K (scores are unchanged up to the
 *     factor d, which the query scales carry), never to V;
 *   - blocks: 128 query rows, 64 keys (the forward's tiles; fa_fp8_block_rows);
 *     amax = max |x| over the block, code = e4m3(x * (448 / amax)) computed in fp32,
 *     scale = amax / 448 (times 1/d for transformed queries); all-zero block: scale 0.
 * Dequantised values are code * scale; the product of a dequantised query and key is the
 * original score up to rounding.
 *
 * fa_fp8_quantize: Q [B][H][N_q][d], K and V [B][H_kv][N_k][d] bf16, read.  Written:
 *   Q8      [B][H][N_q][d]       e4m3 bytes
 *   K8      [B][H_kv][N_k][d]    e4m3 bytes
 *   Vt8     [B][H_kv][T_c][d][64] e4m3 bytes, T_c = ceil(N_k / 64): tile t of key/value head
 *           (b, g) holds, in row j and position p = 32 h + e (h < 2, e < 32), the code of
 *           V[64 t + 32 (e/16) + 8 ((e%16)/4) + 4 h + e%4][j] (zero past N_k): each tile is
 *           transposed and its keys permuted into the order the forward's operands use
 *   q_scale [B][H][ceil(N_q / 128)] fp32;  k_scale, v_scale [B][H_kv][T_c] fp32
 *   incoherent: 1 = apply the transform, 0 = quantise Q and K as they are.
 * The codes and scales are a deterministic function of the inputs (bit-exact).
 * Alignment: tensors 16 bytes, scale arrays 4 bytes.
 *
 * fa_fwd_fp8: exact attention of the dequantised Q, K, V -- softmax(scale * q . k) v with
 * q . k = (Q8 q_scale) . (K8 k_scale) -- computed tile by tile as fa_fwd does, with P
 * rounded to e4m3 for the P V product.  O [B][H][N_q][d] bf16 and LSE [B][H][N_q] fp32 are
 * written; causal and scale as for fa_fwd.  All other arguments are fa_fp8_quantize's
 * outputs for the same shapes.
 */
int fa_fp8_block_rows(int* q_rows, int* kv_rows);

int fa_fp8_quantize(const void* Q, const void* K, const void* V, int incoherent, uint64_t sign_lo, uint64_t sign_hi,
                    void* Q8, void* K8, void* Vt8, float* q_scale, float* k_scale, float* v_scale, int B, int H,
                    int H_kv, int N_q, int N_k, int d, void* stream);

int fa_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, const float* q_scale, const float* k_scale,
               const float* v_scale, void* O, float* LSE, int B, int H, int H_kv, int N_q, int N_k, int d, int causal,
               float scale, void* stream);

/*
 * Flash-decoding split step (Lecture 11 section 6.2, steps 1-2): one query token
 * per sequence; the N_k cached keys are cut into num_splits contiguous segments of
 * L = ceil(N_k / num_splits) keys (the last ones may be short or empty).  The
 * H / H_kv query heads that share a key/value head are processed together, so
 * each K/V element is read once.  No causal mask (the single query sees every
 * cached key).
 *   Q        [B][H][d]               bf16, read
 *   K, V     [B][H_kv][N_k][d]       bf16, read
 *   O_part   [B][H][num_splits][d]   fp32, written: o_s, normalised within the segment
 *   LSE_part [B][H][num_splits]      fp32, written: lse_s (natural log); -inf and
 *                                     o_s = 0 for an empty segment
 * num_splits must lie in [1, N_k].  fa_decode_num_splits gives a default.
 * Limits: d in {64, 128}; H / H_kv <= 64.
 */
int fa_decode_split(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
                    int B, int H, int H_kv, int N_k, int d, int num_splits, float scale, void* stream);

/*
 * Flash-decoding split step over a paged key/value cache (Lecture 11, the
 * flash-decoding section and "State of the field": paged KV needs the attention
 * kernel to address keys indirectly through a block table).  Same computation as
 * fa_decode_split for sequence b over its first seq_lens[b] cached tokens, which
 * are scattered over fixed-size pages:
 *   Q           [B][H][d]                          bf16, read
 *   K_pages,
 *   V_pages     [num_pages][H_kv][page_size][d]    bf16, read: page p holds
 *               page_size consecutive tokens of every key/value head
 *   block_table [B][max_pages]                     int32, read: token t of sequence b
 *               is row t % page_size of page block_table[b][t / page_size]
 *   seq_lens    [B]                                int32, read: valid tokens per sequence
 *   O_part, LSE_part as for fa_decode_split.
 * Segment s of sequence b covers tokens [s*L_b, min((s+1)*L_b, seq_lens[b])), with
 * L_b = ceil(seq_lens[b] / num_splits) rounded up to a multiple of 32; later
 * segments may be empty (o_s = 0, lse_s = -inf), and a sequence of length 0 gives
 * O = 0, LSE = -inf after fa_combine.  Device-side values are not validated:
 * seq_lens[b] is clamped to [0, max_pages * page_size] and table entries to
 * [0, num_pages - 1], so a bad table cannot make the kernel read outside the pools.
 * block_table and seq_lens must be 4-byte aligned; the other pointers 16-byte.
 * Limits: d in {64, 128}; H / H_kv <= 64; page_size a power of two in
 * [16, 4096]; num_splits in [1, max_pages * page_size].
 */
int fa_decode_split_paged(const void* Q, const void* K_pages, const void* V_pages,
                          const int* block_table, const int* seq_lens, float* O_part,
                          float* LSE_part, int B, int H, int H_kv, int page_size, int max_pages,
                          int num_pages, int d, int num_splits, float scale, void* stream);

/*
 * Flash-decoding combine (Lecture 11 section 6.2, step 3): per (b, h),
 *   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) o_s,
 * evaluated with the largest lse_s subtracted first.  If every segment is empty,
 * O = 0 and LSE = -inf.
 *   O_part [B][H][num_splits][d] fp32 and LSE_part [B][H][num_splits] fp32, read
 *   O      [B][H][d]  bf16, written
 *   LSE    [B][H]     fp32, written (may be NULL if not wanted)
 */
int fa_combine(const float* O_part, const float* LSE_part, void* O, float* LSE, int B, int H,
               int d, int num_splits, void* stream);

/*
 * Flash-decoding in one launch (Lecture 11 section 6.2: the split step, then the
 * exact log-sum-exp merge; section 6.4 notes that the merge kernel's fixed cost
 * matters when segments are short): the split step of fa_decode_split, after
 * which the last workgroup to finish for each (sequence, K/V head, group of up
 * to 16 query heads) merges that group's segments as fa_combine does.  Results
 * equal fa_decode_split followed by fa_combine up to the summation order of the
 * merge.
 *   Q, K, V, O_part, LSE_part  as for fa_decode_split (O_part, LSE_part are the
 *                    caller's workspace, fa_decode_workspace_bytes; written)
 *   counters         int[fa_decode_counter_bytes(B, H, H_kv) / 4], device memory,
 *                    4-byte aligned; must be zero before the first call; every
 *                    completed call leaves them zero again.  Calls that overlap on
 *                    the same counters or workspace (other streams) race.  A
 *                    counter that is not zero on entry (never cleared, or shared by
 *                    overlapping calls) makes its group merge at the wrong time:
 *                    the output is wrong and the counter stays wrong.  The kernel
 *                    cannot detect this; fa_decode_counters_check reports such
 *                    counters and fa_decode_counters_reset clears them.
 * Ordering: every workgroup writes its partials with agent-scope atomic stores
 * (written through its XCD's non-coherent L2 to memory) and waits for them
 * (s_waitcnt vmcnt(0)) before the workgroup barrier; then one thread counts with
 * a relaxed agent-scope atomic add.  The counting workgroup therefore reaches the
 * counter only after its partials are in memory, and the merging workgroup reads
 * the partials with agent-scope atomic loads, which bypass a stale L2 line.  This
 * is the completion order a release/acquire pair would give, without its write-back
 * and invalidation of a whole L2 (measured: 42.8 us instead of 18.9 us at N_k=4096).
 *   O [B][H][d] bf16 and LSE [B][H] fp32 (LSE may be NULL) as for fa_combine
 * Validation and limits as for fa_decode_split; counters must be non-NULL.
 * Cost: measured back to back on MI355X (B=4, H=32, H_kv=8, d=128) this one
 * launch takes about the time of fa_decode_split + fa_combine (18.3 us against
 * 17.8 us at N_k=4096, 181 us against 180 us at 65536); it saves the caller the
 * second launch and its dependency.
 */
int fa_decode(const void* Q, const void* K, const void* V, float* O_part, float* LSE_part,
              int* counters, void* O, float* LSE, int B, int H, int H_kv, int N_k, int d,
              int num_splits, float scale, void* stream);

/*
 * fa_decode over a paged cache: the split step of fa_decode_split_paged, then
 * the same in-launch merge as fa_decode.  Results equal fa_decode_split_paged
 * followed by fa_combine up to the summation order of the merge.
 *   Q, K_pages, V_pages, block_table, seq_lens, O_part, LSE_part, page_size,
 *   max_pages, num_pages  as for fa_decode_split_paged
 *   counters, O, LSE      as for fa_decode (fa_decode_counter_bytes(B, H, H_kv))
 * Validation and limits as for fa_decode_split_paged; counters and O must be
 * non-NULL and aligned as for fa_decode.
 */
int fa_decode_paged(const void* Q, const void* K_pages, const void* V_pages, const int* block_table,
                    const int* seq_lens, float* O_part, float* LSE_part, int* counters, void* O,
                    float* LSE, int B, int H, int H_kv, int page_size, int max_pages, int num_pages,
                    int d, int num_splits, float scale, void* stream);

/*
 * fa_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernel
 * and results as fa_decode with the same num_splits, but O_part, LSE_part and the
 * group counters live in a file-scope device array of the library, 16 MiB per
 * device, held from the first call on a device until the process ends.  The
 * entry point calls no hipMalloc, hipFree or other allocating routine.
 *   Q [B][H][d], K, V [B][H_kv][N_k][d] bf16, read
 *   O [B][H][d] bf16 and LSE [B][H] fp32 (LSE may be NULL), written
 * Capacity: 4 * B * H_kv * ceil((H / H_kv) / 16) <= 64 KiB of counters, and
 * 4 * B * H * num_splits * (d + 1) bytes of partials (each part rounded up to 256
 * bytes) within the remaining 16 MiB - 64 KiB; otherwise FA_ERR_CAPACITY and no
 * work is enqueued.  Other validation as for fa_decode.
 * The first call on a device looks up that device's copy of the array and clears
 * its counters on `stream` (one small extra kernel); every completed call leaves
 * them zero.  All calls on one device share its array: calls that overlap on a
 * device (other streams, other threads) race.
 */
int fa_decode_static(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                     int H_kv, int N_k, int d, int num_splits, float scale, void* stream);

/*
 * Group counters of fa_decode / fa_decode_paged (shape as for fa_decode_counter_bytes):
 * fa_decode_counters_reset enqueues a kernel on `stream` that sets them to zero;
 * fa_decode_counters_check enqueues one that writes the number of non-zero counters
 * to *nonzero (a device int, 4-byte aligned; read it after the stream has reached
 * that point).  Neither synchronises or allocates.  Statuses: FA_ERR_NULL,
 * FA_ERR_SHAPE (a size <= 0 or H % H_kv != 0), FA_ERR_ALIGN, FA_ERR_HIP.
 */
int fa_decode_counters_reset(int* counters, int B, int H, int H_kv, void* stream);
int fa_decode_counters_check(const int* counters, int B, int H, int H_kv, int* nonzero, void* stream);

/* Bytes of the counter array fa_decode needs: 4 * B * H_kv * ceil((H / H_kv) / 16)
   (0 if a size is <= 0 or H is not a multiple of H_kv). */
size_t fa_decode_counter_bytes(int B, int H, int H_kv);

/*
 * Default split count for fa_decode_split (Lecture 11 section 6.4: enough
 * workgroups to fill the compute units, segments not so short that fixed
 * costs dominate).  Host-only; queries the current device's compute-unit count
 * once (256 is assumed when no device is visible).  Returns a value in
 * [1, N_k], or 0 if an argument is <= 0.
 */
int fa_decode_num_splits(int B, int H_kv, int N_k, int d);

/* Bytes of O_part plus LSE_part for the given shape (host-only, no HIP call);
 * 0 if an argument is <= 0. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/* Query-tile rows (B_r) and key-tile columns (B_c) that fa_fwd uses for head
 * dimension d; returns FA_OK, or FA_ERR_UNSUPPORTED.  Host-only. */
int fa_fwd_tile_shape(int d, int* block_rows, int* block_cols);

/* Number of (query tile, key tile) pairs fa_fwd computes for one (b, h) -- the
 * causal schedule skips tiles that are entirely masked (Lecture 11 section 5.3).
 * Host-only; -1 on a bad argument. */
long long fa_fwd_tile_count(int N_q, int N_k, int d, int causal);

/* Static description of a status code.  Never NULL. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
