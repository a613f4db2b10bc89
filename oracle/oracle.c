/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU kernels, and nothing in the GPU product
 * path calls it.
 *
 * What it computes (sources: "Lecture 11 - Kernel Optimization Techniques:
 * FlashAttention, flash-decoding and megakernel", and the FlashAttention v1
 * card of the "CUDA Kernel interview course" page):
 *
 *   oracle_attention   standard three-step attention (Lecture 11 section 2,
 *                      "Algorithm 0"): all scores of a row, then the safe
 *                      softmax of the row (max subtracted, section 3.4),
 *                      then the P-weighted sum of V rows; plus the row's
 *                      log-sum-exp L = m + ln(l) (section 5.1).  A key range
 *                      [k_lo, k_hi) restricts the row to a segment, which is
 *                      the per-segment output o_s and lse_s of
 *                      flash-decoding (section 6.2, step 2).
 *   oracle_online_row  the one-pass online softmax times V (section 3.1 and
 *                      the v1 card's pseudocode): per block, new max,
 *                      rescale factor alpha = exp(m_old - m_new), rescaled
 *                      l and accumulator, normalisation once at the end.
 *   oracle_merge       merge of two partial states (m, l, o) (section 3.2).
 *   oracle_lse_combine flash-decoding's combine in log-sum-exp form
 *                      (section 6.2, step 3).
 *   oracle_attention_bwd the backward pass (section 5.1): gradients of
 *                      sum(dO * O) with respect to Q, K, V from the full
 *                      probability matrix P (the "standard" backward that the
 *                      section compares FlashAttention's against).
 *   oracle_fp8_quantize the FP8 path's input quantisation (block scales after a
 *                      random-sign Hadamard transform; the FlashAttention v3
 *                      card of the course page), with its e4m3 encoder and
 *                      the fast Walsh-Hadamard transform; fp32, see its notes.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - layout: Q [B][H][N_q][d], K and V [B][H_kv][N_k][d], row-major;
 *   - query head h reads key/value head g = h / (H / H_kv);
 *   - causal masking is bottom-right aligned: query i sees key j iff
 *     j <= i + N_k - N_q, so N_q = N_k is the lower triangle;
 *   - scores are scale * (q . k); LSE is the natural log over scaled scores;
 *   - a row with no visible key gets O = 0 and LSE = -inf.
 *
 * Arithmetic: every input element is widened exactly to double; dot products
 * and sums run sequentially in ascending index order; exp and log are libm's.
 * Rows are independent, so threads split the list of rows; that changes no
 * arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };

static double widen(const void* base, int dtype, int64_t i) {
    if (dtype == ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    return ((const double*)base)[i];
}

typedef struct {
    const void *Q, *K, *V;
    int dtype;
    int64_t B, H, H_kv, N_q, N_k, d;
    int causal;
    double scale;
    int64_t k_lo, k_hi;
    const int64_t* rows;
    int64_t n_rows;
    double *O, *LSE, *P;
    int64_t next; /* shared work counter */
} attn_job;

/* One query row of Algorithm 0.  `s` is scratch of length N_k. */
static void attention_row(const attn_job* a, int64_t out_idx, double* s) {
    const int64_t r = a->rows ? a->rows[out_idx] : out_idx;
    const int64_t d = a->d;
    const int64_t i = r % a->N_q;
    const int64_t h = (r / a->N_q) % a->H;
    const int64_t b = r / (a->N_q * a->H);
    const int64_t g = h / (a->H / a->H_kv);
    const int64_t q_off = r * d;
    const int64_t kv_head = (b * a->H_kv + g) * a->N_k;

    /* visible keys: the key range, cut by the bottom-right causal bound */
    int64_t j_end = a->k_hi;
    if (a->causal) {
        int64_t last = i + a->N_k - a->N_q; /* last visible key */
        if (last + 1 < j_end) j_end = last + 1;
    }
    const int64_t j_beg = a->k_lo;

    double* o = a->O + out_idx * d;
    double* p_row = a->P ? a->P + out_idx * a->N_k : 0;
    if (p_row)
        for (int64_t j = 0; j < a->N_k; ++j) p_row[j] = 0.0;

    if (j_end <= j_beg) {
        for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
        a->LSE[out_idx] = -INFINITY;
        return;
    }

    /* step 1: S = scale * Q K^T for this row */
    for (int64_t j = j_beg; j < j_end; ++j) {
        double acc = 0.0;
        const int64_t k_off = (kv_head + j) * d;
        for (int64_t k = 0; k < d; ++k) acc += widen(a->Q, a->dtype, q_off + k) * widen(a->K, a->dtype, k_off + k);
        s[j] = a->scale * acc;
    }

    /* step 2: P = softmax(S), with the row maximum subtracted */
    double m = s[j_beg];
    for (int64_t j = j_beg + 1; j < j_end; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = j_beg; j < j_end; ++j) {
        s[j] = exp(s[j] - m); /* s now holds the unnormalised weights */
        l += s[j];
    }
    for (int64_t j = j_beg; j < j_end; ++j) s[j] = s[j] / l; /* s now holds P */
    if (p_row)
        for (int64_t j = j_beg; j < j_end; ++j) p_row[j] = s[j];

    /* step 3: O = P V */
    for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
    for (int64_t j = j_beg; j < j_end; ++j) {
        const int64_t v_off = (kv_head + j) * d;
        for (int64_t k = 0; k < d; ++k) o[k] += s[j] * widen(a->V, a->dtype, v_off + k);
    }

    /* the row's log-sum-exp over the scaled scores */
    a->LSE[out_idx] = m + log(l);
}

static void* attention_worker(void* p) {
    attn_job* a = (attn_job*)p;
    double* s = (double*)malloc(sizeof(double) * (size_t)(a->N_k > 0 ? a->N_k : 1));
    if (!s) return (void*)1;
    for (;;) {
        int64_t base = __sync_fetch_and_add(&a->next, 16);
        if (base >= a->n_rows) break;
        int64_t end = base + 16 < a->n_rows ? base + 16 : a->n_rows;
        for (int64_t t = base; t < end; ++t) attention_row(a, t, s);
    }
    free(s);
    return 0;
}

/*
 * Exact attention for a list of query rows.
 *   Q [B][H][N_q][d], K and V [B][H_kv][N_k][d]; element type `dtype`
 *   (0 = bf16 bit patterns, 1 = float32, 2 = float64).
 *   Keys are restricted to [k_lo, k_hi) (pass 0, N_k for the full row).
 *   rows: flat row ids r = (b*H + h)*N_q + i, or NULL for all B*H*N_q rows in order.
 *   O [n_rows][d] and LSE [n_rows] receive the results; P, if not NULL,
 *   receives the normalised probabilities [n_rows][N_k] (0 where invisible).
 * Returns 0, or -1 on a bad argument, -2 if memory ran out.
 */
int oracle_attention(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                     int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, int causal, double scale,
                     int64_t k_lo, int64_t k_hi, const int64_t* rows, int64_t n_rows, double* O,
                     double* LSE, double* P, int nthreads) {
    if (!Q || !K || !V || !O || !LSE) return -1;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0 || H % H_kv) return -1;
    if (dtype < 0 || dtype > 2 || k_lo < 0 || k_hi > N_k || k_lo > k_hi) return -1;
    if (!rows) n_rows = B * H * N_q;
    if (n_rows <= 0) return 0;
    if (rows)
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= B * H * N_q) return -1;
    attn_job job = {Q, K, V, dtype, B, H, H_kv, N_q, N_k, d, causal != 0, scale, k_lo, k_hi,
                    rows, n_rows, O, LSE, P, 0};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    pthread_t th[512];
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], 0, attention_worker, &job) != 0) break;
        started = t;
    }
    void* rc0 = attention_worker(&job);
    int bad = rc0 != 0;
    for (int t = 1; t <= started; ++t) {
        void* rc;
        pthread_join(th[t], &rc);
        bad |= rc != 0;
    }
    return bad ? -2 : 0;
}

/*
 * One-pass online softmax times V over one row of precomputed scores
 * (Lecture 11 section 3.1; the v1 card's update of m, alpha, P, acc, l).
 *   s[n] scores, Vr[n][d] value rows, keys processed in blocks of `block`.
 *   Outputs: o[d] = acc / l (normalised once at the end), *m_out, *l_out;
 *   m_trace / l_trace / alpha_trace (each [ceil(n/block)], may be NULL)
 *   record m, l and alpha after each block.
 * A state that has seen no key is m = -inf, l = 0, acc = 0.
 */
void oracle_online_row(const double* s, const double* Vr, int64_t n, int64_t d, int64_t block,
                       double* o, double* m_out, double* l_out, double* m_trace, double* l_trace,
                       double* alpha_trace) {
    double m = -INFINITY, l = 0.0;
    double* acc = (double*)calloc((size_t)(d > 0 ? d : 1), sizeof(double));
    if (block < 1) block = 1;
    int64_t nb = 0;
    for (int64_t j0 = 0; j0 < n; j0 += block, ++nb) {
        int64_t j1 = j0 + block < n ? j0 + block : n;
        double m_blk = -INFINITY;
        for (int64_t j = j0; j < j1; ++j)
            if (s[j] > m_blk) m_blk = s[j];
        double m_new = m > m_blk ? m : m_blk;
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
        if (m_new == -INFINITY) alpha = 1.0; /* nothing seen yet */
        l *= alpha;
        for (int64_t k = 0; k < d; ++k) acc[k] *= alpha;
        if (m_new != -INFINITY) {
            for (int64_t j = j0; j < j1; ++j) {
                double p = exp(s[j] - m_new);
                l += p;
                for (int64_t k = 0; k < d; ++k) acc[k] += p * Vr[j * d + k];
            }
        }
        m = m_new;
        if (m_trace) m_trace[nb] = m;
        if (l_trace) l_trace[nb] = l;
        if (alpha_trace) alpha_trace[nb] = alpha;
    }
    for (int64_t k = 0; k < d; ++k) o[k] = l > 0.0 ? acc[k] / l : 0.0;
    *m_out = m;
    *l_out = l;
    free(acc);
}

/*
 * Merge of two partial states of one row (Lecture 11 section 3.2):
 *   m = max(m_a, m_b), l = l_a e^(m_a - m) + l_b e^(m_b - m),
 *   o = (l_a e^(m_a - m) o_a + l_b e^(m_b - m) o_b) / l.
 * o_a, o_b are normalised outputs; an empty state has m = -inf, l = 0.
 * The output may alias either input.
 */
void oracle_merge(double m_a, double l_a, const double* o_a, double m_b, double l_b,
                  const double* o_b, int64_t d, double* m_out, double* l_out, double* o_out) {
    double m = m_a > m_b ? m_a : m_b;
    if (m == -INFINITY) {
        for (int64_t k = 0; k < d; ++k) o_out[k] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double wa = (m_a == -INFINITY) ? 0.0 : l_a * exp(m_a - m);
    double wb = (m_b == -INFINITY) ? 0.0 : l_b * exp(m_b - m);
    double l = wa + wb;
    for (int64_t k = 0; k < d; ++k) o_out[k] = (wa * o_a[k] + wb * o_b[k]) / l;
    *m_out = m;
    *l_out = l;
}

/*
 * Flash-decoding combine in log-sum-exp form (Lecture 11 section 6.2, step 3):
 *   lse = log sum_s e^(lse_s),  o = sum_s e^(lse_s - lse) o_s,
 * evaluated with the largest lse_s subtracted first.  lse_s [S], o_s [S][d].
 * All segments empty (every lse_s = -inf) gives lse = -inf and o = 0.
 */
void oracle_lse_combine(const double* lse_s, const double* o_s, int64_t S, int64_t d,
                        double* lse_out, double* o_out) {
    double M = -INFINITY;
    for (int64_t t = 0; t < S; ++t)
        if (lse_s[t] > M) M = lse_s[t];
    for (int64_t k = 0; k < d; ++k) o_out[k] = 0.0;
    if (M == -INFINITY) {
        *lse_out = -INFINITY;
        return;
    }
    double sum = 0.0;
    for (int64_t t = 0; t < S; ++t) sum += (lse_s[t] == -INFINITY) ? 0.0 : exp(lse_s[t] - M);
    double lse = M + log(sum);
    for (int64_t t = 0; t < S; ++t) {
        if (lse_s[t] == -INFINITY) continue;
        double w = exp(lse_s[t] - lse);
        for (int64_t k = 0; k < d; ++k) o_out[k] += w * o_s[t * d + k];
    }
    *lse_out = lse;
}

/*
 * Backward pass of exact attention (Lecture 11 section 5.1), the standard form that
 * works from the full rows of P.  With S = scale * Q K^T, P = softmax(S) over the
 * visible keys and O = P V, the gradients of the scalar sum(dO * O) are
 *   dV = P^T dO,   dP = dO V^T,   D_i = sum_j dP_ij P_ij,   dS = P * (dP - D),
 *   dQ = scale * dS K,   dK = scale * dS^T Q
 * (the softmax Jacobian applied to dP gives dS; the section's D_i).  Gradients of a
 * key/value head collect every query head of its group.  Same layouts, masking and
 * element types as oracle_attention; outputs are fp64: dQ [B][H][N_q][d],
 * dK and dV [B][H_kv][N_k][d], and D [B][H][N_q] if D is not NULL.
 * Returns 0, or -1 on a bad argument, -2 if memory ran out.
 */
typedef struct {
    const void *Q, *K, *V, *dO;
    int dtype;
    int64_t B, H, H_kv, N_q, N_k, d;
    int causal;
    double scale;
    double *dQ, *dK, *dV, *D;
    int64_t next; /* shared counter over (b, key/value head) jobs */
} bwd_job;

static void bwd_group(const bwd_job* a, int64_t bg, double* p, double* dp) {
    const int64_t d = a->d, N_q = a->N_q, N_k = a->N_k;
    const int64_t b = bg / a->H_kv, g = bg % a->H_kv;
    const int64_t group = a->H / a->H_kv;
    const int64_t kv_head = bg * N_k;
    double* dK = a->dK + kv_head * d;
    double* dV = a->dV + kv_head * d;
    for (int64_t t = 0; t < N_k * d; ++t) dK[t] = dV[t] = 0.0;
    for (int64_t h = g * group; h < (g + 1) * group; ++h) {
        for (int64_t i = 0; i < N_q; ++i) {
            const int64_t r = (b * a->H + h) * N_q + i;
            const int64_t q_off = r * d;
            double* dq = a->dQ + q_off;
            for (int64_t k = 0; k < d; ++k) dq[k] = 0.0;
            int64_t j_end = N_k;
            if (a->causal) {
                int64_t last = i + N_k - N_q;
                if (last + 1 < j_end) j_end = last + 1;
            }
            if (j_end <= 0) {
                if (a->D) a->D[r] = 0.0;
                continue;
            }
            /* P row: scores, safe softmax */
            for (int64_t j = 0; j < j_end; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < d; ++k)
                    acc += widen(a->Q, a->dtype, q_off + k) * widen(a->K, a->dtype, (kv_head + j) * d + k);
                p[j] = a->scale * acc;
            }
            double m = p[0];
            for (int64_t j = 1; j < j_end; ++j)
                if (p[j] > m) m = p[j];
            double l = 0.0;
            for (int64_t j = 0; j < j_end; ++j) {
                p[j] = exp(p[j] - m);
                l += p[j];
            }
            for (int64_t j = 0; j < j_end; ++j) p[j] /= l;
            /* dP row = dO_i V^T, and D_i = sum_j dP_ij P_ij */
            double Di = 0.0;
            for (int64_t j = 0; j < j_end; ++j) {
                double acc = 0.0;
                for (int64_t k = 0; k < d; ++k)
                    acc += widen(a->dO, a->dtype, q_off + k) * widen(a->V, a->dtype, (kv_head + j) * d + k);
                dp[j] = acc;
                Di += acc * p[j];
            }
            if (a->D) a->D[r] = Di;
            for (int64_t j = 0; j < j_end; ++j) {
                const double ds = p[j] * (dp[j] - Di);
                for (int64_t k = 0; k < d; ++k) {
                    dq[k] += a->scale * ds * widen(a->K, a->dtype, (kv_head + j) * d + k);
                    dK[j * d + k] += a->scale * ds * widen(a->Q, a->dtype, q_off + k);
                    dV[j * d + k] += p[j] * widen(a->dO, a->dtype, q_off + k);
                }
            }
        }
    }
}

static void* bwd_worker(void* p) {
    bwd_job* a = (bwd_job*)p;
    double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * (a->N_k > 0 ? a->N_k : 1)));
    if (!buf) return (void*)1;
    for (;;) {
        int64_t bg = __sync_fetch_and_add(&a->next, 1);
        if (bg >= a->B * a->H_kv) break;
        bwd_group(a, bg, buf, buf + a->N_k);
    }
    free(buf);
    return 0;
}

int oracle_attention_bwd(const void* Q, const void* K, const void* V, const void* dO, int dtype, int64_t B,
                         int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, int causal, double scale,
                         double* dQ, double* dK, double* dV, double* D, int nthreads) {
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return -1;
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0 || H % H_kv) return -1;
    if (dtype < 0 || dtype > 2) return -1;
    bwd_job job = {Q, K, V, dO, dtype, B, H, H_kv, N_q, N_k, d, causal != 0, scale, dQ, dK, dV, D, 0};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 512) nthreads = 512;
    pthread_t th[512];
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], 0, bwd_worker, &job) != 0) break;
        started = t;
    }
    void* rc0 = bwd_worker(&job);
    int bad = rc0 != 0;
    for (int t = 1; t <= started; ++t) {
        void* rc;
        pthread_join(th[t], &rc);
        bad |= rc != 0;
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------------------
 * FP8 (e4m3) block quantisation with incoherent processing -- the input side of an FP8
 * attention forward (FlashAttention v3 card of the course page, "FP8 path"; Lecture 11
 * section 4.4's list): one scale per block of rows, and before quantising, multiply the
 * rows by a random orthogonal matrix so that an outlier channel is spread over all
 * channels.  The pages fix nothing further; the readings taken here:
 *   - format: OCP e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
 *     finite 448, subnormals down to 2^-9, code 0x7F / 0xFF is NaN), rounding to nearest,
 *     ties to even;
 *   - transform: x -> (s o x) H, with s a vector of d random signs (bit j of the 128-bit
 *     mask (hi:lo) set means -1) and H the unnormalised Sylvester-Hadamard matrix, applied
 *     by the fast transform whose stage len = 1, 2, 4, ..., d/2 replaces every pair
 *     (x_i, x_{i+len}) with i & len == 0 by (x_i + x_{i+len}, x_i - x_{i+len}).  Since
 *     H H^T = d I, scores of transformed rows are d times the original ones;
 *   - per block of `block` consecutive rows of one head: amax = max |x| over the block,
 *     r = 448 / amax, code = e4m3(x * r), stored scale = (amax / 448) * post_scale
 *     (post_scale = 1/d for transformed queries, so that dequantised q . k equals the
 *     original score; 1 otherwise); an all-zero block gets r = 0 and scale 0;
 *   - arithmetic: fp32, in exactly the order written (the code is an integer decided by
 *     floating point, and the kernel decides it in fp32).
 * --------------------------------------------------------------------------------------- */

/* Round a float to OCP e4m3fn, nearest-even; beyond the largest finite value's rounding
 * range (|x| > 464) or NaN gives the NaN code. */
uint8_t oracle_e4m3_encode(float x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x) || a > 464.0) return (uint8_t)(sign | 0x7F);
    if (a < ldexp(1.0, -6)) {                      /* subnormal range: units of 2^-9 */
        double q = nearbyint(ldexp(a, 9));        /* 0..8; 8 is the smallest normal */
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e;
    (void)frexp(a, &e);                            /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                                        /* a = (1 + m) * 2^e */
    double m8 = nearbyint(ldexp(a, 3 - e)) - 8.0;  /* mantissa in eighths, 0..8 */
    if (m8 >= 8.0) {
        m8 = 0.0;
        e += 1;
    }
    if (e + 7 > 15 || (e + 7 == 15 && m8 >= 7.0)) return (uint8_t)(sign | 0x7F);
    return (uint8_t)(sign | (uint8_t)((e + 7) << 3) | (uint8_t)m8);
}

double oracle_e4m3_decode(uint8_t c) {
    const double s = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return s * ldexp((double)m, -9);
    return s * ldexp(8.0 + m, e - 10);
}

/* In-place fast Walsh-Hadamard transform of one row (fp32, the stage order above). */
void oracle_fwht_f32(float* x, int64_t d) {
    for (int64_t len = 1; len < d; len <<= 1)
        for (int64_t i = 0; i < d; ++i)
            if ((i & len) == 0) {
                const float a = x[i], b = x[i + len];
                x[i] = a + b;
                x[i + len] = a - b;
            }
}

/* X: bf16 [n_heads][N][d].  codes: [n_heads][N][d] e4m3; scales: [n_heads][ceil(N/block)].
 * Returns 0, or -1 for invalid sizes (d not a power of two when transform is set). */
int oracle_fp8_quantize(const uint16_t* X, int64_t n_heads, int64_t N, int64_t d, int64_t block, int transform,
                        uint64_t sign_lo, uint64_t sign_hi, float post_scale, uint8_t* codes, float* scales) {
    if (n_heads <= 0 || N <= 0 || d <= 0 || block <= 0 || d > 128) return -1;
    if (transform && (d & (d - 1))) return -1;
    const int64_t n_blocks = (N + block - 1) / block;
    float* buf = (float*)malloc(sizeof(float) * (size_t)(block * d));
    if (!buf) return -1;
    for (int64_t h = 0; h < n_heads; ++h)
        for (int64_t t = 0; t < n_blocks; ++t) {
            const int64_t r0 = t * block, r1 = (r0 + block < N) ? r0 + block : N;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r) {
                float* x = buf + (r - r0) * d;
                for (int64_t j = 0; j < d; ++j) {
                    uint32_t bits = (uint32_t)X[(h * N + r) * d + j] << 16;
                    memcpy(&x[j], &bits, 4);
                    if (transform) {
                        const int neg = j < 64 ? (int)((sign_lo >> j) & 1u) : (int)((sign_hi >> (j - 64)) & 1u);
                        if (neg) x[j] = -x[j];
                    }
                }
                if (transform) oracle_fwht_f32(x, d);
                for (int64_t j = 0; j < d; ++j)
                    if (fabsf(x[j]) > amax) amax = fabsf(x[j]);
            }
            const float rcp = amax > 0.0f ? 448.0f / amax : 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t j = 0; j < d; ++j) {
                    const float y = buf[(r - r0) * d + j] * rcp;
                    codes[(h * N + r) * d + j] = oracle_e4m3_encode(y);
                }
            scales[h * n_blocks + t] = amax > 0.0f ? (amax / 448.0f) * post_scale : 0.0f;
        }
    free(buf);
    return 0;
}

/* Array forms for the Python front end. */
void oracle_e4m3_encode_n(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}
void oracle_e4m3_decode_n(const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_fwht_rows(float* x, int64_t rows, int64_t d) {
    for (int64_t r = 0; r < rows; ++r) oracle_fwht_f32(x + r * d, d);
}
