/*
 * gen.c -- seeded, index-addressable synthetic inputs.
 *
 * This module is shared by both sides of every parity test (the fp64 oracle
 * and the GPU path).  It holds no attention arithmetic: only a counter-based
 * random stream, the Box-Muller transform and float -> bf16 rounding.
 *
 * Stream definition (counter-based SplitMix64, Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014):
 *   gamma      = 0x9E3779B97F4A7C15
 *   mix(z)     = the SplitMix64 output finaliser (two xor-shift-multiply
 *                rounds with 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB)
 *   s0(seed,t) = mix(seed) XOR (t * 0xD1B54A32D192ED03)     t = tensor id
 *   word k     = mix(s0 + (k + 1) * gamma)                  (mod 2^64)
 * Element i uses words 2*(i/2) and 2*(i/2)+1 as two uniforms
 *   u1 = ((w0 >> 11) + 0.5) * 2^-53   in (0, 1)   (never 0, so log is safe)
 *   u2 =  (w1 >> 11)        * 2^-53   in [0, 1)
 * and the Box-Muller pair (Box & Muller 1958), evaluated in double:
 *   r = sqrt(-2 ln u1), even i -> r cos(2 pi u2), odd i -> r sin(2 pi u2).
 * The double is rounded to float, multiplied by `scale` in float, and (for
 * the bf16 entry point) rounded to bf16 with round-to-nearest-even.
 *
 * All entry points are plain C; `nthreads` <= 1 runs on the calling thread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint32_t tensor_id) {
    return mix64(seed) ^ ((uint64_t)tensor_id * 0xD1B54A32D192ED03ULL);
}

static inline uint64_t stream_word(uint64_t base, uint64_t k) {
    return mix64(base + (k + 1) * GEN_GAMMA);
}

/* Round-to-nearest-even float -> bf16 bit pattern.  NaN stays NaN (quiet). */
uint16_t gen_bf16_rne(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    if ((x & 0x7F800000u) == 0x7F800000u && (x & 0x007FFFFFu)) return (uint16_t)((x >> 16) | 0x0040u);
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

float gen_bf16_to_f32(uint16_t h) {
    uint32_t x = (uint32_t)h << 16;
    float f;
    memcpy(&f, &x, 4);
    return f;
}

static inline float normal_at(uint64_t base, int64_t i, float scale) {
    uint64_t pair = (uint64_t)i >> 1;
    uint64_t w0 = stream_word(base, 2 * pair);
    uint64_t w1 = stream_word(base, 2 * pair + 1);
    double u1 = ((double)(w0 >> 11) + 0.5) * 0x1.0p-53;
    double u2 = (double)(w1 >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    double z = (i & 1) ? r * sin(t) : r * cos(t);
    return (float)z * scale;
}

typedef struct {
    uint64_t base;
    int64_t offset, lo, hi;
    float scale;
    float* out_f32;
    uint16_t* out_bf16;
} gen_job;

static void* gen_worker(void* p) {
    gen_job* j = (gen_job*)p;
    for (int64_t i = j->lo; i < j->hi; ++i) {
        float f = normal_at(j->base, j->offset + i, j->scale);
        if (j->out_f32) j->out_f32[i] = f;
        else j->out_bf16[i] = gen_bf16_rne(f);
    }
    return 0;
}

static void gen_run(uint64_t seed, uint32_t tensor_id, int64_t offset, int64_t n, float scale,
                    float* out_f32, uint16_t* out_bf16, int nthreads) {
    if (n <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n / 65536 + 1) nthreads = (int)(n / 65536 + 1);
    gen_job jobs[256];
    pthread_t th[256];
    uint64_t base = stream_base(seed, tensor_id);
    int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        int64_t lo = (int64_t)t * chunk, hi = lo + chunk < n ? lo + chunk : n;
        jobs[t] = (gen_job){base, offset, lo, hi < lo ? lo : hi, scale, out_f32, out_bf16};
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], 0, gen_worker, &jobs[t]) == 0) started = t; else { gen_worker(&jobs[t]); }
    gen_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
}

/* Elements [offset, offset+n) of stream (seed, tensor_id) as float, times scale. */
void gen_normal_f32(uint64_t seed, uint32_t tensor_id, int64_t offset, int64_t n, float scale,
                    float* out, int nthreads) {
    gen_run(seed, tensor_id, offset, n, scale, out, 0, nthreads);
}

/* Same values, rounded to bf16 (RNE); `out` receives raw bf16 bit patterns. */
void gen_normal_bf16(uint64_t seed, uint32_t tensor_id, int64_t offset, int64_t n, float scale,
                     uint16_t* out, int nthreads) {
    gen_run(seed, tensor_id, offset, n, scale, 0, out, nthreads);
}

/* Elementwise float -> bf16 (RNE) over a host array. */
void gen_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = gen_bf16_rne(in[i]);
}

/* Raw 64-bit stream words, for the generator's own tests. */
void gen_words(uint64_t seed, uint32_t tensor_id, int64_t k0, int64_t n, uint64_t* out) {
    uint64_t base = stream_base(seed, tensor_id);
    for (int64_t i = 0; i < n; ++i) out[i] = stream_word(base, (uint64_t)(k0 + i));
}
