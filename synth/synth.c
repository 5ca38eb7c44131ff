/*
 * Seeded synthetic input generator (test and benchmark infrastructure).
 *
 * Shared by the CPU oracle and the HIP path as the one source of inputs.
 * It holds none of the decode method's arithmetic: it only draws numbers.
 *
 * Generator: counter-based SplitMix64.  The output mixing function is the
 * published SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as in Vigna's
 * public-domain splitmix64.c).  A stream is named by a key derived from
 * (seed, kind, layer, seq, extra); value n of a stream is
 *     mix64(key + (n + 1) * 0x9E3779B97F4A7C15).
 * Any row can therefore be regenerated on its own, in any order, by any
 * thread, with identical results.
 *
 * Normals: Box-Muller (1958) on two 53-bit uniforms, in double precision,
 *     u1 in (0, 1], u2 in [0, 1);  r = sqrt(-2 ln u1);
 *     z0 = r cos(2 pi u2),  z1 = r sin(2 pi u2).
 * Element 2m of a row uses z0 of pair m, element 2m+1 uses z1.
 *
 * bf16 output: double -> float (C conversion, round to nearest even), then
 * float -> bf16 round to nearest even on the bit pattern (finite values).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint32_t kind, uint32_t layer,
                          uint32_t seq, uint64_t extra) {
    uint64_t k = mix64(seed ^ 0x5DEECE66DULL);
    k = mix64(k + (uint64_t)kind * GOLDEN);
    k = mix64(k + (uint64_t)layer * GOLDEN);
    k = mix64(k + (uint64_t)seq * GOLDEN);
    k = mix64(k + extra * GOLDEN);
    return k;
}

static inline uint64_t draw(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * GOLDEN);
}

static inline void normal_pair(uint64_t key, uint64_t pair, double *z0, double *z1) {
    const double inv53 = 1.0 / 9007199254740992.0; /* 2^-53 */
    uint64_t a = draw(key, 2 * pair), b = draw(key, 2 * pair + 1);
    double u1 = (double)((a >> 11) + 1) * inv53; /* (0, 1] */
    double u2 = (double)(b >> 11) * inv53;       /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Fill rows [row0, row0 + nrows) of width `width` (even) with N(0,1) doubles. */
void synth_normal_f64(uint64_t key, uint64_t row0, uint64_t nrows, uint32_t width,
                      double *out) {
    const uint64_t pairs = width / 2;
    long long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < (long long)nrows; ++r) {
        double *o = out + (uint64_t)r * width;
        uint64_t base = (row0 + (uint64_t)r) * pairs;
        for (uint64_t m = 0; m < pairs; ++m) normal_pair(key, base + m, &o[2 * m], &o[2 * m + 1]);
    }
}

/* Same values as synth_normal_f64, rounded to bf16 (via float), written as raw uint16. */
void synth_normal_bf16(uint64_t key, uint64_t row0, uint64_t nrows, uint32_t width,
                       uint16_t *out) {
    const uint64_t pairs = width / 2;
    long long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < (long long)nrows; ++r) {
        uint16_t *o = out + (uint64_t)r * width;
        uint64_t base = (row0 + (uint64_t)r) * pairs;
        for (uint64_t m = 0; m < pairs; ++m) {
            double z0, z1;
            normal_pair(key, base + m, &z0, &z1);
            o[2 * m] = f32_to_bf16_rne((float)z0);
            o[2 * m + 1] = f32_to_bf16_rne((float)z1);
        }
    }
}

/* Raw 64-bit draws (for tests of the generator itself). */
void synth_raw_u64(uint64_t key, uint64_t n0, uint64_t n, uint64_t *out) {
    for (uint64_t i = 0; i < n; ++i) out[i] = draw(key, n0 + i);
}

/* The bare SplitMix64 sequence from a state, as published (for a known-answer test). */
void synth_splitmix64_sequence(uint64_t state, uint64_t n, uint64_t *out) {
    for (uint64_t i = 0; i < n; ++i) {
        state += GOLDEN;
        out[i] = mix64(state);
    }
}

/* Round doubles to bf16 (via float), for query vectors built on the host. */
void synth_f64_to_bf16(const double *in, uint64_t n, uint16_t *out) {
    for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)in[i]);
}
