/*
 * Seeded synthetic inputs for the fused rank-sum + residual add + RMSNorm
 * operator.  This file only draws numbers: it holds no step of the operator's
 * arithmetic, and both the CPU oracle and the GPU library receive the very
 * same bytes it produces.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as in S. Vigna's
 * public-domain splitmix64.c).  It is counter based: output i of a stream is
 * mix64(key + (i + 1) * GAMMA), so every element can be drawn on its own and
 * the bytes do not depend on how many threads fill the buffer.
 *
 * Normal samples use the Box-Muller transform in binary64 on the pair of
 * uniforms (2j, 2j+1): element 2j takes the cosine branch, 2j+1 the sine
 * branch.  Samples are scaled in binary64 and rounded once to binary32; the
 * caller rounds binary32 to bfloat16.
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* Uniform on (0, 1]: the top 53 bits plus one, times 2^-53 (never 0, so log is finite). */
static inline double unit(uint64_t z) { return ((double)(z >> 11) + 1.0) * 0x1p-53; }

/* Key of the stream for (seed, tag): every tensor and every rank has its own tag. */
uint64_t synth_stream_key(uint64_t seed, uint64_t tag) {
    return mix64(mix64(seed + GAMMA) ^ ((tag + 1) * GAMMA));
}

/*
 * out[i] = float(sigma * N_i), N_i standard normal from stream (seed, tag).
 * If outlier_p > 0, element i is also multiplied by outlier_scale (in binary64,
 * before the rounding to binary32) when the i-th uniform of stream
 * (seed, outlier_tag) is below outlier_p: an independent Bernoulli(outlier_p)
 * draw per element.
 */
void synth_normal(uint64_t seed, uint64_t tag, double sigma, int64_t n, float* out,
                  uint64_t outlier_tag, double outlier_p, double outlier_scale) {
    const uint64_t key = synth_stream_key(seed, tag);
    const uint64_t okey = synth_stream_key(seed, outlier_tag);
    const double two_pi = 6.283185307179586476925286766559;
    const int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < pairs; ++j) {
        const double u1 = unit(draw(key, (uint64_t)(2 * j)));
        const double u2 = unit(draw(key, (uint64_t)(2 * j + 1)));
        const double r = sqrt(-2.0 * log(u1));
        const double a = two_pi * u2;
        double v[2] = {sigma * r * cos(a), sigma * r * sin(a)};
        for (int k = 0; k < 2; ++k) {
            const int64_t i = 2 * j + k;
            if (i >= n) break;
            double s = v[k];
            if (outlier_p > 0.0 && unit(draw(okey, (uint64_t)i)) <= outlier_p) s *= outlier_scale;
            out[i] = (float)s;
        }
    }
}

/* out[i] = float(lo + (hi - lo) * U_i), U_i uniform on (0, 1] from stream (seed, tag). */
void synth_uniform(uint64_t seed, uint64_t tag, double lo, double hi, int64_t n, float* out) {
    const uint64_t key = synth_stream_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unit(draw(key, (uint64_t)i)));
}
