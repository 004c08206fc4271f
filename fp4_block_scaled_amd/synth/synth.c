/*
 * Seeded synthetic inputs for the microscaled-FP4 linear layer.
 *
 * This module only draws random numbers: it holds none of the quantization or GEMM arithmetic,
 * so the CPU oracle and the GPU path can both consume what it produces without sharing any of
 * the method's code.
 *
 * Generator: SplitMix64 used as a counter-based stream (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): the i-th output of the stream keyed by `seed`
 * is mix64(key + (i + 1) * GOLDEN), with key = mix64(seed).  Each output therefore depends only
 * on (seed, i), so any thread count produces the same tensor.
 *
 * Normal deviates: Box-Muller (Box and Muller, 1958) in fp64 from the two stream words 2i and
 * 2i+1, keeping the cosine branch; scaled by sigma and rounded once to fp32 (IEEE RNE).
 *
 * Outlier channels: a seeded Fisher-Yates shuffle (Durstenfeld's variant) of 0..K-1; the first
 * `count` entries are the chosen channels.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_word(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* out[i] = fp32(sigma * N_i), N_i standard normal, for i in [0, n). */
void mxs_normal_f32(uint64_t seed, int64_t n, double sigma, float* out) {
    const uint64_t key = mix64(seed);
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t z1 = stream_word(key, 2 * (uint64_t)i);
        uint64_t z2 = stream_word(key, 2 * (uint64_t)i + 1);
        double u1 = (double)((z1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
        double u2 = (double)(z2 >> 11) * 0x1.0p-53;       /* [0, 1) */
        double g = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)(sigma * g);
    }
}

/* Uniform 64-bit words, exposed for tests of the generator itself. */
void mxs_words(uint64_t seed, int64_t n, uint64_t* out) {
    const uint64_t key = mix64(seed);
    for (int64_t i = 0; i < n; ++i) out[i] = stream_word(key, (uint64_t)i);
}

/* First `count` entries of a seeded Fisher-Yates permutation of 0..K-1. */
void mxs_outlier_channels(uint64_t seed, int64_t K, int64_t count, int64_t* perm_scratch,
                          int64_t* out_idx) {
    const uint64_t key = mix64(seed);
    for (int64_t i = 0; i < K; ++i) perm_scratch[i] = i;
    for (int64_t i = K - 1; i > 0; --i) {
        /* unbiased enough for K << 2^64: modulo bias is below 2^-40 */
        int64_t j = (int64_t)(stream_word(key, (uint64_t)(K - 1 - i)) % (uint64_t)(i + 1));
        int64_t t = perm_scratch[i];
        perm_scratch[i] = perm_scratch[j];
        perm_scratch[j] = t;
    }
    /* the channels drawn are the last `count` positions filled, i.e. the tail */
    for (int64_t c = 0; c < count; ++c) out_idx[c] = perm_scratch[K - 1 - c];
}

/* x[r, idx[c]] *= factor in fp32 for every row r (row-major, leading dimension cols). */
void mxs_scale_columns_f32(float* x, int64_t rows, int64_t cols, const int64_t* idx, int64_t count,
                           float factor) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float* row = x + r * cols;
        for (int64_t c = 0; c < count; ++c) row[idx[c]] *= factor;
    }
}
