/*
 * Seeded synthetic inputs shared by the test oracle and the GPU path.
 *
 * This file holds only input generation: a counter-based uniform generator,
 * a tabulated standard-normal sampler built on it, and per-group squared
 * norms used to pick which groups a width schedule forces to high precision.
 * None of the quantized-matmul arithmetic lives here.
 *
 * Uniform source: Philox4x32-10 as published by Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): a 128-bit
 * counter and a 64-bit key, ten rounds of two 32x32->64 multiplies with the
 * round constants and Weyl key increments given in that paper.
 *
 * Element e of a stream keyed by `seed` is word (e & 3) of
 * Philox(counter = {lo32(e >> 2), hi32(e >> 2), 0, 0}, key = seed).
 *
 * Normal sampler: inverse-CDF sampling.  The top 16 bits of a uniform word
 * pick one of 65536 equal-probability cells, the low 16 bits interpolate
 * linearly between the standard-normal quantiles at the cell's edges.  The
 * outermost cell edges are placed at the quantile of 2^-19 (about +-4.62),
 * so samples are truncated there; everywhere else the sampled CDF is the
 * piecewise-linear interpolation of the normal CDF on a 2^-16 grid.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_CELLS 65536

static float g_quantile[SYNTH_CELLS + 1];
static int g_table_ready = 0;

static inline uint32_t mulhilo32(uint32_t a, uint32_t b, uint32_t* hi) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    return (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, hi1;
        uint32_t lo0 = mulhilo32(M0, c0, &hi0);
        uint32_t lo1 = mulhilo32(M1, c2, &hi1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Standard normal CDF through the complementary error function. */
static double norm_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

/* Quantile by safeguarded Newton iteration on the CDF (bracket [-40, 40]). */
static double norm_quantile(double p) {
    double lo = -40.0, hi = 40.0, z = 0.0;
    for (int it = 0; it < 200; ++it) {
        double f = norm_cdf(z) - p;
        if (f == 0.0) return z;
        if (f < 0.0) lo = z; else hi = z;
        double dens = exp(-0.5 * z * z) / sqrt(2.0 * M_PI);
        double zn = (dens > 0.0) ? z - f / dens : 0.5 * (lo + hi);
        if (!(zn > lo && zn < hi)) zn = 0.5 * (lo + hi);
        if (fabs(zn - z) <= 1e-15 * (1.0 + fabs(z))) return zn;
        z = zn;
        if (hi - lo < 1e-15) break;
    }
    return z;
}

void synth_init(void) {
    if (g_table_ready) return;
    /* Symmetric by construction: compute the lower half, mirror it. */
    g_quantile[0] = (float)norm_quantile(1.0 / 524288.0); /* 2^-19 */
    for (int j = 1; j < SYNTH_CELLS / 2; ++j)
        g_quantile[j] = (float)norm_quantile((double)j / SYNTH_CELLS);
    g_quantile[SYNTH_CELLS / 2] = 0.0f;
    for (int j = 0; j < SYNTH_CELLS / 2; ++j)
        g_quantile[SYNTH_CELLS - j] = -g_quantile[j];
    g_table_ready = 1;
}

const float* synth_quantile_table(void) { synth_init(); return g_quantile; }

static inline float normal_from_word(uint32_t r) {
    uint32_t cell = r >> 16;
    float frac = (float)(r & 0xFFFFu) * (1.0f / 65536.0f);
    float a = g_quantile[cell], b = g_quantile[cell + 1];
    return a + frac * (b - a);
}

/* out[i] = sigma * z(seed, first + i) for i in [0, count). */
void synth_fill_normal(uint64_t seed, uint64_t first, uint64_t count, float sigma, float* out) {
    synth_init();
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint64_t blk_begin = first >> 2, blk_end = (first + count + 3) >> 2;
#pragma omp parallel for schedule(static)
    for (int64_t blk = (int64_t)blk_begin; blk < (int64_t)blk_end; ++blk) {
        uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)((uint64_t)blk >> 32), 0u, 0u};
        uint32_t w[4];
        synth_philox4x32_10(ctr, key, w);
        for (int j = 0; j < 4; ++j) {
            uint64_t e = ((uint64_t)blk << 2) + (uint64_t)j;
            if (e < first || e >= first + count) continue;
            out[e - first] = sigma * normal_from_word(w[j]);
        }
    }
}

/* Raw uniform words, same stream definition (used by schedule permutations). */
void synth_fill_u32(uint64_t seed, uint64_t first, uint64_t count, uint32_t* out) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (uint64_t e = first; e < first + count; ++e) {
        uint64_t blk = e >> 2;
        uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
        uint32_t w[4];
        synth_philox4x32_10(ctr, key, w);
        out[e - first] = w[e & 3];
    }
}

/* Rows of a [N][K] row-major matrix, element (n, k) = stream index n*K + k. */
void synth_fill_rows(uint64_t seed, int64_t K, const int64_t* rows, int64_t nrows, float sigma, float* out) {
    for (int64_t r = 0; r < nrows; ++r)
        synth_fill_normal(seed, (uint64_t)(rows[r] * K), (uint64_t)K, sigma, out + r * K);
}

/* Sum of squares of W[:, g*group : (g+1)*group] for each group g, in double.
 * Each group is summed by one thread in a fixed order (n ascending, then i),
 * so the result does not depend on the thread count. */
void synth_group_sq_norms(const float* W, int64_t N, int64_t K, int64_t group, double* out) {
    const int64_t G = K / group;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < G; ++g) {
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const float* p = W + n * K + g * group;
            for (int64_t i = 0; i < group; ++i) {
                double v = p[i];
                s += v * v;
            }
        }
        out[g] = s;
    }
}
