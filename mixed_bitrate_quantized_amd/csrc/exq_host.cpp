// Host half of libexq: status strings, argument checks, the offline packer and
// the split planner.  Nothing here touches HIP, so it also links into CPU-only
// test binaries.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <vector>

#include "exq_internal.h"

namespace exq {

static thread_local char g_last_error[512] = "";

exq_status fail(exq_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

bool width_supported(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }

exq_status check_layer_shape(int K, int N, int group_size, const uint8_t* widths) {
    if (group_size != kGroup) return fail(EXQ_ERR_UNSUPPORTED, "group_size %d (only 128 is implemented)", group_size);
    if (K <= 0 || N <= 0) return fail(EXQ_ERR_INVALID_ARG, "K=%d N=%d must be positive", K, N);
    if (K % kGroup) return fail(EXQ_ERR_INVALID_ARG, "K=%d is not a multiple of 128", K);
    if (!widths) return fail(EXQ_ERR_INVALID_ARG, "widths is NULL");
    for (int g = 0; g < K / kGroup; ++g)
        if (!width_supported(widths[g]))
            return fail(EXQ_ERR_INVALID_ARG, "width %d of group %d is not in {2,3,4,5,6,8}", (int)widths[g], g);
    return EXQ_OK;
}

// ---------------------------------------------------------------- fp16 bits

static inline uint32_t f32_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static inline float bits_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// fp32 -> fp16, round to nearest even, subnormals kept, overflow to infinity.
static inline uint16_t f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u, ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
    if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);          // >= 65520 rounds to inf
    if (ax < 0x38800000u) {                                             // below 2^-14: subnormal
        float scaled = bits_f32(ax) * 16777216.0f;                      // exact: times 2^24
        return (uint16_t)(sign | (uint32_t)std::nearbyint(scaled));
    }
    uint32_t r = (ax + 0x0FFFu + ((ax >> 13) & 1u)) >> 13;            // round 23 -> 10 mantissa bits
    return (uint16_t)(sign | (r - ((127u - 15u) << 10)));
}

static inline float f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    if (e == 0) {
        float v = (float)m * 5.9604644775390625e-8f;  // m * 2^-24, exact
        return sign ? -v : v;
    }
    if (e == 31) return bits_f32(sign | 0x7F800000u | (m << 13));
    return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

// ------------------------------------------------------------------ layout

// Builds the 4*b dwords of one column's group from its 128 codes, walking the
// decoder's units: plane-0 dword d carries units u = d*per .. d*per+per-1,
// unit u's codes 4u+e at offsets p0*t + {0,16,8,24}[e]; a plane-1 dword serves
// R = p0/p1 plane-0 dwords, the high field of the same code sitting at
// p0*t + 16*(e&1) + p1*delta + 8*(e>>1).
static void pack_column_group(const uint8_t* c, int b, uint32_t* dw) {
    const int p0 = (b <= 3) ? 2 : (b == 8 ? 8 : 4);
    const int p1 = b - p0;
    const int per = 8 / p0;
    const uint32_t lo_mask = (1u << p0) - 1u;
    std::memset(dw, 0, sizeof(uint32_t) * 4 * b);
    static const int off[4] = {0, 16, 8, 24};
    for (int d = 0; d < 4 * p0; ++d)
        for (int t = 0; t < per; ++t)
            for (int e = 0; e < 4; ++e) {
                int k = 4 * (d * per + t) + e;
                dw[d] |= ((uint32_t)c[k] & lo_mask) << (p0 * t + off[e]);
            }
    if (p1 == 0) return;
    const int R = p0 / p1;
    for (int d = 0; d < 4 * p0; ++d) {
        int h = d / R, delta = d % R;
        for (int t = 0; t < per; ++t)
            for (int e = 0; e < 4; ++e) {
                int k = 4 * (d * per + t) + e;
                uint32_t hi = (uint32_t)c[k] >> p0;
                int pos = p0 * t + 16 * (e & 1) + p1 * delta + 8 * (e >> 1);
                dw[4 * p0 + h] |= hi << pos;
            }
    }
}

std::vector<uint32_t> group_meta(int K, const uint8_t* widths) {
    int G = K / kGroup;
    std::vector<uint32_t> meta(G);
    uint32_t P = 0;
    for (int g = 0; g < G; ++g) {
        meta[g] = (P << 4) | widths[g];
        P += widths[g];
    }
    return meta;
}

// ------------------------------------------------------------ wave plan

WavePlan plan_waves(int K, const uint8_t* widths) {
    const int G = K / kGroup;
    WavePlan p;
    std::vector<uint32_t> prefix(G + 1, 0);
    for (int g = 0; g < G; ++g) prefix[g + 1] = prefix[g] + widths[g];
    std::vector<int> idx(G);
    for (int g = 0; g < G; ++g) idx[g] = g;
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return widths[a] < widths[b]; });
    p.order.resize(G);
    for (int i = 0; i < G; ++i) p.order[i] = (uint32_t)idx[i] | (prefix[idx[i]] << 16);
    // Balanced cuts of the sorted list.  Decode is bound by instruction
    // issue, so a group costs the instructions its decode issues per wave
    // (masks, the exact zero-point subtracts, field merges of split widths,
    // MFMAs): about 178, 258, 186, 272, 272 and 192 at widths 2, 3, 4, 5, 6, 8,
    // counted in the 64-column kernel's code.  (Measured on the 70B block: a
    // byte-balanced cut left the waves with the most 2- and 3-bit groups last
    // in every workgroup, and the 16-row kernel ran 3.6 % slower.)
    auto cost = [](int b) {
        return b == 2 ? 178.0 : b == 3 ? 258.0 : b == 4 ? 186.0 : b == 8 ? 192.0 : 272.0;
    };
    std::vector<double> cum(G + 1, 0.0);
    for (int i = 0; i < G; ++i) cum[i + 1] = cum[i] + cost(widths[idx[i]]);
    p.bounds.assign(kWaves + 1, 0);
    p.bounds[kWaves] = (uint16_t)G;
    int i = 0;
    for (int w = 1; w < kWaves; ++w) {
        double target = cum[G] * w / kWaves;
        while (i < G && cum[i + 1] <= target) ++i;
        int cut = i;
        if (i < G && (cum[i + 1] - target) < (target - cum[i])) cut = i + 1;
        cut = std::max<int>(cut, p.bounds[w - 1]);
        p.bounds[w] = (uint16_t)cut;
    }
    p.runs.assign((size_t)kWaves * kNumWidths, 0);
    for (int w = 0; w < kWaves; ++w)
        for (int j = p.bounds[w]; j < p.bounds[w + 1]; ++j)
            for (int wi = 0; wi < kNumWidths; ++wi)
                if (widths[idx[j]] == kWidthOrder[wi]) p.runs[(size_t)w * kNumWidths + wi]++;
    return p;
}

// --------------------------------------------------- quantized group scales

// fp16 scale of 4-bit scale code q at width b under column range reference R:
// t = R (q+1)^2 / 256 is exact in fp32; one fp32 product with the fp32
// reciprocal of 2^(b-1)-1, then fp16 round to nearest even.
static uint16_t qs_scale_bits(float R, int q, int b) {
    const float t = R * (float)((q + 1) * (q + 1)) * 0.00390625f;
    const float inv = 1.0f / (float)((1 << (b - 1)) - 1);
    return f32_to_f16(t * inv);
}

// Codes of one column's group at scale s16 (the exq_pack rule) and their
// squared error sum_i (w_i - w_hat_i)^2, accumulated in double in index order.
static double codes_at_scale(const float* w, int b, uint16_t s16, uint8_t* codes) {
    const int z = 1 << (b - 1), qmax = z - 1;
    const float s = f16_to_f32(s16);
    double e = 0.0;
    for (int i = 0; i < kGroup; ++i) {
        float q = 0.0f;
        if (s != 0.0f) q = std::min(std::max(std::nearbyint(w[i] / s), (float)-qmax), (float)qmax);
        codes[i] = (uint8_t)((int)q + z);
        const double d = (double)w[i] - (double)f16_to_f32(f32_to_f16(q * s));
        e += d * d;
    }
    return e;
}

// ------------------------------------------------------- width allocation

constexpr int kNumOpts = 6;
constexpr int kOptWidth[kNumOpts] = {2, 3, 4, 5, 6, 8};

// Squared error sum_i (w_i - w_hat_i)^2 of one column's group at width b,
// with the packer's quantizer and the exact dequantization rounding.
static double column_group_error(const float* w, int b) {
    const int qmax = (1 << (b - 1)) - 1;
    float amax = 0.0f;
    for (int i = 0; i < kGroup; ++i) amax = std::max(amax, std::fabs(w[i]));
    const float s = f16_to_f32(f32_to_f16(amax / (float)qmax));
    double e = 0.0;
    for (int i = 0; i < kGroup; ++i) {
        float q = 0.0f;
        if (s != 0.0f) q = std::min(std::max(std::nearbyint(w[i] / s), (float)-qmax), (float)qmax);
        const double d = (double)w[i] - (double)f16_to_f32(f32_to_f16(q * s));   // q * s is exact in fp32
        e += d * d;
    }
    return e;
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): a 64-bit counter passed
// through a fixed mixing function; one draw per call.
struct SplitMix64 {
    uint64_t x;
    uint64_t next() {
        uint64_t z = (x += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return (double)(next() >> 11) * 0x1.0p-53; }   // [0, 1)
    uint32_t below(uint32_t n) { return (uint32_t)(((next() >> 32) * (uint64_t)n) >> 32); }
};

}  // namespace exq

using namespace exq;

extern "C" {

const char* exq_status_string(exq_status s) {
    switch (s) {
        case EXQ_OK: return "EXQ_OK";
        case EXQ_ERR_INVALID_ARG: return "EXQ_ERR_INVALID_ARG";
        case EXQ_ERR_UNSUPPORTED: return "EXQ_ERR_UNSUPPORTED";
        case EXQ_ERR_HIP: return "EXQ_ERR_HIP";
        case EXQ_ERR_OOM: return "EXQ_ERR_OOM";
    }
    return "EXQ_ERR_UNKNOWN";
}

const char* exq_last_error(void) { return g_last_error; }

size_t exq_packed_bytes(int K, int N, int group_size, const uint8_t* widths) {
    if (check_layer_shape(K, N, group_size, widths) != EXQ_OK) return 0;
    size_t total = 0;
    for (int g = 0; g < K / kGroup; ++g) total += (size_t)widths[g] * kGroup * (size_t)N / 8;
    return total;
}

exq_status exq_pack_qs(const float* W, int K, int N, int group_size, const uint8_t* widths, void* qweight_out,
                       uint8_t* qscale_out, uint16_t* ref_out) {
    exq_status st = check_layer_shape(K, N, group_size, widths);
    if (st != EXQ_OK) return st;
    if (!W || !qweight_out || !qscale_out || !ref_out) return fail(EXQ_ERR_INVALID_ARG, "NULL buffer");
    if (N % 2) return fail(EXQ_ERR_INVALID_ARG, "N=%d must be even for 4-bit scale codes", N);
    const int G = K / kGroup;
    std::vector<uint64_t> P(G + 1, 0);
    for (int g = 0; g < G; ++g) P[g + 1] = P[g] + widths[g];
    std::vector<uint8_t> qcode((size_t)G * N);
    uint8_t* qw = static_cast<uint8_t*>(qweight_out);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int n = 0; n < N; ++n) {
        const float* row = W + (size_t)n * K;
        float range = 0.0f;
        for (int k = 0; k < K; ++k) {
            const float a = std::fabs(row[k]);
            if (!(a <= 3.4e38f)) bad |= 1;
            range = std::max(range, a);
        }
        const uint16_t r16 = f32_to_f16(range);
        if ((r16 & 0x7C00u) == 0x7C00u) bad |= 2;
        if (bad) continue;
        ref_out[n] = r16;
        const float R = f16_to_f32(r16);
        uint8_t codes[kGroup], alt[kGroup];
        uint32_t dw[32];
        for (int g = 0; g < G; ++g) {
            const int b = widths[g];
            const float* w = row + (size_t)g * kGroup;
            float amax = 0.0f;
            for (int i = 0; i < kGroup; ++i) amax = std::max(amax, std::fabs(w[i]));
            // the smallest code whose scale covers the group's range, then one
            // code lower if that quantizes the group with less squared error
            int q = 0;
            if (R != 0.0f) {
                const float c = std::ceil(16.0f * std::sqrt(amax / R));
                q = (c < 1.0f ? 1 : (c > 16.0f ? 16 : (int)c)) - 1;
            }
            uint16_t s16 = qs_scale_bits(R, q, b);
            const double e = codes_at_scale(w, b, s16, codes);
            if (q >= 1) {
                const uint16_t lower = qs_scale_bits(R, q - 1, b);
                if (codes_at_scale(w, b, lower, alt) < e) {
                    --q;
                    s16 = lower;
                    std::memcpy(codes, alt, kGroup);
                }
            }
            qcode[(size_t)g * N + n] = (uint8_t)q;
            pack_column_group(codes, b, dw);
            uint8_t* base = qw + 16 * ((size_t)N * P[g] + (size_t)n);
            for (int j = 0; j < b; ++j) std::memcpy(base + 16 * (size_t)j * N, dw + 4 * j, 16);
        }
    }
    if (bad & 1) return fail(EXQ_ERR_INVALID_ARG, "W holds a NaN or infinity");
    if (bad & 2) return fail(EXQ_ERR_INVALID_ARG, "a column range overflows fp16 (|w| too large)");
    for (int g = 0; g < G; ++g)
        for (int n = 0; n < N; n += 2)
            qscale_out[(size_t)g * (N / 2) + n / 2] =
                (uint8_t)(qcode[(size_t)g * N + n] | (qcode[(size_t)g * N + n + 1] << 4));
    return EXQ_OK;
}

exq_status exq_pack(const float* W, int K, int N, int group_size, const uint8_t* widths,
                    void* qweight_out, uint16_t* scales_out) {
    exq_status st = check_layer_shape(K, N, group_size, widths);
    if (st != EXQ_OK) return st;
    if (!W || !qweight_out || !scales_out) return fail(EXQ_ERR_INVALID_ARG, "NULL buffer");
    const int G = K / kGroup;
    std::vector<uint64_t> P(G + 1, 0);
    for (int g = 0; g < G; ++g) P[g + 1] = P[g] + widths[g];
    uint8_t* qw = static_cast<uint8_t*>(qweight_out);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int n = 0; n < N; ++n) {
        const float* row = W + (size_t)n * K;
        uint8_t codes[kGroup];
        uint32_t dw[32];
        for (int g = 0; g < G; ++g) {
            const int b = widths[g], z = 1 << (b - 1), qmax = z - 1;
            const float* w = row + (size_t)g * kGroup;
            float amax = 0.0f;
            for (int i = 0; i < kGroup; ++i) {
                float a = std::fabs(w[i]);
                if (!(a <= 3.4e38f)) bad |= 1;  // NaN or infinity
                amax = std::max(amax, a);
            }
            uint16_t s16 = f32_to_f16(amax / (float)qmax);
            if ((s16 & 0x7C00u) == 0x7C00u) bad |= 2;
            scales_out[(size_t)g * N + n] = s16;
            const float s = f16_to_f32(s16);
            for (int i = 0; i < kGroup; ++i) {
                int q = 0;
                if (s != 0.0f) {
                    float r = std::nearbyint(w[i] / s);
                    r = std::min(std::max(r, (float)-qmax), (float)qmax);
                    q = (int)r;
                }
                codes[i] = (uint8_t)(q + z);
            }
            pack_column_group(codes, b, dw);
            uint8_t* base = qw + 16 * ((size_t)N * P[g] + (size_t)n);
            for (int j = 0; j < b; ++j) std::memcpy(base + 16 * (size_t)j * N, dw + 4 * j, 16);
        }
    }
    if (bad & 1) return fail(EXQ_ERR_INVALID_ARG, "W holds a NaN or infinity");
    if (bad & 2) return fail(EXQ_ERR_INVALID_ARG, "a group scale overflows fp16 (|w| too large)");
    return EXQ_OK;
}

double exq_trimmed_mean(const float* samples, int n) {
    if (!samples || n < 1) return -1.0;
    std::vector<float> s(samples, samples + n);
    std::sort(s.begin(), s.end());
    const int lo = (5 * n) / 16, hi = std::max((11 * n + 15) / 16, lo + 1);
    double sum = 0.0;
    for (int i = lo; i < hi; ++i) sum += s[i];
    return sum / (hi - lo);
}

exq_status exq_group_errors(const float* W, int K, int N, int group_size, double* err_out) {
    if (!W || !err_out) return fail(EXQ_ERR_INVALID_ARG, "NULL buffer");
    if (K <= 0 || N <= 0 || K % kGroup) return fail(EXQ_ERR_INVALID_ARG, "bad shape K=%d N=%d", K, N);
    if (group_size != kGroup) return fail(EXQ_ERR_UNSUPPORTED, "group_size=%d (only 128)", group_size);
    const int G = K / kGroup;
    int bad = 0;
    // One group per task, columns in order: the sums do not depend on the thread count.
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int g = 0; g < G; ++g) {
        double acc[kNumOpts] = {0, 0, 0, 0, 0, 0};
        for (int n = 0; n < N; ++n) {
            const float* w = W + (size_t)n * K + (size_t)g * kGroup;
            float amax = 0.0f;
            for (int i = 0; i < kGroup; ++i) {
                const float a = std::fabs(w[i]);
                if (!(a <= 3.4e38f)) bad |= 1;
                amax = std::max(amax, a);
            }
            if (amax / 1.0f > 65504.0f) bad |= 2;   // the 2-bit scale max|w| / 1 must stay finite in fp16
            if (bad) continue;
            for (int j = 0; j < kNumOpts; ++j) acc[j] += column_group_error(w, kOptWidth[j]);
        }
        for (int j = 0; j < kNumOpts; ++j) err_out[(size_t)g * kNumOpts + j] = acc[j];
    }
    if (bad & 1) return fail(EXQ_ERR_INVALID_ARG, "W holds a NaN or infinity");
    if (bad & 2) return fail(EXQ_ERR_INVALID_ARG, "a group scale overflows fp16 (|w| too large)");
    return EXQ_OK;
}

exq_status exq_allocate_widths(const double* err, const int32_t* size, int G, int64_t budget,
                               const uint8_t* min_width, uint64_t seed, int64_t iterations, uint8_t* widths_out,
                               double* total_err_out) {
    if (!err || !size || !widths_out) return fail(EXQ_ERR_INVALID_ARG, "NULL buffer");
    if (G < 1) return fail(EXQ_ERR_INVALID_ARG, "G=%d must be >= 1", G);
    if (iterations < 0) return fail(EXQ_ERR_INVALID_ARG, "iterations must be >= 0");
    // Allowed options of each group: lo[g] .. 5 (widths at or above min_width).
    std::vector<int> lo(G), cur(G);
    int64_t cost = 0;
    for (int g = 0; g < G; ++g) {
        if (size[g] < 1) return fail(EXQ_ERR_INVALID_ARG, "size[%d]=%d must be >= 1", g, size[g]);
        for (int j = 0; j < kNumOpts; ++j)
            if (!(err[(size_t)g * kNumOpts + j] >= 0.0) || !std::isfinite(err[(size_t)g * kNumOpts + j]))
                return fail(EXQ_ERR_INVALID_ARG, "err[%d][%d] is negative or not finite", g, j);
        const int mw = min_width ? min_width[g] : 0;
        if (mw > 8) return fail(EXQ_ERR_INVALID_ARG, "min_width[%d]=%d above 8", g, mw);
        lo[g] = 0;
        while (kOptWidth[lo[g]] < mw) ++lo[g];
        cur[g] = lo[g];
        cost += (int64_t)kOptWidth[lo[g]] * size[g];
    }
    if (cost > budget)
        return fail(EXQ_ERR_INVALID_ARG, "budget %lld is below the smallest allowed cost %lld", (long long)budget,
                    (long long)cost);
    auto E = [&](int g, int j) { return err[(size_t)g * kNumOpts + j]; };
    auto C = [&](int g, int j) { return (int64_t)kOptWidth[j] * size[g]; };

    // Start: the greedy of the multiple-choice knapsack.  Each group's
    // options are reduced to the lower convex hull of (cost, error) above
    // its minimum; hull steps are taken in order of error saved per bit as
    // long as they fit.
    {
        struct Step { double gain; int g, from, to; };
        std::vector<std::vector<int>> hull(G);
        for (int g = 0; g < G; ++g) {
            std::vector<int>& h = hull[g];
            h.push_back(lo[g]);
            for (int j = lo[g] + 1; j < kNumOpts; ++j) {
                if (E(g, j) >= E(g, h.back())) continue;   // dominated: costs more, saves nothing
                while (h.size() >= 2) {
                    const int a = h[h.size() - 2], b = h.back();
                    // b is not on the lower hull if the slope a->j is at least as steep as a->b
                    const double sab = (E(g, a) - E(g, b)) / (double)(C(g, b) - C(g, a));
                    const double saj = (E(g, a) - E(g, j)) / (double)(C(g, j) - C(g, a));
                    if (saj >= sab) h.pop_back();
                    else break;
                }
                h.push_back(j);
            }
        }
        auto cmp = [](const Step& x, const Step& y) { return x.gain < y.gain || (x.gain == y.gain && x.g > y.g); };
        std::vector<Step> heap;
        std::vector<size_t> pos(G, 0);
        auto push_next = [&](int g) {
            if (pos[g] + 1 < hull[g].size()) {
                const int a = hull[g][pos[g]], b = hull[g][pos[g] + 1];
                heap.push_back({(E(g, a) - E(g, b)) / (double)(C(g, b) - C(g, a)), g, a, b});
                std::push_heap(heap.begin(), heap.end(), cmp);
            }
        };
        for (int g = 0; g < G; ++g) push_next(g);
        while (!heap.empty()) {
            std::pop_heap(heap.begin(), heap.end(), cmp);
            const Step s = heap.back();
            heap.pop_back();
            const int64_t dc = C(s.g, s.to) - C(s.g, s.from);
            if (cost + dc > budget) continue;   // this group stops here
            cost += dc;
            cur[s.g] = s.to;
            ++pos[s.g];
            push_next(s.g);
        }
    }

    // Simulated annealing from the greedy start.  A move sets one group to
    // another allowed width.  If that breaks the budget, it is paid for by
    // lowering other groups one allowed step at a time, each time the one
    // that adds the least error per bit freed among four random candidates,
    // until the move fits (at most 64 steps): one wide group can so be paid
    // for by many narrow ones.  The whole move is accepted by the Metropolis
    // rule at a temperature falling geometrically over six decades from a
    // tenth of the mean size of single-step changes at the start; the best
    // state seen, topped up greedily with any budget it leaves, is returned.
    double total = 0.0;
    for (int g = 0; g < G; ++g) total += E(g, cur[g]);
    std::vector<int> best = cur;
    double best_total = total;
    SplitMix64 rng{seed};
    if (iterations > 0) {
        double t0 = 0.0;
        int samples = 0;
        for (int i = 0; i < 256; ++i) {
            const int g = (int)rng.below((uint32_t)G), j = cur[g];
            const int k = (j + 1 < kNumOpts) ? j + 1 : j - 1;
            if (k < lo[g] || k < 0) continue;
            t0 += std::fabs(E(g, k) - E(g, j));
            ++samples;
        }
        t0 = samples ? t0 / samples : 1.0;
        if (!(t0 > 0.0)) t0 = 1.0;
        const double cool = std::pow(1e-6, 1.0 / (double)iterations);
        double T = 0.1 * t0;
        std::vector<std::pair<int, int>> undo;   // (group, previous option) of the groups a move lowered
        for (int64_t it = 0; it < iterations; ++it, T *= cool) {
            const int g = (int)rng.below((uint32_t)G);
            const int span = kNumOpts - lo[g];
            if (span < 2) continue;
            int j = lo[g] + (int)rng.below((uint32_t)(span - 1));
            if (j >= cur[g]) ++j;   // any allowed option but the current one
            const int jg = cur[g];
            int64_t dc = C(g, j) - C(g, jg);
            double de = E(g, j) - E(g, jg);
            cur[g] = j;
            undo.clear();
            bool fits = cost + dc <= budget;
            for (int step = 0; !fits && step < 64; ++step) {
                int h = -1;
                double rate = 0.0;
                for (int t = 0; t < 4; ++t) {
                    const int c = (int)rng.below((uint32_t)G);
                    if (c == g || cur[c] == lo[c]) continue;
                    const double r = (E(c, cur[c] - 1) - E(c, cur[c])) / (double)(C(c, cur[c]) - C(c, cur[c] - 1));
                    if (h < 0 || r < rate) {
                        h = c;
                        rate = r;
                    }
                }
                if (h < 0) continue;
                undo.push_back({h, cur[h]});
                dc += C(h, cur[h] - 1) - C(h, cur[h]);
                de += E(h, cur[h] - 1) - E(h, cur[h]);
                --cur[h];
                fits = cost + dc <= budget;
            }
            if (fits && (de <= 0.0 || rng.uniform() < std::exp(-de / T))) {
                cost += dc;
                total += de;
                if (total < best_total) {
                    best_total = total;
                    best = cur;
                }
            } else {
                for (size_t u = undo.size(); u-- > 0;) cur[undo[u].first] = undo[u].second;
                cur[g] = jg;
            }
        }
    }
    // Polish: spend any budget left over on the single-group upgrades that
    // save the most error per bit.
    {
        cost = 0;
        for (int g = 0; g < G; ++g) cost += C(g, best[g]);
        for (;;) {
            int bg = -1, bj = -1;
            double bgain = 0.0;
            for (int g = 0; g < G; ++g)
                for (int j = best[g] + 1; j < kNumOpts; ++j) {
                    const int64_t dc = C(g, j) - C(g, best[g]);
                    const double gain = (E(g, best[g]) - E(g, j)) / (double)dc;
                    if (cost + dc <= budget && gain > bgain) {
                        bgain = gain;
                        bg = g;
                        bj = j;
                    }
                }
            if (bg < 0) break;
            cost += C(bg, bj) - C(bg, best[bg]);
            best[bg] = bj;
        }
    }
    double sum = 0.0;   // recomputed in group order, free of the running sum's drift
    for (int g = 0; g < G; ++g) {
        widths_out[g] = (uint8_t)kOptWidth[best[g]];
        sum += E(g, best[g]);
    }
    if (total_err_out) *total_err_out = sum;
    return EXQ_OK;
}

}  // extern "C"
