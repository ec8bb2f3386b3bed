// Host half of libexq: status strings, argument checks, the offline packer and
// the split planner.  Nothing here touches HIP, so it also links into CPU-only
// test binaries.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>

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
    // Byte-balanced cuts of the sorted list: a group costs b_g words per
    // column plus a fixed share for its scale, activations and epilogue.
    std::vector<double> cum(G + 1, 0.0);
    for (int i = 0; i < G; ++i) cum[i + 1] = cum[i] + widths[idx[i]] + 1.0;
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

}  // extern "C"
