/*
 * TEST INFRASTRUCTURE ONLY -- the plain, slow CPU oracle for the mixed-bitrate
 * quantized matmul y = x * W^T.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this; the library never does, and
 * this file shares no code, header or table with it.
 *
 * What is computed (the method):
 *   - EXL2-style storage: each group of 128 consecutive input channels of a
 *     linear layer has its own bit width from {2,3,4,5,6,8}, mixed inside one
 *     layer toward a target average bits-per-weight, with the important
 *     columns at higher precision.  (nightvoyager.top exllamav2 report, "key
 *     design decisions" and "innovations"; promptquorum.com "ExLlamaV2
 *     explained", section "what is EXL2 quantization").
 *   - one fp16 scale per (group, output column), symmetric round-to-nearest
 *     with scale = max|w| / (2^(b-1) - 1) (the GPTQ "4-bit (group 128)"
 *     convention that ainews.cool's exllamav3 benchmark table compares to).
 *   - dequantize on the fly and multiply (the "Q-GEMM" the exllamav2 report
 *     names under "solution philosophy").
 * The pages give no bit layout, rounding rule or scale granularity; those
 * readings are fixed by the EXQ1 layout description below and in the
 * library's public header.
 *
 * EXQ1 layout (K inputs, N outputs, G = K/128 groups, widths b_g, prefix
 * P_g = sum_{h<g} b_h).  Group g of column n owns b_g 16-byte words; word j
 * sits at byte 16*(N*P_g + j*N + n); a column's dwords are numbered
 * m = 4*j + r (r = dword within the word, little endian).  A width is split
 * into planes, low bits first: 2:[2] 3:[2,1] 4:[4] 5:[4,1] 6:[4,2] 8:[8].
 * For code k in [0,128): u = k/4, e = k%4, e1 = e%2, e2 = e/2.
 *   plane 0 (width p0, dwords m in [0, 4*p0)): per = 8/p0, dword u/per,
 *     bit L = p0*(u%per) + 8*e2 + 16*e1, field width p0 (code bits 0..p0-1).
 *   plane 1 (width p1, dwords m in [4*p0, 4*p0+4*p1)): with d = u/per the
 *     plane-0 dword, R = p0/p1: dword 4*p0 + d/R, bit
 *     p0*(u%per) + 16*e1 + p1*(d%R) + 8*e2, field width p1 (code bits p0..).
 * Dequantized weight: w_hat = fp16_RNE((c - 2^(b-1)) * s), s the fp16 scale.
 *
 * Every function here walks bits and elements one at a time, in the order of
 * the definitions above, in double precision where floating point is
 * involved.  Pins: see the tests (brute-force code enumeration, an
 * independent pure-Python bit reader, numpy float16 rounding, the integer
 * closed form and one-hot rows).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 128

/* ------------------------------------------------------------------ fp16 */

/* IEEE 754 binary16 from a double, round to nearest, ties to even,
 * subnormals kept, overflow to infinity. */
uint16_t oracle_f16_from_double(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return 0x7E00u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a) || a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;          /* a in [2^E, 2^(E+1)) */
    if (E < -14) {
        /* subnormal range: spacing 2^-24 */
        double m = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m); /* m == 1024 is the smallest normal */
    }
    double m = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024));
}

double oracle_f16_to_double(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* ---------------------------------------------------------------- layout */

static int plane0_width(int b) { return (b == 2 || b == 3) ? 2 : (b == 8 ? 8 : 4); }
static int plane1_width(int b) { return b - plane0_width(b); }

static int width_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }

/* Position of the `plane` field of code k in a width-b group: column-local
 * dword index and bit offset.  Returns the field width. */
int oracle_field_position(int b, int k, int plane, int* dword_out, int* bit_out) {
    int p0 = plane0_width(b), p1 = plane1_width(b);
    int u = k / 4, e = k % 4, e1 = e % 2, e2 = e / 2;
    int per = 8 / p0;
    int d = u / per, t = u % per;
    if (plane == 0) {
        *dword_out = d;
        *bit_out = p0 * t + 8 * e2 + 16 * e1;
        return p0;
    }
    if (p1 == 0) return 0;
    int R = p0 / p1;
    *dword_out = 4 * p0 + d / R;
    *bit_out = p0 * t + 16 * e1 + p1 * (d % R) + 8 * e2;
    return p1;
}

static uint64_t prefix_words(const uint8_t* widths, int g) {
    uint64_t p = 0;
    for (int h = 0; h < g; ++h) p += widths[h];
    return p;
}

/* Byte address of column-local dword m of column n in group g. */
static uint64_t dword_byte(int N, uint64_t Pg, int n, int m) {
    int j = m / 4, r = m % 4;
    return 16ull * ((uint64_t)N * Pg + (uint64_t)j * (uint64_t)N + (uint64_t)n) + 4ull * (uint64_t)r;
}

static int get_bit(const uint8_t* buf, uint64_t byte, int bit) {
    /* dwords are little endian: bit t of a dword is bit t%8 of byte t/8 */
    return (buf[byte + (uint64_t)(bit / 8)] >> (bit % 8)) & 1;
}

static void set_bit(uint8_t* buf, uint64_t byte, int bit, int v) {
    uint8_t mask = (uint8_t)(1u << (bit % 8));
    if (v) buf[byte + (uint64_t)(bit / 8)] |= mask;
    else buf[byte + (uint64_t)(bit / 8)] &= (uint8_t)~mask;
}

uint64_t oracle_packed_bytes(int K, int N, const uint8_t* widths) {
    int G = K / ORACLE_GROUP;
    uint64_t total = 0;
    for (int g = 0; g < G; ++g) total += (uint64_t)widths[g] * ORACLE_GROUP * (uint64_t)N / 8;
    return total;
}

static int read_code(const uint8_t* qw, int N, uint64_t Pg, int b, int n, int k) {
    int c = 0, shift = 0;
    for (int plane = 0; plane < 2; ++plane) {
        int dw, bit;
        int w = oracle_field_position(b, k, plane, &dw, &bit);
        if (w == 0) break;
        uint64_t byte = dword_byte(N, Pg, n, dw);
        for (int i = 0; i < w; ++i) c |= get_bit(qw, byte, bit + i) << (shift + i);
        shift += w;
    }
    return c;
}

/* codes: uint8 [N][K] row-major, code c in [0, 2^b). */
int oracle_pack(const uint8_t* codes, int K, int N, const uint8_t* widths, uint8_t* qweight) {
    if (K % ORACLE_GROUP) return 1;
    int G = K / ORACLE_GROUP;
    memset(qweight, 0, (size_t)oracle_packed_bytes(K, N, widths));
    for (int g = 0; g < G; ++g)
        if (!width_ok(widths[g])) return 1;
    int bad = 0;
    /* groups own disjoint byte ranges, so they can be filled concurrently */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int g = 0; g < G; ++g) {
        int b = widths[g];
        uint64_t Pg = prefix_words(widths, g);
        for (int n = 0; n < N; ++n) {
            for (int k = 0; k < ORACLE_GROUP; ++k) {
                int c = codes[(size_t)n * K + (size_t)g * ORACLE_GROUP + k];
                if (c >= (1 << b)) { bad = 1; continue; }
                int shift = 0;
                for (int plane = 0; plane < 2; ++plane) {
                    int dw, bit;
                    int w = oracle_field_position(b, k, plane, &dw, &bit);
                    if (w == 0) break;
                    uint64_t byte = dword_byte(N, Pg, n, dw);
                    for (int i = 0; i < w; ++i) set_bit(qweight, byte, bit + i, (c >> (shift + i)) & 1);
                    shift += w;
                }
            }
        }
    }
    return bad;
}

int oracle_unpack(const uint8_t* qweight, int K, int N, const uint8_t* widths, uint8_t* codes) {
    if (K % ORACLE_GROUP) return 1;
    int G = K / ORACLE_GROUP;
    for (int g = 0; g < G; ++g)
        if (!width_ok(widths[g])) return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int g = 0; g < G; ++g) {
        int b = widths[g];
        uint64_t Pg = prefix_words(widths, g);
        for (int n = 0; n < N; ++n)
            for (int k = 0; k < ORACLE_GROUP; ++k)
                codes[(size_t)n * K + (size_t)g * ORACLE_GROUP + k] = (uint8_t)read_code(qweight, N, Pg, b, n, k);
    }
    return 0;
}

/* -------------------------------------------------------------- quantize */

/* Symmetric round-to-nearest group quantizer.
 * s = fp16_RNE(fp32(max|w|) / fp32(2^(b-1)-1)), the division in fp32;
 * q = clamp(rint_even(fp32(w) / fp32(s)), -(2^(b-1)-1), 2^(b-1)-1);
 * c = q + 2^(b-1).  If s == 0 every code is 2^(b-1).
 * Returns 2 if a scale is not a finite fp16. */
int oracle_quantize(const float* W, int K, int N, const uint8_t* widths, uint8_t* codes, uint16_t* scales) {
    if (K % ORACLE_GROUP) return 1;
    int G = K / ORACLE_GROUP;
    for (int g = 0; g < G; ++g) {
        int b = widths[g];
        if (!width_ok(b)) return 1;
        int z = 1 << (b - 1), qmax = z - 1;
        int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
        for (int n = 0; n < N; ++n) {
            const float* w = W + (size_t)n * K + (size_t)g * ORACLE_GROUP;
            float amax = 0.0f;
            for (int i = 0; i < ORACLE_GROUP; ++i) {
                float a = fabsf(w[i]);
                if (a > amax) amax = a;
            }
            volatile float quotient = amax / (float)qmax;
            uint16_t s16 = oracle_f16_from_double((double)quotient);
            if ((s16 & 0x7C00u) == 0x7C00u) { overflow = 1; continue; }
            scales[(size_t)g * N + n] = s16;
            float s = (float)oracle_f16_to_double(s16);
            uint8_t* c = codes + (size_t)n * K + (size_t)g * ORACLE_GROUP;
            for (int i = 0; i < ORACLE_GROUP; ++i) {
                if (s == 0.0f) { c[i] = (uint8_t)z; continue; }
                volatile float r = w[i] / s;
                float q = nearbyintf(r);
                if (q > (float)qmax) q = (float)qmax;
                if (q < (float)-qmax) q = (float)-qmax;
                c[i] = (uint8_t)((int)q + z);
            }
        }
        if (overflow) return 2;
    }
    return 0;
}

/* Codes of one column's group at fp16 scale s16 (the rule of
 * oracle_quantize); returns sum_i (w_i - w_hat_i)^2 in double, i ascending,
 * w_hat = fp16_RNE((c - z) * s). */
static double quantize_group_at(const float* w, int b, uint16_t s16, uint8_t* c) {
    int z = 1 << (b - 1), qmax = z - 1;
    float s = (float)oracle_f16_to_double(s16);
    double err = 0.0;
    for (int i = 0; i < ORACLE_GROUP; ++i) {
        int q = 0;
        if (s != 0.0f) {
            volatile float r = w[i] / s;
            float qq = nearbyintf(r);
            if (qq > (float)qmax) qq = (float)qmax;
            if (qq < (float)-qmax) qq = (float)-qmax;
            q = (int)qq;
        }
        c[i] = (uint8_t)(q + z);
        double wh = oracle_f16_to_double(oracle_f16_from_double((double)q * (double)s));
        double d = (double)w[i] - wh;
        err += d * d;
    }
    return err;
}

/* The fp16 scale of 4-bit scale code q under column reference R at width b:
 * fp16_RNE(fp32(t * fp32(1 / (2^(b-1)-1)))) with t = R (q+1)^2 / 256 (exact). */
static uint16_t qs_scale(float R, int q, int b) {
    volatile float t = R * (float)((q + 1) * (q + 1)) * 0.00390625f;
    volatile float inv = 1.0f / (float)((1 << (b - 1)) - 1);
    volatile float u = t * inv;
    return oracle_f16_from_double((double)u);
}

/* Quantized group scales: a 4-bit code per (group, column) relative to a
 * per-column reference, on a square-root scale (the exllamav2 report's 4-bit
 * second-level scale code, section "innovations", with a scan of candidate
 * scales by their error; the formula printed there is garbled, so this is
 * our specification).  The coded quantity is the group's range max|w|,
 * which does not depend on its width:
 *   amax[g][n] = max |w| over the group (fp32)
 *   R[n]       = fp16_RNE(max_g amax[g][n])
 *   qc[g][n]   = clamp(ceil(16 * sqrtf(amax / fp32(R))), 1, 16) - 1, in fp32
 *                (IEEE division and square root): the smallest code whose
 *                scale covers the range; 0 if R == 0
 *   scale(q)   = fp16_RNE(fp32(t * fp32(1 / (2^(b-1) - 1)))), t = fp32(R)(q+1)^2/256
 *   q[g][n]    = qc, or qc - 1 if that gives a strictly smaller squared error
 *                sum_i (w_i - w_hat_i)^2 (double, i ascending; qc >= 1)
 * with codes by the rule of oracle_quantize at scale(q).  Storage: R fp16 [N];
 * qscale bytes [G][N/2], byte g*(N/2) + n/2 holding q of column n in its low
 * nibble for even n and its high nibble for odd n.  scales_out receives the
 * expanded scale(q) [G][N].  N must be even.  Returns 2 if R is not a finite
 * fp16. */
int oracle_quantize_qs(const float* W, int K, int N, const uint8_t* widths, uint8_t* codes, uint16_t* ref_out,
                       uint8_t* qscale, uint16_t* scales_out) {
    if (K % ORACLE_GROUP || N % 2) return 1;
    int G = K / ORACLE_GROUP;
    for (int g = 0; g < G; ++g)
        if (!width_ok(widths[g])) return 1;
    int overflow = 0;
    uint8_t* qcode = (uint8_t*)malloc((size_t)G * N);   /* q[g][n], packed into nibbles at the end */
    if (!qcode) return 3;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int n = 0; n < N; ++n) {
        float mx = 0.0f;
        for (int g = 0; g < G; ++g)
            for (int i = 0; i < ORACLE_GROUP; ++i) {
                float a = fabsf(W[(size_t)n * K + (size_t)g * ORACLE_GROUP + i]);
                if (a > mx) mx = a;
            }
        uint16_t r16 = oracle_f16_from_double((double)mx);
        if ((r16 & 0x7C00u) == 0x7C00u) { overflow = 1; continue; }
        ref_out[n] = r16;
        float R = (float)oracle_f16_to_double(r16);
        uint8_t alt[ORACLE_GROUP];
        for (int g = 0; g < G; ++g) {
            int b = widths[g];
            const float* w = W + (size_t)n * K + (size_t)g * ORACLE_GROUP;
            uint8_t* c = codes + (size_t)n * K + (size_t)g * ORACLE_GROUP;
            float amax = 0.0f;
            for (int i = 0; i < ORACLE_GROUP; ++i) {
                float a = fabsf(w[i]);
                if (a > amax) amax = a;
            }
            int q = 0;
            if (R != 0.0f) {
                volatile float ratio = amax / R;
                volatile float root = sqrtf(ratio);
                float t = ceilf(16.0f * root);
                q = (t < 1.0f ? 1 : (t > 16.0f ? 16 : (int)t)) - 1;
            }
            uint16_t s16 = qs_scale(R, q, b);
            double e = quantize_group_at(w, b, s16, c);
            if (q >= 1) {
                uint16_t s16b = qs_scale(R, q - 1, b);
                double eb = quantize_group_at(w, b, s16b, alt);
                if (eb < e) {
                    q -= 1;
                    s16 = s16b;
                    memcpy(c, alt, ORACLE_GROUP);
                }
            }
            qcode[(size_t)g * N + n] = (uint8_t)q;
            scales_out[(size_t)g * N + n] = s16;
        }
    }
    for (int g = 0; g < G && !overflow; ++g)
        for (int n = 0; n < N; n += 2)
            qscale[(size_t)g * (N / 2) + n / 2] =
                (uint8_t)(qcode[(size_t)g * N + n] | (qcode[(size_t)g * N + n + 1] << 4));
    free(qcode);
    return overflow ? 2 : 0;
}

/* ---------------------------------------------------------------- dequant */

/* w_hat fp16 bits [K][N] row-major from codes [N][K] and scales [G][N]. */
int oracle_dequant(const uint8_t* codes, const uint16_t* scales, int K, int N, const uint8_t* widths, uint16_t* w_hat) {
    if (K % ORACLE_GROUP) return 1;
#pragma omp parallel for schedule(static)
    for (int k = 0; k < K; ++k) {
        int g = k / ORACLE_GROUP, b = widths[g], z = 1 << (b - 1);
        for (int n = 0; n < N; ++n) {
            double s = oracle_f16_to_double(scales[(size_t)g * N + n]);
            double prod = (double)((int)codes[(size_t)n * K + k] - z) * s; /* exact */
            w_hat[(size_t)k * N + n] = oracle_f16_from_double(prod);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ gemm */

/* y[m][n] = sum_k x[m][k] * w_hat[k][n], k ascending, in double;
 * bound[m][n] = sum_k |x[m][k] * w_hat[k][n]|. */
void oracle_gemm(const uint16_t* x, int M, const uint16_t* w_hat, int K, int N, double* y, double* bound) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n) {
        for (int m = 0; m < M; ++m) {
            double acc = 0.0, abs_acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double p = oracle_f16_to_double(x[(size_t)m * K + k]) * oracle_f16_to_double(w_hat[(size_t)k * N + n]);
                acc += p;
                abs_acc += fabs(p);
            }
            y[(size_t)m * N + n] = acc;
            if (bound) bound[(size_t)m * N + n] = abs_acc;
        }
    }
}

/* The whole path from packed storage for the listed columns: read each code
 * bit by bit, dequantize, and accumulate in double.  y, bound: [M][ncols]. */
int oracle_gemm_packed_cols(const uint16_t* x, int M, const uint8_t* qweight, const uint16_t* scales,
                            const uint8_t* widths, int K, int N, const int64_t* cols, int64_t ncols,
                            double* y, double* bound) {
    if (K % ORACLE_GROUP) return 1;
    int G = K / ORACLE_GROUP;
    uint64_t* P = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(G + 1));
    if (!P) return 3;
    P[0] = 0;
    for (int g = 0; g < G; ++g) {
        if (!width_ok(widths[g])) { free(P); return 1; }
        P[g + 1] = P[g] + widths[g];
    }
    double* xd = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
    if (!xd) { free(P); return 3; }
    for (size_t i = 0; i < (size_t)M * (size_t)K; ++i) xd[i] = oracle_f16_to_double(x[i]);
#pragma omp parallel
    {
        double* wcol = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t ci = 0; ci < ncols; ++ci) {
            int n = (int)cols[ci];
            for (int g = 0; g < G; ++g) {
                int b = widths[g], z = 1 << (b - 1);
                double s = oracle_f16_to_double(scales[(size_t)g * N + n]);
                for (int k = 0; k < ORACLE_GROUP; ++k) {
                    int c = read_code(qweight, N, P[g], b, n, k);
                    wcol[g * ORACLE_GROUP + k] = oracle_f16_to_double(oracle_f16_from_double((double)(c - z) * s));
                }
            }
            for (int m = 0; m < M; ++m) {
                double acc = 0.0, abs_acc = 0.0;
                const double* xr = xd + (size_t)m * K;
                for (int k = 0; k < K; ++k) {
                    double p = xr[k] * wcol[k];
                    acc += p;
                    abs_acc += fabs(p);
                }
                y[(size_t)m * ncols + ci] = acc;
                if (bound) bound[(size_t)m * ncols + ci] = abs_acc;
            }
        }
        free(wcol);
    }
    free(xd);
    free(P);
    return 0;
}
