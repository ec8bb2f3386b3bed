// Device half of libexq for gfx950: decode GEMV, dequantization, layer and
// plan management.  The prefill GEMM lives in exq_prefill.hip.
//
// Decode design (M <= 16, HBM-bound):
//   * one lane per output column, 64 columns per wave, all four waves of a
//     workgroup on the same 64 columns but on different byte-balanced runs of
//     K groups; the column's b_g 16-byte words of a group arrive as b_g
//     coalesced 1 KB wave loads;
//   * a code field is masked in place into the low bits of an fp16 half, which
//     then *is* the fp16 value c * 2^(o-24) (a subnormal): one AND per two
//     weights, no conversion, no zero-point subtraction per weight;
//   * the multiply-accumulate runs on the matrix cores with
//     v_mfma_f32_4x4x4_16b_f16: 16 blocks of 4 columns, the activation operand
//     of one block broadcast to all 16 (cbsz = 4), so the activations of a
//     whole group fit in four VGPRs per row block;
//   * per group, the per-offset partial sums are rescaled by 2^(24-o), the
//     zero point is removed once with the group's activation sum (computed per
//     workgroup into LDS), and the fp16 scale is applied in fp32:
//       y += s * (sum_k x_k c_k - 2^(b-1) sum_k x_k);
//   * waves reduce through LDS in fixed order; when K is split across
//     workgroups the last one to finish adds the fp32 partials in split order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <type_traits>
#include <vector>

#include "exq_internal.h"

namespace exq {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));

// Everything a kernel needs about one linear of a launch.
struct LinearDev {
    const uint8_t* qweight;   // EXQ1 words
    const uint16_t* scales;   // fp16 [G][N]
    const uint32_t* meta;     // [G]: (P_g << 4) | b_g
    const uint16_t* bounds;   // [S*kWaves + 1] group cut points
    const uint16_t* x;        // fp16 [M][K]
    uint16_t* y;              // fp16 [M][N]
    float* partial;           // fp32 [S][M][N] split-K partial sums (S > 1)
    uint32_t* counters;       // [N/64] arrival counters (S > 1), zero between launches
    int K, N, G, S, tiles, wg_begin;
};

template <int I> using IC = std::integral_constant<int, I>;

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// Plane split of a width: plane 0 of p0 bits, plane 1 of p1 bits (or none).
template <int B> struct Width {
    static constexpr int p0 = (B <= 3) ? 2 : (B == 8 ? 8 : 4);
    static constexpr int p1 = B - p0;
    static constexpr int per = 8 / p0;            // decoder units per plane-0 dword
    static constexpr int R = p1 ? p0 / p1 : 1;    // plane-0 dwords per plane-1 dword
};

__device__ __forceinline__ h4 as_h4(uint32_t a, uint32_t b) {
    u2v v = {a, b};
    return __builtin_bit_cast(h4, v);
}

// Decoder unit U of a width-B group (U in [0,32)): returns two dwords whose
// 16-bit halves hold codes 4U, 4U+1 (b0) and 4U+2, 4U+3 (b1), each code at bit
// offset o = p0*(U % per) of its half and every other bit clear.  Read as fp16
// the halves are exactly c * 2^(o-24).  The bit positions follow the EXQ1
// layout of include/exq.h.
template <int B, int U>
__device__ __forceinline__ void unit_pair(const uint32_t* D, uint32_t& b0, uint32_t& b1) {
    using T = Width<B>;
    constexpr int d = U / T::per, t = U % T::per, o = T::p0 * t;
    constexpr uint32_t mlo = (((1u << T::p0) - 1u) * 0x00010001u) << o;
    const uint32_t lo0 = D[d], lo1 = D[d] >> 8;
    if constexpr (T::p1 == 0) {
        b0 = lo0 & mlo;
        b1 = lo1 & mlo;
    } else {
        constexpr int h = d / T::R, delta = d % T::R;
        constexpr uint32_t mhi = (((1u << T::p1) - 1u) * 0x00010001u) << (o + T::p0);
        constexpr int sh0 = T::p0 - T::p1 * delta;      // left shift, high fields of codes 4U, 4U+1
        constexpr int sh1 = T::p1 * delta + 8 - T::p0;  // right shift, codes 4U+2, 4U+3
        static_assert(sh0 > 0 && sh1 > 0, "plane-1 alignment");
        const uint32_t H = D[4 * T::p0 + h];
        b0 = (lo0 & mlo) | ((H << sh0) & mhi);
        b1 = (lo1 & mlo) | ((H >> sh1) & mhi);
    }
}

template <int B> __device__ constexpr float class_factor(int t) {
    // 2^(24 - o), o = p0 * t: turns c * 2^(o-24) back into c.
    return (float)(1u << (24 - Width<B>::p0 * t));
}

// ----------------------------------------------------------------- decode

template <int MB>
__device__ __forceinline__ void load_group(const LinearDev& L, int g, int M, int n, int lane,
                                           uint32_t (&D)[32], u4v (&X)[MB], uint16_t& s, int& b) {
    const uint32_t meta = L.meta[g];
    b = (int)(meta & 15u);
    const size_t P = meta >> 4;
    const u4v* base = reinterpret_cast<const u4v*>(L.qweight) + ((size_t)L.N * P + (size_t)n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < b) {
            u4v v = __builtin_nontemporal_load(base + (size_t)j * (size_t)L.N);
            D[4 * j + 0] = v[0];
            D[4 * j + 1] = v[1];
            D[4 * j + 2] = v[2];
            D[4 * j + 3] = v[3];
        }
    }
    s = L.scales[(size_t)g * L.N + n];
    const int a = lane >> 2, i = lane & 3;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
        const int row = min(4 * rb + i, M - 1);
        X[rb] = *reinterpret_cast<const u4v*>(L.x + (size_t)row * L.K + (size_t)g * kGroup + 8 * a);
    }
}

template <int B, int MB>
__device__ __forceinline__ void group_compute(const uint32_t (&D)[32], const u4v (&X)[MB], uint16_t s16,
                                              const float* xs, int xs_stride, int M, float (&yacc)[MB][4]) {
    constexpr int C = Width<B>::per;
    f4 acc[C][MB];
#pragma unroll
    for (int t = 0; t < C; ++t)
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) acc[t][rb] = f4{0.f, 0.f, 0.f, 0.f};
    static_for<0, 32>([&](auto UC) {
        constexpr int U = decltype(UC)::value;
        constexpr int t = U % C;
        uint32_t b0, b1;
        unit_pair<B, U>(D, b0, b1);
        const h4 bv = as_h4(b0, b1);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            const h4 av = (U & 1) ? as_h4(X[rb][2], X[rb][3]) : as_h4(X[rb][0], X[rb][1]);
            acc[t][rb] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bv, acc[t][rb], 4, U >> 1, 0);
        }
    });
    const float s = (float)__builtin_bit_cast(_Float16, s16);
    constexpr float z = (float)(1 << (B - 1));
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (4 * rb + r < M) {
                float tv = acc[0][rb][r] * class_factor<B>(0);
#pragma unroll
                for (int t = 1; t < C; ++t) tv = __builtin_fmaf(acc[t][rb][r], class_factor<B>(t), tv);
                tv = __builtin_fmaf(-z, xs[(4 * rb + r) * xs_stride], tv);
                yacc[rb][r] = __builtin_fmaf(s, tv, yacc[rb][r]);
            }
        }
}

template <int MB>
__device__ __forceinline__ void group_dispatch(int b, const uint32_t (&D)[32], const u4v (&X)[MB], uint16_t s,
                                               const float* xs, int xs_stride, int M, float (&yacc)[MB][4]) {
    switch (b) {
        case 2: group_compute<2, MB>(D, X, s, xs, xs_stride, M, yacc); break;
        case 3: group_compute<3, MB>(D, X, s, xs, xs_stride, M, yacc); break;
        case 4: group_compute<4, MB>(D, X, s, xs, xs_stride, M, yacc); break;
        case 5: group_compute<5, MB>(D, X, s, xs, xs_stride, M, yacc); break;
        case 6: group_compute<6, MB>(D, X, s, xs, xs_stride, M, yacc); break;
        default: group_compute<8, MB>(D, X, s, xs, xs_stride, M, yacc); break;
    }
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// One workgroup of the decode GEMV: 64 columns, one split of K.
template <int MB>
__device__ __forceinline__ void decode_wg(const LinearDev& L, int local, int M, float* lds) {
    const int tile = local % L.tiles, split = local / L.tiles;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = tile * kTileCols + lane;
    const int g0 = L.bounds[split * kWaves], g1 = L.bounds[split * kWaves + kWaves];
    const int gs = g1 - g0;
    float* xsum = lds;                       // [M][gs]
    float* red = lds + ((M * gs + 3) & ~3);  // [kWaves][M][64]

    // Activation sums of every group of this split, 32 values per thread,
    // combined in a fixed order.
    for (int idx = threadIdx.x; idx < M * gs * 4; idx += 256) {
        const int m = idx / (gs * 4), rem = idx - m * gs * 4;
        const int gl = rem >> 2, part = rem & 3;
        const u4v* p = reinterpret_cast<const u4v*>(L.x + (size_t)m * L.K + (size_t)(g0 + gl) * kGroup + 32 * part);
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            u4v v = p[q];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc += (float)__builtin_bit_cast(_Float16, (uint16_t)(v[w] & 0xFFFFu));
                acc += (float)__builtin_bit_cast(_Float16, (uint16_t)(v[w] >> 16));
            }
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if (part == 0) xsum[m * gs + gl] = acc;
    }
    __syncthreads();

    const int wb = L.bounds[split * kWaves + wave], we = L.bounds[split * kWaves + wave + 1];
    float yacc[MB][4];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[rb][r] = 0.f;

    uint32_t DA[32], DB[32];
    u4v XA[MB], XB[MB];
    uint16_t sA = 0, sB = 0;
    int bA = 2, bB = 2;
    if (wb < we) load_group<MB>(L, wb, M, n, lane, DA, XA, sA, bA);
    for (int g = wb; g < we; g += 2) {
        if (g + 1 < we) load_group<MB>(L, g + 1, M, n, lane, DB, XB, sB, bB);
        group_dispatch<MB>(bA, DA, XA, sA, xsum + (g - g0), gs, M, yacc);
        if (g + 1 < we) {
            if (g + 2 < we) load_group<MB>(L, g + 2, M, n, lane, DA, XA, sA, bA);
            group_dispatch<MB>(bB, DB, XB, sB, xsum + (g + 1 - g0), gs, M, yacc);
        }
    }

#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (4 * rb + r < M) red[(wave * M + 4 * rb + r) * 64 + lane] = yacc[rb][r];
    __syncthreads();

    const int ncol0 = tile * kTileCols;
    if (L.S == 1) {
        for (int t = threadIdx.x; t < M * 64; t += 256) {
            const int m = t >> 6, c = t & 63;
            float v = red[(0 * M + m) * 64 + c];
            v += red[(1 * M + m) * 64 + c];
            v += red[(2 * M + m) * 64 + c];
            v += red[(3 * M + m) * 64 + c];
            L.y[(size_t)m * L.N + ncol0 + c] = f32_to_f16_bits(v);
        }
        return;
    }
    for (int t = threadIdx.x; t < M * 64; t += 256) {
        const int m = t >> 6, c = t & 63;
        float v = red[(0 * M + m) * 64 + c];
        v += red[(1 * M + m) * 64 + c];
        v += red[(2 * M + m) * 64 + c];
        v += red[(3 * M + m) * 64 + c];
        L.partial[((size_t)split * M + m) * L.N + ncol0 + c] = v;
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (threadIdx.x == 0) last = (atomicAdd(&L.counters[tile], 1u) == (uint32_t)(L.S - 1));
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int t = threadIdx.x; t < M * 64; t += 256) {
        const int m = t >> 6, c = t & 63;
        float v = 0.f;
        for (int sp = 0; sp < L.S; ++sp) v += L.partial[((size_t)sp * M + m) * L.N + ncol0 + c];
        L.y[(size_t)m * L.N + ncol0 + c] = f32_to_f16_bits(v);
    }
    if (threadIdx.x == 0) L.counters[tile] = 0u;
}

template <int MB>
__global__ __launch_bounds__(256) void decode_kernel(LinearDev L, int M) {
    extern __shared__ float lds[];
    decode_wg<MB>(L, blockIdx.x, M, lds);
}

template <int MB>
__global__ __launch_bounds__(256) void decode_plan_kernel(const LinearDev* __restrict__ list,
                                                          const uint16_t* __restrict__ wg_map, int M) {
    extern __shared__ float lds[];
    const int li = wg_map[blockIdx.x];
    const LinearDev L = list[li];
    decode_wg<MB>(L, blockIdx.x - L.wg_begin, M, lds);
}

// ---------------------------------------------------------------- dequant

template <int B>
__device__ __forceinline__ void dequant_group(const uint32_t (&D)[32], float s, int N, int n, uint16_t* out) {
    constexpr int C = Width<B>::per;
    constexpr int z = 1 << (B - 1);
    static_for<0, 32>([&](auto UC) {
        constexpr int U = decltype(UC)::value;
        constexpr int o = Width<B>::p0 * (U % C);
        uint32_t b0, b1;
        unit_pair<B, U>(D, b0, b1);
        const uint32_t c[4] = {(b0 & 0xFFFFu) >> o, b0 >> (16 + o), (b1 & 0xFFFFu) >> o, b1 >> (16 + o)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // (c - z) * s is exact in fp32; one rounding to fp16.
            const float w = (float)((int)c[e] - z) * s;
            out[(size_t)(4 * U + e) * N + n] = f32_to_f16_bits(w);
        }
    });
}

__global__ __launch_bounds__(64) void dequant_kernel(LinearDev L, uint16_t* __restrict__ w_out) {
    const int g = blockIdx.y;
    const int n = blockIdx.x * kTileCols + threadIdx.x;
    uint32_t D[32];
    u4v X[1];
    uint16_t s16;
    int b;
    // reuse the decode loader; x is not needed but its row-0 load is harmless
    load_group<1>(L, g, 1, n, threadIdx.x, D, X, s16, b);
    const float s = (float)__builtin_bit_cast(_Float16, s16);
    uint16_t* out = w_out + (size_t)g * kGroup * L.N;
    switch (b) {
        case 2: dequant_group<2>(D, s, L.N, n, out); break;
        case 3: dequant_group<3>(D, s, L.N, n, out); break;
        case 4: dequant_group<4>(D, s, L.N, n, out); break;
        case 5: dequant_group<5>(D, s, L.N, n, out); break;
        case 6: dequant_group<6>(D, s, L.N, n, out); break;
        default: dequant_group<8>(D, s, L.N, n, out); break;
    }
}

}  // namespace exq

// =================================================================== host

using namespace exq;

struct exq_layer {
    int K, N, G;
    std::vector<uint8_t> widths;
    const void* qweight;
    const void* scales;
    SplitPlan plan;
    uint32_t* d_meta = nullptr;
    uint16_t* d_bounds = nullptr;
    float* d_partial = nullptr;
    uint32_t* d_counters = nullptr;
    uint16_t* d_zero_x = nullptr;  // K fp16 zeros, a valid x for the dequant launch
};

struct exq_plan {
    int count = 0, M = 1, total_wgs = 0;
    size_t lds_bytes = 0;
    LinearDev* d_list = nullptr;
    uint16_t* d_wg_map = nullptr;
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return v ? atoi(v) : dflt;
}

exq_status hip_fail(hipError_t e, const char* what) {
    return fail(EXQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

LinearDev linear_dev(const exq_layer* L, const void* x, void* y) {
    LinearDev d;
    d.qweight = static_cast<const uint8_t*>(L->qweight);
    d.scales = static_cast<const uint16_t*>(L->scales);
    d.meta = L->d_meta;
    d.bounds = L->d_bounds;
    d.x = static_cast<const uint16_t*>(x);
    d.y = static_cast<uint16_t*>(y);
    d.partial = L->d_partial;
    d.counters = L->d_counters;
    d.K = L->K;
    d.N = L->N;
    d.G = L->G;
    d.S = L->plan.S;
    d.tiles = L->N / kTileCols;
    d.wg_begin = 0;
    return d;
}

size_t decode_lds_bytes(int M, int split_groups) {
    return sizeof(float) * (size_t)(((M * split_groups + 3) & ~3) + kWaves * M * 64);
}

exq_status launch_decode(const LinearDev& d, int M, int max_split_groups, hipStream_t stream) {
    const size_t lds = decode_lds_bytes(M, max_split_groups);
    const dim3 grid(d.tiles * d.S), block(256);
    switch ((M + 3) / 4) {
        case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, block, lds, stream, d, M); break;
        case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, lds, stream, d, M); break;
        case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, lds, stream, d, M); break;
        default: hipLaunchKernelGGL(decode_kernel<4>, grid, block, lds, stream, d, M); break;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "decode launch");
}

}  // namespace

extern exq_status exq_prefill_launch(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream);

// Decode kernel over consecutive 16-row slices of x (any M).
exq_status exq_decode_rows(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream) {
    for (int r0 = 0; r0 < M; r0 += kMaxDecodeM) {
        const int m = std::min(kMaxDecodeM, M - r0);
        const void* xs = static_cast<const uint16_t*>(x) + (size_t)r0 * L->K;
        void* ys = static_cast<uint16_t*>(y) + (size_t)r0 * L->N;
        exq_status st = launch_decode(linear_dev(L, xs, ys), m, L->plan.max_split_groups, stream);
        if (st != EXQ_OK) return st;
    }
    return EXQ_OK;
}

extern "C" {

exq_status exq_layer_create(int K, int N, int group_size, const uint8_t* widths_host,
                            const void* d_qweight, const void* d_scales, exq_layer_t* out) {
    if (!out) return fail(EXQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    exq_status st = check_layer_shape(K, N, group_size, widths_host);
    if (st != EXQ_OK) return st;
    if (N % kTileCols) return fail(EXQ_ERR_INVALID_ARG, "N=%d is not a multiple of 64", N);
    if (!d_qweight || !d_scales) return fail(EXQ_ERR_INVALID_ARG, "NULL device buffer");
    if (!aligned16(d_qweight) || !aligned16(d_scales))
        return fail(EXQ_ERR_INVALID_ARG, "qweight and scales must be 16-byte aligned");
    const int G = K / kGroup;
    if ((size_t)8 * (size_t)G >= (1u << 28))
        return fail(EXQ_ERR_UNSUPPORTED, "K too large for 28-bit per-column word offsets");
    exq_layer* L = new (std::nothrow) exq_layer();
    if (!L) return fail(EXQ_ERR_OOM, "host allocation");
    L->K = K;
    L->N = N;
    L->G = G;
    L->widths.assign(widths_host, widths_host + G);
    L->qweight = d_qweight;
    L->scales = d_scales;
    L->plan = plan_splits(K, N, widths_host, env_int("EXQ_FORCE_SPLITS", 0));
    std::vector<uint32_t> meta = group_meta(K, widths_host);
    const int tiles = N / kTileCols;
    hipError_t e = hipSuccess;
    auto cleanup = [&](exq_status s) { exq_layer_destroy(L); return s; };
    if ((e = hipMalloc(&L->d_meta, sizeof(uint32_t) * G)) != hipSuccess) return cleanup(fail(EXQ_ERR_OOM, "hipMalloc meta"));
    if ((e = hipMalloc(&L->d_bounds, sizeof(uint16_t) * L->plan.bounds.size())) != hipSuccess)
        return cleanup(fail(EXQ_ERR_OOM, "hipMalloc bounds"));
    if ((e = hipMalloc(&L->d_zero_x, sizeof(uint16_t) * K)) != hipSuccess) return cleanup(fail(EXQ_ERR_OOM, "hipMalloc x"));
    if (L->plan.S > 1) {
        if ((e = hipMalloc(&L->d_partial, sizeof(float) * (size_t)L->plan.S * kMaxDecodeM * N)) != hipSuccess)
            return cleanup(fail(EXQ_ERR_OOM, "hipMalloc workspace"));
        if ((e = hipMalloc(&L->d_counters, sizeof(uint32_t) * tiles)) != hipSuccess)
            return cleanup(fail(EXQ_ERR_OOM, "hipMalloc counters"));
        if ((e = hipMemset(L->d_counters, 0, sizeof(uint32_t) * tiles)) != hipSuccess)
            return cleanup(hip_fail(e, "hipMemset counters"));
    }
    if ((e = hipMemcpy(L->d_meta, meta.data(), sizeof(uint32_t) * G, hipMemcpyHostToDevice)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMemcpy meta"));
    if ((e = hipMemcpy(L->d_bounds, L->plan.bounds.data(), sizeof(uint16_t) * L->plan.bounds.size(),
                       hipMemcpyHostToDevice)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMemcpy bounds"));
    if ((e = hipMemset(L->d_zero_x, 0, sizeof(uint16_t) * K)) != hipSuccess) return cleanup(hip_fail(e, "hipMemset x"));
    *out = L;
    return EXQ_OK;
}

void exq_layer_destroy(exq_layer_t L) {
    if (!L) return;
    if (L->d_meta) (void)hipFree(L->d_meta);
    if (L->d_bounds) (void)hipFree(L->d_bounds);
    if (L->d_partial) (void)hipFree(L->d_partial);
    if (L->d_counters) (void)hipFree(L->d_counters);
    if (L->d_zero_x) (void)hipFree(L->d_zero_x);
    delete L;
}

exq_status exq_gemm(const void* x, int M, exq_layer_t L, void* y, void* stream) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!x || !y) return fail(EXQ_ERR_INVALID_ARG, "NULL x or y");
    if (M < 1) return fail(EXQ_ERR_INVALID_ARG, "M=%d must be >= 1", M);
    if (!aligned16(x) || !aligned16(y)) return fail(EXQ_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (overlap(x, 2 * (size_t)M * L->K, y, 2 * (size_t)M * L->N)) return fail(EXQ_ERR_INVALID_ARG, "y overlaps x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M > kMaxDecodeM) return exq_prefill_launch(L, x, M, y, s);
    return launch_decode(linear_dev(L, x, y), M, L->plan.max_split_groups, s);
}

exq_status exq_dequant(exq_layer_t L, void* w_out, void* stream) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!w_out) return fail(EXQ_ERR_INVALID_ARG, "w_out is NULL");
    if (!aligned16(w_out)) return fail(EXQ_ERR_INVALID_ARG, "w_out must be 16-byte aligned");
    LinearDev d = linear_dev(L, L->d_zero_x, nullptr);
    hipLaunchKernelGGL(dequant_kernel, dim3(L->N / kTileCols, L->G), dim3(64), 0, static_cast<hipStream_t>(stream), d,
                       static_cast<uint16_t*>(w_out));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "dequant launch");
}

exq_status exq_plan_create(int count, const exq_layer_t* layers, const void* const* xs, const void* const* ys, int M,
                           exq_plan_t* out) {
    if (!out) return fail(EXQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (count < 1 || !layers || !xs || !ys) return fail(EXQ_ERR_INVALID_ARG, "empty or NULL plan arrays");
    if (M < 1 || M > kMaxDecodeM) return fail(EXQ_ERR_INVALID_ARG, "plan M=%d must be in [1, 16]", M);
    std::vector<LinearDev> list(count);
    std::vector<uint16_t> wg_map;
    int max_groups = 0;
    for (int i = 0; i < count; ++i) {
        const exq_layer* L = layers[i];
        if (!L || !xs[i] || !ys[i]) return fail(EXQ_ERR_INVALID_ARG, "plan entry %d is NULL", i);
        for (int j = 0; j < i; ++j)
            if (layers[j] == L) return fail(EXQ_ERR_INVALID_ARG, "layer of entry %d repeats entry %d (shared workspace)", i, j);
        if (!aligned16(xs[i]) || !aligned16(ys[i])) return fail(EXQ_ERR_INVALID_ARG, "plan entry %d misaligned", i);
        for (int j = 0; j < count; ++j) {
            if (overlap(ys[i], 2 * (size_t)M * L->N, xs[j], 2 * (size_t)M * layers[j]->K))
                return fail(EXQ_ERR_INVALID_ARG, "output %d overlaps input %d", i, j);
            if (j != i && overlap(ys[i], 2 * (size_t)M * L->N, ys[j], 2 * (size_t)M * layers[j]->N))
                return fail(EXQ_ERR_INVALID_ARG, "outputs %d and %d overlap", i, j);
        }
        list[i] = linear_dev(L, xs[i], const_cast<void*>(ys[i]));
        list[i].wg_begin = (int)wg_map.size();
        const int wgs = list[i].tiles * list[i].S;
        if (i >= 65535 || wg_map.size() + wgs > (size_t)INT32_MAX)
            return fail(EXQ_ERR_UNSUPPORTED, "plan too large");
        wg_map.insert(wg_map.end(), wgs, (uint16_t)i);
        max_groups = std::max(max_groups, L->plan.max_split_groups);
    }
    exq_plan* P = new (std::nothrow) exq_plan();
    if (!P) return fail(EXQ_ERR_OOM, "host allocation");
    P->count = count;
    P->M = M;
    P->total_wgs = (int)wg_map.size();
    P->lds_bytes = decode_lds_bytes(M, max_groups);
    hipError_t e;
    if ((e = hipMalloc(&P->d_list, sizeof(LinearDev) * count)) != hipSuccess ||
        (e = hipMalloc(&P->d_wg_map, sizeof(uint16_t) * wg_map.size())) != hipSuccess) {
        exq_plan_destroy(P);
        return fail(EXQ_ERR_OOM, "hipMalloc plan");
    }
    if ((e = hipMemcpy(P->d_list, list.data(), sizeof(LinearDev) * count, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(P->d_wg_map, wg_map.data(), sizeof(uint16_t) * wg_map.size(), hipMemcpyHostToDevice)) !=
            hipSuccess) {
        exq_plan_destroy(P);
        return hip_fail(e, "hipMemcpy plan");
    }
    *out = P;
    return EXQ_OK;
}

exq_status exq_plan_run(exq_plan_t P, void* stream) {
    if (!P) return fail(EXQ_ERR_INVALID_ARG, "plan is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(P->total_wgs), block(256);
    switch ((P->M + 3) / 4) {
        case 1: hipLaunchKernelGGL(decode_plan_kernel<1>, grid, block, P->lds_bytes, s, P->d_list, P->d_wg_map, P->M); break;
        case 2: hipLaunchKernelGGL(decode_plan_kernel<2>, grid, block, P->lds_bytes, s, P->d_list, P->d_wg_map, P->M); break;
        case 3: hipLaunchKernelGGL(decode_plan_kernel<3>, grid, block, P->lds_bytes, s, P->d_list, P->d_wg_map, P->M); break;
        default: hipLaunchKernelGGL(decode_plan_kernel<4>, grid, block, P->lds_bytes, s, P->d_list, P->d_wg_map, P->M); break;
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "plan launch");
}

void exq_plan_destroy(exq_plan_t P) {
    if (!P) return;
    if (P->d_list) (void)hipFree(P->d_list);
    if (P->d_wg_map) (void)hipFree(P->d_wg_map);
    delete P;
}

}  // extern "C"
