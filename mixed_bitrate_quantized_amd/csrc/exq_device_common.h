// Device-side definitions shared by the decode and prefill kernels of libexq
// (gfx950): the per-linear launch descriptor, buffer-resource and global
// pointer helpers, and the EXQ1 decoder-unit extraction.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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
    const uint32_t* order;    // [G]: g | (P_g << 16), sorted by width
    const uint16_t* bounds;   // [kWaves + 1] wave chunks of `order`
    const uint16_t* runs;     // [kWaves][6] groups of width 2,3,4,5,6,8 per chunk
    const uint16_t* x;        // fp16 [M][K]
    uint16_t* y;              // fp16 [M][N]
    int K, N, G, tiles;
    uint32_t qbytes;          // bytes of qweight (< 2^31)
    uint32_t sbytes;          // bytes of scales
    const uint8_t* qscale;    // quantized scales: 4-bit codes [G][N/2] (else null)
    const uint16_t* ref;      // quantized scales: fp16 column range references [N]
    uint32_t qsbytes;         // bytes of qscale
    int qs;                   // 1: decode reads qscale/ref (scales holds their expansion)
};

// Weights and scales are read with raw buffer loads.  A load whose offset is
// past the buffer's size returns zeros without touching memory: the
// pipeline's tail steps use that to keep a fixed load count per step at no
// memory cost.
constexpr uint32_t kBufOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Global-address-space views: loads through them are global_load (vmcnt
// only), never flat_load, whose lgkmcnt coupling would make every LDS read
// wait for all weight loads in flight.
#define EXQ_GLOBAL __attribute__((address_space(1)))
template <class T> __device__ __forceinline__ const EXQ_GLOBAL T* gptr(const void* p) {
    return (const EXQ_GLOBAL T*)p;
}
template <class T> __device__ __forceinline__ EXQ_GLOBAL T* gptr_w(void* p) { return (EXQ_GLOBAL T*)p; }

// LDS destination of a buffer load that writes LDS directly.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Decoder unit U of a width-B group, on the dwords of NQ consecutive
// K-quarters (NQ = 4: the whole group, U in [0, 32); NQ = 1: quarter q, U in
// [0, 8) covering codes 32q + 4U ..).  Q holds the NQ*p0 plane-0 dwords then
// the NQ*p1 plane-1 dwords.  Returns two dwords whose 16-bit
// halves hold codes 4U, 4U+1 (b0) and 4U+2, 4U+3 (b1), each at bit offset
// o = p0 * (U % per) of its half, every other bit clear.  Read as fp16 the
// halves are exactly c * 2^(o-24).  Bit positions follow the EXQ1 layout
// (include/exq.h); the quarter split keeps dword-local positions unchanged.
template <int B, int U, int NQ = 1>
__device__ __forceinline__ void unit_pair(const uint32_t* Q, uint32_t& b0, uint32_t& b1) {
    using T = Width<B>;
    constexpr int d = U / T::per, t = U % T::per, o = T::p0 * t;
    constexpr uint32_t mlo = (((1u << T::p0) - 1u) * 0x00010001u) << o;
    const uint32_t lo0 = Q[d], lo1 = Q[d] >> 8;
    if constexpr (T::p1 == 0) {
        b0 = lo0 & mlo;
        b1 = lo1 & mlo;
    } else {
        constexpr int h = d / T::R, delta = d % T::R;
        constexpr uint32_t mhi = (((1u << T::p1) - 1u) * 0x00010001u) << (o + T::p0);
        constexpr int sh0 = T::p0 - T::p1 * delta;      // left shift, high fields of codes 4U, 4U+1
        constexpr int sh1 = T::p1 * delta + 8 - T::p0;  // right shift, codes 4U+2, 4U+3
        static_assert(sh0 > 0 && sh1 > 0, "plane-1 alignment");
        const uint32_t H = Q[NQ * T::p0 + h];
        b0 = (lo0 & mlo) | ((H << sh0) & mhi);
        b1 = (lo1 & mlo) | ((H >> sh1) & mhi);
    }
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// fp16 pair view of a dword.  The argument is a plain scalar on purpose:
// __builtin_bit_cast applied directly to an ext_vector element (x[i]) has
// been seen to read element 0 whatever i is.
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// Descriptor of `layer` bound to x and y (device pointers).
LinearDev linear_dev(const exq_layer* layer, const void* x, void* y);

}  // namespace exq
