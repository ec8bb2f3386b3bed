// Device half of libexq for gfx950: decode GEMV, dequantization, layer and
// plan management.  The prefill GEMM (M > 16) lives in exq_prefill.hip.
//
// Decode design (M <= 16 per launch; larger M in 16-row slices):
//   * a workgroup owns 64 output columns (16 when N % 64 != 0) over the whole
//     of K; its 8 waves share the groups, pre-sorted by width and cut into
//     instruction-balanced chunks, so a wave streams one or two runs of
//     equal-width groups, each pipelined a fixed number of groups deep with
//     compile-time load counts (whole rounds, then the last partial round);
//   * a code field is masked in place into the low bits of an fp16 half,
//     which then *is* the fp16 value c * 2^(o-24) (a subnormal): one AND per
//     two weights, no conversion; one packed fp16 FMA by 2^-o with addend
//     -z * 2^-24 then gives (c - z) * 2^-24 exactly (the product and the
//     result are multiples of 2^-24 below 2^-14), so a weight whose code is
//     the zero point contributes an exact zero whatever its activation, and
//     fields at every bit offset feed one accumulator;
//   * M <= 4: lane l owns column l of the tile over the whole group (or
//     K-quarter l / 16 of column l % 16 in 16-column tiles), and
//     v_mfma_f32_4x4x4_16b_f16 multiplies with one activation block shared
//     by a set of 4x4 blocks (cbsz); a plan with at least 4 workgroups per
//     CU runs a high-occupancy instance (64 VGPRs, shallower pipelines);
//   * M = 5..16: the 16-row layout on v_mfma_f32_16x16x32_f16 (lane (j, c):
//     K-quarter j of columns c, c+16, c+32, c+48), with each group's
//     activations staged in a per-wave LDS ring for widths up to 6 bits;
//   * per group the partial sum is rescaled by 2^24 and the fp16 scale is
//     applied in fp32:  y += s * sum x * (c - z);
//   * quarters and waves are reduced in a fixed order: no atomics, the result
//     is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <type_traits>
#include <vector>

#include "exq_device_common.h"
#include "exq_internal.h"

namespace exq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// 2^24: the decoded weights are (c - z) * 2^-24 (see unbias); a wave's
// partial sums are multiplied by it once, on their way out.  With fp32
// partials far above the subnormal range (|x|, s >= 2^-24 give products of
// at least 2^-72) the power of two commutes exactly with every product and
// sum, so the result is bit for bit the one of unscaled arithmetic.
constexpr float kUnit = 16777216.0f;

// P_DW consecutive dwords at byte voff + soff of a buffer (voff per lane,
// soff uniform); aux 2: streamed once.
template <int P_DW>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t rw, uint32_t voff, uint32_t soff, uint32_t* dst) {
    if constexpr (P_DW == 1) {
        dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff, soff, 2);
    } else if constexpr (P_DW == 2) {
        const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rw, voff, soff, 2);
        dst[0] = v[0];
        dst[1] = v[1];
    } else {
        const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rw, voff, soff, 2);
        dst[0] = v[0];
        dst[1] = v[1];
        dst[2] = v[2];
        dst[3] = v[3];
    }
}

// Where quarter q of a column's group words sits.  Column-local dword m of a
// group is dword m % 4 of word m / 4, and word j of column n lies at byte
// 16 (N (P + j) + n) of the weight buffer (P: the group's first word row).
// Plane 0 of quarter q is dwords [p0 q, p0 (q + 1)), plane 1 (if any)
// [4 p0 + p1 q, 4 p0 + p1 (q + 1)).  v0 and v1 are the per-lane parts of
// the two planes' byte offsets (column and quarter); the uniform rest,
// 16 N P (plus 16 N p0 for plane 1), comes with the group.
struct QuarterOffsets {
    uint32_t v0, v1;
};
template <int B>
__device__ __forceinline__ QuarterOffsets quarter_offsets(uint32_t n16, int q, uint32_t N16) {
    using T = Width<B>;
    const uint32_t m0 = (uint32_t)(T::p0 * q), m1 = (uint32_t)(T::p1 * q);
    return {n16 + (m0 >> 2) * N16 + 4u * (m0 & 3u), n16 + (m1 >> 2) * N16 + 4u * (m1 & 3u)};
}

// The B dwords of one quarter: plane 0's then plane 1's.  soff = 16 N P.
template <int B>
__device__ __forceinline__ void load_quarter(__amdgpu_buffer_rsrc_t rw, const QuarterOffsets& o, uint32_t soff,
                                             uint32_t N16, uint32_t (&Q)[B]) {
    using T = Width<B>;
    if constexpr (T::p0 == 8) {
        load_dwords<4>(rw, o.v0, soff, Q);
        load_dwords<4>(rw, o.v0, soff + N16, Q + 4);
    } else {
        load_dwords<T::p0>(rw, o.v0, soff, Q);
    }
    if constexpr (T::p1 > 0) load_dwords<T::p1>(rw, o.v1, soff + (uint32_t)T::p0 * N16, Q + T::p0);
}

// All B words of one column of a group (one 1 KB wave load each): per-lane
// n16 = 16 n, uniform soff = 16 N P.
template <int B>
__device__ __forceinline__ void load_group_words(__amdgpu_buffer_rsrc_t rw, uint32_t n16, uint32_t soff,
                                                 uint32_t N16, uint32_t (&D)[4 * B]) {
#pragma unroll
    for (int j = 0; j < B; ++j) load_dwords<4>(rw, n16, soff + (uint32_t)j * N16, D + 4 * j);
}

struct DecodeCtx {
    int M, lane, q, n;
    float ref;                       // quantized scales: the column's range reference R / 256 (exact)
    float ref4[4];                   // the same for the four columns of a lane in the 16-row layout
    __amdgpu_buffer_rsrc_t rw, rs;   // weight and scale (or 4-bit scale code) buffers
    // The same buffers with no valid byte: every load through them returns
    // zeros without touching memory (the pipeline's steps past a run's end).
    __amdgpu_buffer_rsrc_t rw0, rs0;
    __amdgpu_buffer_rsrc_t rx;       // activations, M rows of K
};

// The group scale.  fp16 scales: the loaded value.  Quantized scales (QS):
// the loaded byte holds the column's 4-bit code q in its low (even column)
// or high (odd column) nibble, and s = fp16_RNE(fp32(t * fp32(1/(2^(b-1)-1))))
// with t = R (q+1)^2 / 256, exact in fp32; ref holds R / 256, so t is one
// exact product.
template <int B, bool QS>
__device__ __forceinline__ float group_scale(float ref, int n, uint16_t raw) {
    if constexpr (!QS) {
        return (float)__builtin_bit_cast(_Float16, raw);
    } else {
        // Two roundings, as specified: the fp32 product, then fp16.  The
        // empty asm (no side effects) hands the product over in a register;
        // without it the product and the conversion fuse into one
        // mixed-precision multiply (v_fma_mixlo_f16) that rounds once, to fp16.
        constexpr float inv = 1.0f / (float)((1 << (B - 1)) - 1);
        const int q1 = (int)((raw >> (4 * (n & 1))) & 15u) + 1;
        const float t = ref * (float)(q1 * q1);
        float u = t * inv;
        asm("" : "+v"(u));
        return (float)(_Float16)u;
    }
}

template <int TC> struct Tile {
    static constexpr int NQ = TC == 64 ? 4 : 1;     // K-quarters of a group per lane
    static constexpr int UNITS = 8 * NQ;            // decoder units per lane per group
    static constexpr int CBSZ = TC == 64 ? 4 : 2;   // 16 or 4 blocks share one activation block
};

// Activation operand of row block rb: the per-lane byte offset in x of the
// operand of group 0 (group g adds 256 g).  TC = 64: lane (a = l/4, i = l%4)
// holds x[4rb + i][128g + 8a .. +8).  TC = 16: lane (q, a = (l%16)/4, i)
// holds x[4rb + i][128g + 32q + 8a .. +8).  Rows past M repeat row M-1
// (unused).
template <int TC>
__device__ __forceinline__ uint32_t act_offset(const LinearDev& L, const DecodeCtx& c, int rb) {
    const int a = (TC == 64 ? c.lane : (c.lane & 15)) >> 2, i = c.lane & 3;
    const int row = min(4 * rb + i, c.M - 1);
    return 2u * ((uint32_t)row * (uint32_t)L.K + (TC == 64 ? 0u : 32u * (uint32_t)c.q) + 8u * (uint32_t)a);
}

// (c - z) * 2^-24 in both fp16 halves of a masked decoder-unit dword
// holding c * 2^(o-24) (o = p0 * t, the unit's bit offset in its half): one
// packed fp16 FMA, c * 2^(o-24) * 2^-o - z * 2^-24 (a packed add at o = 0).
// c << o and z << o stay below 2^10 for every width and offset, so every
// operand but the normal factor 2^-o, the exact product and the sum are
// fp16 subnormals (or zero) on the 2^-24 grid: the single rounding is
// exact, c = z gives +0, and units of every offset share one accumulator.
template <int B, int O>
__device__ __forceinline__ uint32_t unbias(uint32_t v) {
    static_assert(((1u << (B - 1)) << O) < 1024u, "zero point must stay subnormal");
    constexpr uint32_t zb = 0x8000u | (1u << (B - 1));
    const h2 bias = as_h2(zb | (zb << 16));
    if constexpr (O == 0) {
        return __builtin_bit_cast(uint32_t, as_h2(v) + bias);
    } else {
        constexpr _Float16 f = (_Float16)(1.0f / (float)(1u << O));
        const h2 fv = {f, f};
        return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(as_h2(v), fv, bias));
    }
}

template <int B, int MB, int TC, bool M1, bool QS>
__device__ __forceinline__ void group_compute(const DecodeCtx& c, const uint32_t (&Q)[B * Tile<TC>::NQ],
                                              const u4v (&X)[MB], uint16_t s16, float (&yacc)[MB][4]) {
    using TT = Tile<TC>;
    constexpr int C = Width<B>::per;
    f4 acc[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) acc[rb] = f4{0.f, 0.f, 0.f, 0.f};
    static_for<0, TT::UNITS>([&](auto UC) {
        constexpr int U = decltype(UC)::value;
        constexpr int O = Width<B>::p0 * (U % C);
        uint32_t b0, b1;
        unit_pair<B, U, TT::NQ>(Q, b0, b1);
        const h4 bv = as_h4(unbias<B, O>(b0), unbias<B, O>(b1));
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) {
            const h4 av = (U & 1) ? as_h4(X[rb][2], X[rb][3]) : as_h4(X[rb][0], X[rb][1]);
            acc[rb] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, bv, acc[rb], TT::CBSZ, U >> 1, 0);
        }
    });
    // The sums stay 2^-24 times too small until the wave's partials leave
    // (kUnit): scaling by a power of two commutes exactly with every step.
    const float s = group_scale<B, QS>(c.ref, c.n, s16);
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
#pragma unroll
        for (int r = 0; r < (M1 ? 1 : 4); ++r) {
            if (M1 || 4 * rb + r < c.M) yacc[rb][r] = __builtin_fmaf(s, acc[rb][r], yacc[rb][r]);
        }
    }
}

// Which compute layout a (row blocks, tile width) pair uses, and the shape
// of a lane's partial sums: [row block][row] for the 4x4x4 layout,
// [column block][row] for the 16-row layout.
template <int MB, int TC> struct Rows {
    static constexpr bool MMA = TC == 64 && MB >= 2;
    static constexpr int YB = MMA ? 4 : MB;
    // Waves per SIMD the launch bounds ask for: 4 (at most 128 VGPRs, two
    // 8-wave workgroups per CU) for the 16-row layout, whose two groups in
    // flight fit (measured 1.2x faster than one workgroup with deeper
    // pipelines), and for M <= 4, whose pipelines fit too; the 16-column
    // layout with more rows keeps its registers.
    static constexpr int WAVES_PER_EU = (MMA || MB == 1) ? 4 : 1;
};

// The 16-row layout (64-column tiles, M > 4).  Lane (j = l / 16, c = l % 16)
// decodes K-quarter j of columns c, c + 16, c + 32, c + 48: exactly the B
// operand of v_mfma_f32_16x16x32_f16 when MFMA k-slot 8j + t of K-step kk is
// code 32j + 8kk + t of the group (units 2kk and 2kk + 1 of quarter j).  The
// A operand is x in the same k order: lane (j, r) holds
// x[r][128g + 32j + 8kk .. +8].  Lane (j, c) ends with rows 4j .. 4j + 3 of
// its four columns.  Units 2kk and 2kk + 1 sit at different bit offsets;
// unbias brings both to (c - z) * 2^-24 while removing the zero point, so
// every MFMA of a column block adds to one sum.
template <int B, bool QS>
__device__ __forceinline__ void group_compute_mma(const DecodeCtx& c, const uint32_t (&Q)[4 * B], const u4v (&X)[4],
                                                  const uint16_t (&S)[4], float (&yacc)[4][4]) {
    using T = Width<B>;
    f4 acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = f4{0.f, 0.f, 0.f, 0.f};
    static_for<0, 4>([&](auto KC) {
        constexpr int kk = decltype(KC)::value;
        constexpr int O0 = T::p0 * ((2 * kk) % T::per);       // bit offsets of units 2kk and 2kk + 1
        constexpr int O1 = T::p0 * ((2 * kk + 1) % T::per);
        const h8 xop = __builtin_bit_cast(h8, X[kk]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            uint32_t a0, a1, b0, b1;
            unit_pair<B, 2 * kk, 1>(Q + cb * B, a0, a1);
            unit_pair<B, 2 * kk + 1, 1>(Q + cb * B, b0, b1);
            const h8 wop = __builtin_bit_cast(
                h8, u4v{unbias<B, O0>(a0), unbias<B, O0>(a1), unbias<B, O1>(b0), unbias<B, O1>(b1)});
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, wop, acc[cb], 0, 0, 0);
        }
    });
    // Sums 2^-24 times too small, as in group_compute.
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const float s = group_scale<B, QS>(c.ref4[cb], c.n + 16 * cb, S[cb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) yacc[cb][i] = __builtin_fmaf(s, acc[cb][i], yacc[cb][i]);
    }
}

// Steps K, K+1, .. of a run's last partial round while K < rem, nested so
// that each step is reached only from the one before it.  Guarded steps in
// sequence (or a round that may end early and then reach the loop's back
// edge) give the compiler's wait-count analysis paths, which the counts rule
// out, on which loads are still in flight at the top of the next round; it
// then drains every load there, every round.
template <int K, int N, class F>
__device__ __forceinline__ void tail_steps(int rem, F&& f) {
    if constexpr (K < N) {
        if (K < rem) {
            f(IC<K>{});
            tail_steps<K + 1, N>(rem, f);
        }
    }
}

// Empty volatile asm statements that take every element of r as input and
// output: work that reads r cannot start before them, work that writes r
// cannot end after them, and, having side effects, they keep their place
// among the loads of the pipeline.
template <class T, int N>
__device__ __forceinline__ void pin_regs(T (&r)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

template <int B, int TC, bool WIDE = false> struct Depth {
    // groups in flight per wave (the one being computed included); WIDE:
    // the high-occupancy plan kernel (8 waves per SIMD, 64 VGPRs)
    static constexpr int value = WIDE ? (B <= 4 ? 2 : 1)
                               : TC == 64 ? ((B <= 2) ? 4 : (B <= 4 ? 3 : 2)) : ((B <= 3) ? 6 : (B <= 6 ? 4 : 3));
};

// Plans at M <= 4 with at least this many workgroups per compute unit run
// the high-occupancy kernel: four 8-wave workgroups per CU with shallower
// pipelines instead of two with deeper ones.  On the 70B block (1312
// workgroups) it measured 5 % faster at M = 1 and M = 4; a single linear
// (fewer workgroups than CUs) took twice as long with it, its waves' own
// pipelines being all that hides the memory latency.  Plans of layers with
// quantized scales run it too: with the pipeline steps pinned it took 8
// such blocks from 59.7-60.0 to 56.7-57.5 us per block.
constexpr int kWideWgsPerCu = 4;

// Activation ring of the 16-row layout in decode and plan launches: two
// 4 KiB slots per wave, each one group's 16 rows x 128 activations.
constexpr int kXSlot = 4096;
constexpr int kXRing = 2 * kXSlot;

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// The 16-row layout's run with its activations staged in LDS.  Held in
// registers, a group's activations are 4 loads of 16 bytes per lane in the
// MFMA's operand order: each touches 32 cache lines for 1 KiB (row r's 16
// bytes at 64-byte strides), and the vector memory pipeline stalls on the L1
// cache.  Here 4 buffer loads with the LDS flag copy whole rows instead
// (8 cache lines per KiB): copy i, lane l moves row r = 4i + l/16 (rows past
// M repeat row M-1) and chunk (l % 16) ^ r of the group's 256 bytes to byte
// 16 l of the slot's KiB i, so chunk ch of row r sits at 256 r + 16 (ch ^ r)
// and the operand reads of 16 rows hit distinct banks.  Two groups in
// flight, as in registers: step s issues group s+1 (ring slot (s+1) mod 2)
// and waits until only those loads are in flight before reading group s.
// The copies write LDS behind the compiler's back, hence the explicit count
// and the scheduling barriers.
template <int B, bool QS>
__device__ __forceinline__ void run_width_mma_ring(const LinearDev& L, const DecodeCtx& c, const uint32_t* ord,
                                                   int cnt, float (&yacc)[4][4], char* ring) {
    using T = Width<B>;
    constexpr int STEP = 4 * ((T::p0 == 8 ? 2 : 1) + (T::p1 > 0 ? 1 : 0) + 1) + 4;   // loads a step issues
    static_assert(STEP < 64, "vmcnt range");
    uint32_t Q[2][4 * B];
    uint32_t S[2][4];   // fp16 scales (or scale-code bytes) in the low bits
    // Read-only for the kernel: a constant-space load stays scalar although
    // the copies count as memory writes.
    const __attribute__((address_space(4))) uint32_t* og = (const __attribute__((address_space(4))) uint32_t*)ord;
    const uint32_t N16 = 16u * (uint32_t)L.N;
    const QuarterOffsets qo = quarter_offsets<B>(16u * (uint32_t)c.n, c.q, N16);
    const uint32_t sv = QS ? (uint32_t)c.n >> 1 : 2u * (uint32_t)c.n;   // the lane's scale, column block 0
    uint32_t xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (c.lane >> 4);
        xv[i] = 2u * (uint32_t)min(r, c.M - 1) * (uint32_t)L.K + 16u * (uint32_t)((c.lane & 15) ^ r);
    }
    auto issue = [&](int step, uint32_t (&Qd)[4 * B], uint32_t (&Sd)[4], int slot) {
        const bool valid = step < cnt;
        const uint32_t e = og[min(step, cnt - 1)];
        const uint32_t g = e & 0xFFFFu, P = e >> 16;
        const __amdgpu_buffer_rsrc_t rw = valid ? c.rw : c.rw0, rs = valid ? c.rs : c.rs0;
        char* dst = ring + slot * kXSlot;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_ptr_t)(dst + 1024 * i), 16, (int)xv[i],
                                                     (int)(256u * g), 0, 0);
        // Column block cb: columns n + 16 cb, 256 cb bytes on in every word
        // row, 16 cb scales on.
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            load_quarter<B>(rw, qo, N16 * P + 256u * cb, N16, *reinterpret_cast<uint32_t(*)[B]>(Qd + cb * B));
            if constexpr (QS) Sd[cb] = __builtin_amdgcn_raw_buffer_load_b8(rs, sv, g * ((uint32_t)L.N >> 1) + 8u * cb, 0);
            else Sd[cb] = __builtin_amdgcn_raw_buffer_load_b16(rs, sv, 2u * g * (uint32_t)L.N + 32u * cb, 0);
        }
    };
    // Group in slot k once at most `wait` loads are in flight.
    auto compute = [&](auto KC, auto WC) {
        constexpr int k = decltype(KC)::value;
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(WC)::value));
        __builtin_amdgcn_sched_barrier(0);
        const int r = c.lane & 15;
        const char* src = ring + k * kXSlot + 256 * r;
        u4v X[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) X[kk] = *reinterpret_cast<const u4v*>(src + 16 * ((4 * c.q + kk) ^ r));
        const uint16_t s16[4] = {(uint16_t)S[k][0], (uint16_t)S[k][1], (uint16_t)S[k][2], (uint16_t)S[k][3]};
        group_compute_mma<B, QS>(c, Q[k], X, s16, yacc);
        __builtin_amdgcn_sched_barrier(0);
    };
    issue(0, Q[0], S[0], 0);
    int i = 0;
    for (; i + 2 <= cnt; i += 2) {
        static_for<0, 2>([&](auto KC) {
            constexpr int k = decltype(KC)::value;
            issue(i + k + 1, Q[(k + 1) % 2], S[(k + 1) % 2], (k + 1) % 2);
            compute(KC, IC<STEP>{});
        });
    }
    if (i < cnt) compute(IC<0>{}, IC<0>{});   // nothing was issued after the last group
}

// A run of `cnt` width-B groups (entries ord[0..cnt)), pipelined DEPTH deep:
// while group i is computed, groups i+1 .. i+DEPTH-1 are in flight.  Every
// step issues exactly one group's loads -- weights, scale, activation
// operands, in that order -- so each wait is a compile-time count.  Steps
// past the end of the run load through buffer descriptors of size zero:
// they keep the count fixed, return zeros and cost no memory traffic.  Only
// the uniform parts of the offsets change from group to group (scalar
// offsets); the per-lane parts are set once per run.
template <int B, int MB, int TC, bool M1, bool QS, bool XR, bool WIDE = false>
__device__ __forceinline__ void run_width(const LinearDev& L, const DecodeCtx& c, const uint32_t* ord, int cnt,
                                          float (&yacc)[Rows<MB, TC>::YB][4], char* ring) {
    constexpr bool MMA = Rows<MB, TC>::MMA;
    // Activation rings for widths up to 6 bits (4 with quantized scales,
    // whose kernels spill otherwise); 8-bit groups keep the register path.
    if constexpr (MMA && XR && B <= (QS ? 4 : 6)) {
        run_width_mma_ring<B, QS>(L, c, ord, cnt, yacc, ring);
        return;
    }
    static_assert(!WIDE || (!MMA && TC == 64), "the high-occupancy kernel is the 64-column 4x4x4 layout");
    constexpr int DEPTH = MMA ? 2 : Depth<B, TC, WIDE>::value;
    constexpr int NDW = MMA ? 4 * B : B * Tile<TC>::NQ;
    constexpr int NS = MMA ? 4 : 1;             // scales per lane and group
    constexpr int NX = MMA ? 4 : MB;            // activation operands per lane and group
    uint32_t Q[DEPTH][NDW];
    uint16_t S[DEPTH][NS];
    u4v X[DEPTH][NX];
    // Read-only for the kernel.  For M <= 4 a constant-space load keeps the
    // entries scalar beside the pinning asm statements (which count as memory
    // side effects); the 16-row layout keeps the global view, with which its
    // wide groups fit their registers.
    using OrdPtr = std::conditional_t<MMA, const EXQ_GLOBAL uint32_t*, const __attribute__((address_space(4))) uint32_t*>;
    const OrdPtr og = (OrdPtr)ord;
    const uint32_t N16 = 16u * (uint32_t)L.N;
    // Per-lane parts of every load's offset (the uniform parts come with the
    // group): weights, scale, activations.
    const QuarterOffsets qo = quarter_offsets<B>(16u * (uint32_t)c.n, c.q, N16);
    const uint32_t sv = QS ? (uint32_t)c.n >> 1 : 2u * (uint32_t)c.n;
    uint32_t xv[MMA ? 1 : MB];
    if constexpr (MMA) {
        // Lane (j, r) reads x[r][128g + 32j ..]; rows past M repeat row M-1 (unused).
        xv[0] = 2u * ((uint32_t)min(c.lane & 15, c.M - 1) * (uint32_t)L.K + 32u * (uint32_t)c.q);
    } else {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) xv[rb] = act_offset<TC>(L, c, rb);
    }
    auto issue = [&](int step, uint32_t (&Qd)[NDW], uint16_t (&Sd)[NS], u4v (&Xd)[NX]) {
        const bool valid = step < cnt;
        const uint32_t e = og[min(step, cnt - 1)];
        const uint32_t g = e & 0xFFFFu, P = e >> 16;
        const __amdgpu_buffer_rsrc_t rw = valid ? c.rw : c.rw0, rs = valid ? c.rs : c.rs0;
#pragma unroll
        for (int cb = 0; cb < NS; ++cb) {
            const uint32_t wo = N16 * P + 256u * cb;   // column block cb: columns n + 16 cb
            if constexpr (MMA) load_quarter<B>(rw, qo, wo, N16, *reinterpret_cast<uint32_t(*)[B]>(Qd + cb * B));
            else if constexpr (TC == 64) load_group_words<B>(rw, 16u * (uint32_t)c.n, wo, N16, Qd);
            else load_quarter<B>(rw, qo, wo, N16, Qd);
            if constexpr (QS) Sd[cb] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b8(rs, sv, g * ((uint32_t)L.N >> 1) + 8u * cb, 0);
            else Sd[cb] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, sv, 2u * g * (uint32_t)L.N + 32u * cb, 0);
        }
        if constexpr (MMA) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) Xd[kk] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, xv[0], 256u * g + 16u * kk, 0);
        } else {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) Xd[rb] = __builtin_amdgcn_raw_buffer_load_b128(c.rx, xv[rb], 256u * g, 0);
        }
    };
    static_for<0, DEPTH - 1>([&](auto KC) {
        constexpr int k = decltype(KC)::value;
        issue(k, Q[k], S[k], X[k]);
    });
    auto compute = [&](auto KC) {
        constexpr int k = decltype(KC)::value;
        if constexpr (!MMA) {
            pin_regs(Q[k]);
            pin_regs(X[k]);
        }
        if constexpr (MMA) group_compute_mma<B, QS>(c, Q[k], X[k], S[k], yacc);
        else group_compute<B, MB, TC, M1, QS>(c, Q[k], X[k], S[k][0], yacc);
        if constexpr (!MMA) {
#pragma unroll
            for (int rb = 0; rb < Rows<MB, TC>::YB; ++rb) pin_regs(yacc[rb]);
        }
    };
    if constexpr (MMA && B >= 5) {
        // The 16-row layout's wide groups (4b code dwords per group in
        // flight): guarded steps, and a round that ends the run leaves the
        // loop at once.  The structure below spills here; this one does not,
        // at the price of conservative waits inside a round.
        for (int i = 0; i < cnt; i += DEPTH) {
            bool done = false;
            static_for<0, DEPTH>([&](auto KC) {
                constexpr int k = decltype(KC)::value;
                constexpr int nk = (k + DEPTH - 1) % DEPTH;
                if (done || i + k >= cnt) {
                    done = true;
                    return;
                }
                issue(i + k + DEPTH - 1, Q[nk], S[nk], X[nk]);
                compute(KC);
            });
            if (done) break;
        }
        return;
    }
    // Whole rounds of DEPTH steps with no exit inside, then the last partial
    // round (see tail_steps).  Scheduling barriers close each step; for
    // M <= 4 the compute is also pinned between its inputs and its partial
    // sums (pin_regs).  Scheduling barriers alone do not hold arithmetic: the
    // compiler gathered a round's computes between its first and its other
    // issues, so the last group of every round waited for a load issued just
    // before it.
    int i = 0;
    for (; i + DEPTH <= cnt; i += DEPTH) {
        static_for<0, DEPTH>([&](auto KC) {
            constexpr int k = decltype(KC)::value;
            constexpr int nk = (k + DEPTH - 1) % DEPTH;
            issue(i + k + DEPTH - 1, Q[nk], S[nk], X[nk]);
            if constexpr (!MMA) __builtin_amdgcn_sched_barrier(0);
            compute(KC);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    // The last cnt - i < DEPTH groups are in flight already.
    tail_steps<0, DEPTH - 1>(cnt - i, compute);
}

// One decode tile: TC columns, all of K, kWaves waves.  No prologue: every
// wave starts streaming at once and only the final reduction is shared.
// decode_stream leaves each wave's partial sums in red (kWaves x M x TC
// fp32); after a workgroup barrier the waves are added in order.
// XR (16-row layout only): activations go through per-wave rings at xlds,
// memory that red reuses once every wave has finished its runs.
template <int MB, int TC, bool M1, bool QS, bool XR = false, bool WIDE = false>
__device__ __forceinline__ void decode_stream(const LinearDev& L, int tile, int M, float* red, char* xlds = nullptr) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    static_assert(!XR || Rows<MB, TC>::MMA, "activation rings belong to the 16-row layout");
    char* ring = XR ? xlds + wave * kXRing : nullptr;
    constexpr bool MMA = Rows<MB, TC>::MMA;
    constexpr int YB = Rows<MB, TC>::YB;
    DecodeCtx c;
    c.M = M;
    c.lane = lane;
    c.q = (TC == 64 && !MMA) ? 0 : lane >> 4;
    c.n = tile * TC + ((TC == 64 && !MMA) ? lane : (lane & 15));
    c.rw = buffer_rsrc(L.qweight, L.qbytes);
    c.rw0 = buffer_rsrc(L.qweight, 0);
    c.rx = buffer_rsrc(L.x, 2u * (uint32_t)M * (uint32_t)L.K);
    c.ref = 0.0f;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) c.ref4[cb] = 0.0f;
    if constexpr (QS) {
        c.rs = buffer_rsrc(L.qscale, L.qsbytes);
        c.rs0 = buffer_rsrc(L.qscale, 0);
        if constexpr (MMA) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                c.ref4[cb] = (float)__builtin_bit_cast(_Float16, gptr<uint16_t>(L.ref)[c.n + 16 * cb]) * 0.00390625f;
        } else {
            c.ref = (float)__builtin_bit_cast(_Float16, gptr<uint16_t>(L.ref)[c.n]) * 0.00390625f;
        }
    } else {
        c.rs = buffer_rsrc(L.scales, L.sbytes);
        c.rs0 = buffer_rsrc(L.scales, 0);
    }

    float yacc[YB][4];
#pragma unroll
    for (int rb = 0; rb < YB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[rb][r] = 0.f;
    {
        const uint32_t* ord = L.order + gptr<uint16_t>(L.bounds)[wave];
        const EXQ_GLOBAL uint16_t* cnt = gptr<uint16_t>(L.runs) + wave * kNumWidths;
        int k;
        if ((k = cnt[0]) > 0) { run_width<2, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); ord += k; }
        if ((k = cnt[1]) > 0) { run_width<3, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); ord += k; }
        if ((k = cnt[2]) > 0) { run_width<4, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); ord += k; }
        if ((k = cnt[3]) > 0) { run_width<5, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); ord += k; }
        if ((k = cnt[4]) > 0) { run_width<6, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); ord += k; }
        if ((k = cnt[5]) > 0) { run_width<8, MB, TC, M1, QS, XR, WIDE>(L, c, ord, k, yacc, ring); }
    }

    // 16-row layout: every (row, column) of the tile belongs to one lane.
    if constexpr (MMA) {
        if constexpr (XR) {
            // Every copy into the rings has landed and every wave has left
            // its runs before red overwrites them.
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * c.q + i;
                if (row < M) red[(wave * M + row) * TC + (lane & 15) + 16 * cb] = yacc[cb][i] * kUnit;
            }
        return;
    }
    // TC = 16: quarters ((q0 + q1) + (q2 + q3)) in every lane of a column.
    // Then waves, in order, through LDS.
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = yacc[rb][r] * kUnit;
            if constexpr (TC == 16) {
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
            }
            if (4 * rb + r < M && lane < TC) red[(wave * M + 4 * rb + r) * TC + lane] = v;
        }
}

// Output (m, col) of a tile: the wave partials added in wave order.
template <int TC>
__device__ __forceinline__ float tile_sum(const float* red, int M, int m, int col) {
    float v = red[(0 * M + m) * TC + col];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += red[(w * M + m) * TC + col];
    return v;
}

template <int MB, int TC, bool M1, bool QS, bool XR = false, bool WIDE = false>
__device__ __forceinline__ void decode_wg(const LinearDev& L, int tile, int M, float* red, char* xlds = nullptr) {
    decode_stream<MB, TC, M1, QS, XR, WIDE>(L, tile, M, red, xlds);
    __syncthreads();
    for (int t = threadIdx.x; t < M * TC; t += kWaves * 64) {
        const int m = t / TC, col = t % TC;
        *gptr_w<uint16_t>(L.y + (size_t)m * L.N + tile * TC + col) = f32_to_f16_bits(tile_sum<TC>(red, M, m, col));
    }
}

// SiLU(g) * u in fp32: g / (1 + e^-g) * u.  For g far below zero e^-g
// overflows to +inf and the product is a signed zero, the limit.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// A gate/up pair sharing x: every wave streams its share of the gate
// linear's groups, then the same share of the up linear's, into two sets of
// partials; the workgroup then writes h = SiLU(g) * u for its TC columns.
template <int MB, int TC, bool M1, bool QS>
__global__ __launch_bounds__(kWaves * 64, (Rows<MB, TC>::WAVES_PER_EU)) void gated_decode_kernel(LinearDev G, LinearDev U,
                                                                                        int M) {
    __shared__ float red[2][kWaves * 4 * MB * TC];
    decode_stream<MB, TC, M1, QS>(G, blockIdx.x, M, red[0]);
    decode_stream<MB, TC, M1, QS>(U, blockIdx.x, M, red[1]);
    __syncthreads();
    for (int t = threadIdx.x; t < M * TC; t += kWaves * 64) {
        const int m = t / TC, col = t % TC;
        const float g = tile_sum<TC>(red[0], M, m, col), u = tile_sum<TC>(red[1], M, m, col);
        *gptr_w<uint16_t>(G.y + (size_t)m * G.N + blockIdx.x * TC + col) = f32_to_f16_bits(silu_mul(g, u));
    }
}

// LDS of a decode workgroup: the wave partials and, in the 16-row layout,
// the activation rings, which the partials reuse.
template <int MB, int TC> struct DecodeLds {
    static constexpr int RED = kWaves * 4 * MB * TC * 4;
    static constexpr int BYTES = Rows<MB, TC>::MMA && kWaves * kXRing > RED ? kWaves * kXRing : RED;
};

template <int MB, int TC, bool M1, bool QS>
__global__ __launch_bounds__(kWaves * 64, (Rows<MB, TC>::WAVES_PER_EU)) void decode_kernel(LinearDev L, int M) {
    __shared__ __attribute__((aligned(16))) char lds[DecodeLds<MB, TC>::BYTES];
    decode_wg<MB, TC, M1, QS, Rows<MB, TC>::MMA>(L, blockIdx.x, M, reinterpret_cast<float*>(lds), lds);
}

template <int MB, bool M1, bool QS, bool WIDE>
__global__ __launch_bounds__(kWaves * 64, (WIDE ? 8 : Rows<MB, 64>::WAVES_PER_EU)) void decode_plan_kernel(const LinearDev* __restrict__ list,
                                                                   const uint32_t* __restrict__ wg_map, int M) {
    __shared__ __attribute__((aligned(16))) char lds[DecodeLds<MB, 64>::BYTES];
    const uint32_t e = gptr<uint32_t>(wg_map)[blockIdx.x];   // linear | tile << 16
    LinearDev L;
    {
        static_assert(sizeof(LinearDev) % 4 == 0, "descriptor copy");
        const EXQ_GLOBAL uint32_t* src = gptr<uint32_t>(list + (e & 0xFFFFu));
        uint32_t* dst = reinterpret_cast<uint32_t*>(&L);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(LinearDev) / 4); ++i)
            dst[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)src[i]);   // uniform: SGPRs
    }
    decode_wg<MB, 64, M1, QS, Rows<MB, 64>::MMA, WIDE>(L, (int)(e >> 16), M, reinterpret_cast<float*>(lds), lds);
}

// ------------------------------------------------- quantized scale expansion

// s[g][n] = fp16_RNE(fp32(t * fp32(1/(2^(b-1)-1)))), t = R[n] (q+1)^2 / 256 with
// q the 4-bit code of (g, n): the fp16 scales the prefill and dequant kernels
// read for a layer stored with quantized scales.  One thread per (g, n).
__global__ __launch_bounds__(256) void expand_qs_kernel(const uint8_t* __restrict__ qscale,
                                                        const uint16_t* __restrict__ ref,
                                                        const uint32_t* __restrict__ meta, int G, int N,
                                                        uint16_t* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)G * N) return;
    const int g = (int)(i / N), n = (int)(i % N);
    const int b = (int)(gptr<uint32_t>(meta)[g] & 15u);
    const float inv = b == 2 ? 1.0f / 1.0f : b == 3 ? 1.0f / 3.0f : b == 4 ? 1.0f / 7.0f
                    : b == 5 ? 1.0f / 15.0f : b == 6 ? 1.0f / 31.0f : 1.0f / 127.0f;
    const int q1 = (int)((gptr<uint8_t>(qscale)[(size_t)g * (N / 2) + n / 2] >> (4 * (n & 1))) & 15u) + 1;
    const float R = (float)__builtin_bit_cast(_Float16, gptr<uint16_t>(ref)[n]);
    const float t = R * (float)(q1 * q1) * 0.00390625f;
    float u = t * inv;
    asm("" : "+v"(u));   // the fp32 product, then fp16 (see group_scale)
    *gptr_w<uint16_t>(out + i) = __builtin_bit_cast(uint16_t, (_Float16)u);
}

// ------------------------------------------------ allocation-free scratch

// Device scratch of exq_gemm_noalloc: the fp16 expansion of a quantized-scale
// layer's group scales, remade by every call that needs it.  Each device the
// library runs on holds its own copy until the process ends.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// ---------------------------------------------------------------- dequant

// One lane per (column, quarter): decodes its 32 codes of group g and writes
// fp16_RNE((c - z) * s) to w_out[k][n].
template <int B>
__device__ __forceinline__ void dequant_quarter(const LinearDev& L, size_t P, int g, int n, int q,
                                                uint16_t* __restrict__ w_out) {
    uint32_t Q[B];
    const uint32_t N16 = 16u * (uint32_t)L.N;
    load_quarter<B>(buffer_rsrc(L.qweight, L.qbytes), quarter_offsets<B>(16u * (uint32_t)n, q, N16),
                    N16 * (uint32_t)P, N16, Q);
    const uint16_t s16 = *gptr<uint16_t>(L.scales + (size_t)g * L.N + n);
    const float s = (float)__builtin_bit_cast(_Float16, s16);
    constexpr int C = Width<B>::per;
    constexpr int z = 1 << (B - 1);
    static_for<0, 8>([&](auto UC) {
        constexpr int U = decltype(UC)::value;
        constexpr int o = Width<B>::p0 * (U % C);
        uint32_t b0, b1;
        unit_pair<B, U>(Q, b0, b1);
        const uint32_t cv[4] = {(b0 & 0xFFFFu) >> o, b0 >> (16 + o), (b1 & 0xFFFFu) >> o, b1 >> (16 + o)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // (c - z) * s is exact in fp32; one rounding to fp16.
            const float w = (float)((int)cv[e] - z) * s;
            const size_t k = (size_t)g * kGroup + 32 * q + 4 * U + e;
            *gptr_w<uint16_t>(w_out + k * L.N + n) = f32_to_f16_bits(w);
        }
    });
}

__global__ __launch_bounds__(64) void dequant_kernel(LinearDev L, uint16_t* __restrict__ w_out) {
    const int g = blockIdx.y;
    const int n = blockIdx.x * kTileCols + (threadIdx.x & 15);
    const int q = threadIdx.x >> 4;
    const uint32_t meta = gptr<uint32_t>(L.meta)[g];
    const size_t P = meta >> 4;
    switch (meta & 15u) {
        case 2: dequant_quarter<2>(L, P, g, n, q, w_out); break;
        case 3: dequant_quarter<3>(L, P, g, n, q, w_out); break;
        case 4: dequant_quarter<4>(L, P, g, n, q, w_out); break;
        case 5: dequant_quarter<5>(L, P, g, n, q, w_out); break;
        case 6: dequant_quarter<6>(L, P, g, n, q, w_out); break;
        default: dequant_quarter<8>(L, P, g, n, q, w_out); break;
    }
}

// ---------------------------------------------------------------- diagnostic

// Plain streaming read: workgroup w reads 16-byte words [w*chunk, (w+1)*chunk)
// of `a` (clipped to n16) with non-temporal loads, four in flight per lane,
// and stores the XOR of every 32-bit word it read to sink[w].  It has the
// decode kernel's access unit (a 1 KB wave load) and no arithmetic, so its
// rate is the read ceiling a weight-streaming kernel can reach.
__global__ __launch_bounds__(512) void stream_read_kernel(const u4v* __restrict__ a, size_t n16, size_t chunk,
                                                          uint32_t* __restrict__ sink) {
    const size_t begin = (size_t)blockIdx.x * chunk;
    const size_t end = begin < n16 ? (n16 - begin < chunk ? n16 : begin + chunk) : begin;
    const EXQ_GLOBAL u4v* g = gptr<u4v>(a);
    uint32_t acc = 0;
    size_t i = begin + threadIdx.x;
    for (; i + 3 * 512 < end; i += 4 * 512) {
        const u4v v0 = __builtin_nontemporal_load(g + i), v1 = __builtin_nontemporal_load(g + i + 512);
        const u4v v2 = __builtin_nontemporal_load(g + i + 1024), v3 = __builtin_nontemporal_load(g + i + 1536);
        acc ^= (v0[0] ^ v0[1] ^ v0[2] ^ v0[3]) ^ (v1[0] ^ v1[1] ^ v1[2] ^ v1[3]) ^
               (v2[0] ^ v2[1] ^ v2[2] ^ v2[3]) ^ (v3[0] ^ v3[1] ^ v3[2] ^ v3[3]);
    }
    for (; i < end; i += 512) {
        const u4v v = __builtin_nontemporal_load(g + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
    __shared__ uint32_t part[8];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) x ^= part[w];
        *gptr_w<uint32_t>(sink + blockIdx.x) = x;
    }
}

}  // namespace exq

// =================================================================== host

using namespace exq;


constexpr int kXcds = 8;                     // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr uint32_t kPlanEmpty = 0xFFFFFFFFu;  // prefill plan entry of a workgroup with no tile

struct exq_plan {
    int count = 0, M = 1, total_wgs = 0;
    bool prefill = false;   // M > 16: prefill tiles, else decode column tiles
    bool qs = false;        // decode plan of layers with quantized scales
    bool wide = false;      // decode plan at M <= 4 run by the high-occupancy kernel
    LinearDev* d_list = nullptr;
    uint32_t* d_wg_map = nullptr;
    uint32_t* d_part_map = nullptr;   // prefill: K-piece of each workgroup's tile
    float* d_ws = nullptr;            // prefill: partial sums of tiles cut along K
    uint32_t* d_counters = nullptr;   // prefill: arrivals at each cut tile (zero between launches)
};

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

exq_status hip_fail(hipError_t e, const char* what) {
    return fail(EXQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

LinearDev exq::linear_dev(const exq_layer* L, const void* x, void* y) {
    LinearDev d;
    d.qweight = static_cast<const uint8_t*>(L->qweight);
    d.scales = L->qs ? L->d_scales_own.load(std::memory_order_acquire) : static_cast<const uint16_t*>(L->scales);
    d.meta = L->d_meta;
    d.order = L->d_order;
    d.bounds = L->d_bounds;
    d.runs = L->d_runs;
    d.x = static_cast<const uint16_t*>(x);
    d.y = static_cast<uint16_t*>(y);
    d.K = L->K;
    d.N = L->N;
    d.G = L->G;
    d.tiles = L->N / kTileCols;
    size_t words = 0;
    for (int g = 0; g < L->G; ++g) words += L->widths[g];
    d.qbytes = (uint32_t)(16 * words * (size_t)L->N);
    d.sbytes = (uint32_t)(2 * (size_t)L->G * (size_t)L->N);
    d.qscale = static_cast<const uint8_t*>(L->qscale);
    d.ref = static_cast<const uint16_t*>(L->ref);
    d.qsbytes = L->qs ? (uint32_t)((size_t)L->G * (size_t)(L->N / 2)) : 0u;
    d.qs = L->qs ? 1 : 0;
    return d;
}

namespace {

// Tile width for a single-linear launch of m <= 16 rows: 64 columns when
// that still gives a workgroup per CU, or half that from 4 rows on (where the
// wider tile's shared activation loads pay for the emptier machine: measured
// 1.2x at 4 rows and 1.6x at 16 on 8192 columns); else 16.
// 64 columns for wide layers, and always above 4 rows (the 16-row MFMA layout).
// N not a multiple of 64: 16 always.
int tile_cols_for(int N, int m) {
    if (N % 64) return 16;
    return (m > 4 || N / 64 >= 256 || (m >= 4 && N / 64 >= 128)) ? 64 : 16;
}

template <int MB, int TC, bool M1>
void launch_decode_t(LinearDev d, int M, hipStream_t stream) {
    d.tiles = d.N / TC;
    if (d.qs) hipLaunchKernelGGL((decode_kernel<MB, TC, M1, true>), dim3(d.tiles), dim3(kWaves * 64), 0, stream, d, M);
    else hipLaunchKernelGGL((decode_kernel<MB, TC, M1, false>), dim3(d.tiles), dim3(kWaves * 64), 0, stream, d, M);
}

template <int TC>
void launch_decode_mb(const LinearDev& d, int M, hipStream_t stream) {
    switch ((M + 3) / 4) {
        case 1:
            if (M == 1) launch_decode_t<1, TC, true>(d, M, stream);
            else launch_decode_t<1, TC, false>(d, M, stream);
            break;
        case 2: launch_decode_t<2, TC, false>(d, M, stream); break;
        case 3: launch_decode_t<3, TC, false>(d, M, stream); break;
        default: launch_decode_t<4, TC, false>(d, M, stream); break;
    }
}

template <int MB, int TC, bool M1>
void launch_gated_t(LinearDev g, LinearDev u, int M, hipStream_t stream) {
    if (g.qs)
        hipLaunchKernelGGL((gated_decode_kernel<MB, TC, M1, true>), dim3(g.N / TC), dim3(kWaves * 64), 0, stream, g, u, M);
    else
        hipLaunchKernelGGL((gated_decode_kernel<MB, TC, M1, false>), dim3(g.N / TC), dim3(kWaves * 64), 0, stream, g, u,
                           M);
}

template <int TC>
void launch_gated_mb(const LinearDev& g, const LinearDev& u, int M, hipStream_t stream) {
    switch ((M + 3) / 4) {
        case 1:
            if (M == 1) launch_gated_t<1, TC, true>(g, u, M, stream);
            else launch_gated_t<1, TC, false>(g, u, M, stream);
            break;
        case 2: launch_gated_t<2, TC, false>(g, u, M, stream); break;
        case 3: launch_gated_t<3, TC, false>(g, u, M, stream); break;
        default: launch_gated_t<4, TC, false>(g, u, M, stream); break;
    }
}

exq_status launch_decode(const LinearDev& d, int M, hipStream_t stream) {
    if (tile_cols_for(d.N, M) == 64) launch_decode_mb<64>(d, M, stream);
    else launch_decode_mb<16>(d, M, stream);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "decode launch");
}

template <int MB, bool M1, bool WIDE>
void launch_plan_w(const exq_plan* P, hipStream_t s) {
    if (P->qs)
        hipLaunchKernelGGL((decode_plan_kernel<MB, M1, true, WIDE>), dim3(P->total_wgs), dim3(kWaves * 64), 0, s,
                           P->d_list, P->d_wg_map, P->M);
    else
        hipLaunchKernelGGL((decode_plan_kernel<MB, M1, false, WIDE>), dim3(P->total_wgs), dim3(kWaves * 64), 0, s,
                           P->d_list, P->d_wg_map, P->M);
}

template <int MB, bool M1>
void launch_plan_t(const exq_plan* P, hipStream_t s) {
    if constexpr (MB == 1) {
        if (P->wide) {
            launch_plan_w<1, M1, true>(P, s);
            return;
        }
    }
    launch_plan_w<MB, M1, false>(P, s);
}

void launch_plan(const exq_plan* P, hipStream_t s) {
    switch ((P->M + 3) / 4) {
        case 1:
            if (P->M == 1) launch_plan_t<1, true>(P, s);
            else launch_plan_t<1, false>(P, s);
            break;
        case 2: launch_plan_t<2, false>(P, s); break;
        case 3: launch_plan_t<3, false>(P, s); break;
        default: launch_plan_t<4, false>(P, s); break;
    }
}

}  // namespace

extern exq_status exq_prefill_launch(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream);
extern exq_status exq_prefill_launch_gated(const exq_layer* U, const void* x, int M, void* h, hipStream_t stream);
extern exq_status exq_prefill_launch_desc(const LinearDev& d, int M, hipStream_t stream);
extern int exq_prefill_tiles(const exq_layer* L, int M);
extern exq_status exq_prefill_plan_launch(const LinearDev* d_list, const uint32_t* d_wg_map, const uint32_t* d_part_map,
                                          float* d_ws, uint32_t* d_counters, int total_wgs, int M, hipStream_t stream);

// Decode kernel over consecutive slices of at most 16 rows of x (any M);
// tc = 0: the tile width of tile_cols_for, else 16 or 64.
// The device address of `scratch` on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept.  (The array's
// name in host code is a host-side stand-in, never a device address.)
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

exq_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(EXQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(EXQ_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess || !p)
                return fail(EXQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return EXQ_OK;
}

}  // namespace

exq_status exq_decode_rows(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream, int tc = 0) {
    for (int r0 = 0; r0 < M; r0 += kMaxDecodeM) {
        const int m = std::min(kMaxDecodeM, M - r0);
        const void* xs = static_cast<const uint16_t*>(x) + (size_t)r0 * L->K;
        void* ys = static_cast<uint16_t*>(y) + (size_t)r0 * L->N;
        const LinearDev d = linear_dev(L, xs, ys);
        if (tc == 0) {
            exq_status st = launch_decode(d, m, stream);
            if (st != EXQ_OK) return st;
        } else {
            if (tc == 64 && L->N % 64)
                return fail(EXQ_ERR_UNSUPPORTED, "64-column decode tiles need N %% 64 == 0 (N=%d)", L->N);
            if (tc == 64) launch_decode_mb<64>(d, m, stream);
            else launch_decode_mb<16>(d, m, stream);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e, "decode launch");
        }
    }
    return EXQ_OK;
}

// The fp16 scales the prefill and dequant kernels read.  A layer with
// quantized scales makes them on the first call that needs them: allocated,
// filled on `stream` and waited for before the pointer is published, so
// calls on other streams never see a partial table.
exq_status ensure_scales(exq_layer* L, hipStream_t stream) {
    if (!L->qs || L->d_scales_own.load(std::memory_order_acquire)) return EXQ_OK;
    std::lock_guard<std::mutex> lock(L->expand_mu);
    if (L->d_scales_own.load(std::memory_order_acquire)) return EXQ_OK;
    const size_t n = (size_t)L->G * L->N;
    uint16_t* d = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&d, 2 * n)) != hipSuccess) return fail(EXQ_ERR_OOM, "hipMalloc expanded scales");
    hipLaunchKernelGGL(expand_qs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(L->qscale), static_cast<const uint16_t*>(L->ref), L->d_meta, L->G,
                       L->N, d);
    if ((e = hipGetLastError()) != hipSuccess || (e = hipStreamSynchronize(stream)) != hipSuccess) {
        (void)hipFree(d);
        return hip_fail(e, "expanding the quantized scales");
    }
    L->d_scales_own.store(d, std::memory_order_release);
    return EXQ_OK;
}

namespace {

// exq_gemm with a given kernel choice (kVarDefault: M <= kTuneMaxM decode in
// 16-row slices with the tile_cols_for width, else prefill: a 256-row prefill
// tile mostly empty is slower than a few decode slices, measured 3x at 32
// rows on every 70B shape).
exq_status prefill_with_scales(exq_layer* L, const void* x, int M, void* y, hipStream_t s) {
    exq_status st = ensure_scales(L, s);
    return st != EXQ_OK ? st : exq_prefill_launch(L, x, M, y, s);
}

exq_status run_variant(exq_layer* L, const void* x, int M, void* y, hipStream_t s, int v) {
    switch (v) {
        case kVarDecode16: return exq_decode_rows(L, x, M, y, s, 16);
        case kVarDecode64: return exq_decode_rows(L, x, M, y, s, 64);
        case kVarPrefill: return prefill_with_scales(L, x, M, y, s);
        default: return M > kTuneMaxM ? prefill_with_scales(L, x, M, y, s) : exq_decode_rows(L, x, M, y, s);
    }
}

}  // namespace

extern "C" {

// Shared by exq_layer_create (d_scales given) and exq_layer_create_qs
// (d_qscale and d_ref given; the fp16 expansion is allocated and filled here).
static exq_status layer_create(int K, int N, int group_size, const uint8_t* widths_host, const void* d_qweight,
                               const void* d_scales, const void* d_qscale, const void* d_ref, exq_layer_t* out) {
    if (!out) return fail(EXQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    exq_status st = check_layer_shape(K, N, group_size, widths_host);
    if (st != EXQ_OK) return st;
    if (N % 16) return fail(EXQ_ERR_INVALID_ARG, "N=%d is not a multiple of 16", N);
    const bool qs = d_scales == nullptr;
    if (!d_qweight || (!qs && !d_scales) || (qs && (!d_qscale || !d_ref)))
        return fail(EXQ_ERR_INVALID_ARG, "NULL device buffer");
    if (!aligned16(d_qweight) || (!qs && !aligned16(d_scales)) || (qs && (!aligned16(d_qscale) || !aligned16(d_ref))))
        return fail(EXQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    const int G = K / kGroup;
    {
        size_t words = 0;
        for (int g = 0; g < G; ++g) words += widths_host[g];
        if (words >= 65536 || G >= 65536)
            return fail(EXQ_ERR_UNSUPPORTED, "K=%d is too large for 16-bit per-column word offsets", K);
        if (16 * words * (size_t)N >= kBufOOB)
            return fail(EXQ_ERR_UNSUPPORTED, "packed layer of %zu bytes exceeds the 2 GiB per-layer limit",
                        16 * words * (size_t)N);
    }
    exq_layer* L = new (std::nothrow) exq_layer();
    if (!L) return fail(EXQ_ERR_OOM, "host allocation");
    L->K = K;
    L->N = N;
    L->G = G;
    L->widths.assign(widths_host, widths_host + G);
    L->qweight = d_qweight;
    L->scales = d_scales;
    L->qs = qs;
    L->qscale = d_qscale;
    L->ref = d_ref;
    L->plan = plan_waves(K, widths_host);
    std::vector<uint32_t> meta = group_meta(K, widths_host);
    hipError_t e = hipSuccess;
    auto cleanup = [&](exq_status s) { exq_layer_destroy(L); return s; };
    if ((e = hipMalloc(&L->d_meta, sizeof(uint32_t) * G)) != hipSuccess ||
        (e = hipMalloc(&L->d_order, sizeof(uint32_t) * G)) != hipSuccess ||
        (e = hipMalloc(&L->d_bounds, sizeof(uint16_t) * L->plan.bounds.size())) != hipSuccess ||
        (e = hipMalloc(&L->d_runs, sizeof(uint16_t) * L->plan.runs.size())) != hipSuccess)
        return cleanup(fail(EXQ_ERR_OOM, "hipMalloc layer metadata"));
    if ((e = hipMemcpy(L->d_meta, meta.data(), sizeof(uint32_t) * G, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(L->d_order, L->plan.order.data(), sizeof(uint32_t) * G, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(L->d_bounds, L->plan.bounds.data(), sizeof(uint16_t) * L->plan.bounds.size(),
                       hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(L->d_runs, L->plan.runs.data(), sizeof(uint16_t) * L->plan.runs.size(),
                       hipMemcpyHostToDevice)) != hipSuccess)
        return cleanup(hip_fail(e, "hipMemcpy layer metadata"));
    *out = L;
    return EXQ_OK;
}

exq_status exq_layer_create(int K, int N, int group_size, const uint8_t* widths_host, const void* d_qweight,
                            const void* d_scales, exq_layer_t* out) {
    if (!d_scales) {
        if (out) *out = nullptr;
        return fail(EXQ_ERR_INVALID_ARG, "NULL device buffer");
    }
    return layer_create(K, N, group_size, widths_host, d_qweight, d_scales, nullptr, nullptr, out);
}

exq_status exq_layer_create_qs(int K, int N, int group_size, const uint8_t* widths_host, const void* d_qweight,
                               const void* d_qscale, const void* d_ref, exq_layer_t* out) {
    if (!d_qscale || !d_ref) {
        if (out) *out = nullptr;
        return fail(EXQ_ERR_INVALID_ARG, "NULL device buffer");
    }
    return layer_create(K, N, group_size, widths_host, d_qweight, nullptr, d_qscale, d_ref, out);
}

void exq_layer_destroy(exq_layer_t L) {
    if (!L) return;
    if (L->d_meta) (void)hipFree(L->d_meta);
    if (L->d_order) (void)hipFree(L->d_order);
    if (L->d_bounds) (void)hipFree(L->d_bounds);
    if (L->d_runs) (void)hipFree(L->d_runs);
    if (uint16_t* s = L->d_scales_own.load()) (void)hipFree(s);
    delete L;
}

exq_status exq_gemm(const void* x, int M, exq_layer_t L, void* y, void* stream) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!x || !y) return fail(EXQ_ERR_INVALID_ARG, "NULL x or y");
    if (M < 1) return fail(EXQ_ERR_INVALID_ARG, "M=%d must be >= 1", M);
    if (!aligned16(x) || !aligned16(y)) return fail(EXQ_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (overlap(x, 2 * (size_t)M * L->K, y, 2 * (size_t)M * L->N)) return fail(EXQ_ERR_INVALID_ARG, "y overlaps x");
    const int v = M <= kTuneMaxM ? L->tuned[M].load(std::memory_order_relaxed) : kVarDefault;
    return run_variant(L, x, M, y, static_cast<hipStream_t>(stream), v);
}

exq_status exq_gemm_noalloc(const void* x, int M, exq_layer_t L, void* y, void* stream) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!x || !y) return fail(EXQ_ERR_INVALID_ARG, "NULL x or y");
    if (M < 1) return fail(EXQ_ERR_INVALID_ARG, "M=%d must be >= 1", M);
    if (!aligned16(x) || !aligned16(y)) return fail(EXQ_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (overlap(x, 2 * (size_t)M * L->K, y, 2 * (size_t)M * L->N)) return fail(EXQ_ERR_INVALID_ARG, "y overlaps x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int v = M <= kTuneMaxM ? L->tuned[M].load(std::memory_order_relaxed) : kVarDefault;
    const bool prefill = v == kVarPrefill || (v == kVarDefault && M > kTuneMaxM);
    // Decode kernels read the 4-bit codes or the fp16 scales, and fp16-scale
    // layers need nothing more: those launches allocate nothing already.
    if (!prefill || !L->qs) return run_variant(L, x, M, y, s, v);
    const size_t need = 2 * (size_t)L->G * (size_t)L->N;
    if (need > kScratchBytes)
        return fail(EXQ_ERR_UNSUPPORTED, "the fp16 scales of this layer (%zu bytes) exceed the %zu-byte scratch", need,
                    kScratchBytes);
    void* scr = nullptr;
    exq_status st = scratch_address(&scr);
    if (st != EXQ_OK) return st;
    const size_t n = (size_t)L->G * L->N;
    hipLaunchKernelGGL(expand_qs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t*>(L->qscale), static_cast<const uint16_t*>(L->ref), L->d_meta, L->G,
                       L->N, static_cast<uint16_t*>(scr));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scale expansion launch");
    LinearDev d = linear_dev(L, x, y);
    d.scales = static_cast<const uint16_t*>(scr);
    return exq_prefill_launch_desc(d, M, s);
}

exq_status exq_set_variant(exq_layer_t L, int M, int variant) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (M < 1 || M > kTuneMaxM) return fail(EXQ_ERR_INVALID_ARG, "M=%d outside 1..%d", M, kTuneMaxM);
    if (variant < 0 || variant >= kNumVariants) return fail(EXQ_ERR_INVALID_ARG, "variant %d", variant);
    if (variant == kVarPrefill && M <= kMaxDecodeM)
        return fail(EXQ_ERR_INVALID_ARG, "the prefill kernel serves M > %d", kMaxDecodeM);
    if (variant == kVarDecode64 && L->N % 64)
        return fail(EXQ_ERR_UNSUPPORTED, "64-column decode tiles need N %% 64 == 0 (N=%d)", L->N);
    L->tuned[M].store((uint8_t)variant, std::memory_order_relaxed);
    return EXQ_OK;
}

exq_status exq_autotune(const void* x, int M, exq_layer_t L, void* y, void* stream, int warmup, int reps,
                        int* choice_out, float* times_us_out) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!x || !y) return fail(EXQ_ERR_INVALID_ARG, "NULL x or y");
    if (M < 1 || M > kTuneMaxM) return fail(EXQ_ERR_INVALID_ARG, "M=%d outside 1..%d", M, kTuneMaxM);
    if (warmup < 0 || reps < 1 || reps > 100000) return fail(EXQ_ERR_INVALID_ARG, "warmup=%d reps=%d", warmup, reps);
    if (!aligned16(x) || !aligned16(y)) return fail(EXQ_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (overlap(x, 2 * (size_t)M * L->K, y, 2 * (size_t)M * L->N)) return fail(EXQ_ERR_INVALID_ARG, "y overlaps x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<hipEvent_t> ev(2 * (size_t)reps, nullptr);
    hipError_t e = hipSuccess;
    for (auto& v : ev)
        if ((e = hipEventCreate(&v)) != hipSuccess) break;
    auto release = [&]() {
        for (auto& v : ev)
            if (v) (void)hipEventDestroy(v);
    };
    if (e != hipSuccess) {
        release();
        return hip_fail(e, "hipEventCreate");
    }
    const int first = kVarDecode16, last = M > kMaxDecodeM ? kVarPrefill : kVarDecode64;
    std::vector<float> samples(reps);
    int best = kVarDefault;
    double best_t = 0.0;
    for (int v = first; v <= last; ++v) {
        if (v == kVarDecode64 && L->N % 64) {   // not served: no time
            if (times_us_out) times_us_out[v - first] = -1.0f;
            continue;
        }
        exq_status st = EXQ_OK;
        for (int i = 0; i < warmup && st == EXQ_OK; ++i) st = run_variant(L, x, M, y, s, v);
        for (int i = 0; i < reps && st == EXQ_OK; ++i) {
            (void)hipEventRecord(ev[2 * i], s);
            st = run_variant(L, x, M, y, s, v);
            (void)hipEventRecord(ev[2 * i + 1], s);
        }
        if (st != EXQ_OK) {
            (void)hipStreamSynchronize(s);
            release();
            return st;
        }
        if ((e = hipEventSynchronize(ev[2 * reps - 1])) != hipSuccess) {
            release();
            return hip_fail(e, "hipEventSynchronize");
        }
        for (int i = 0; i < reps; ++i)
            if ((e = hipEventElapsedTime(&samples[i], ev[2 * i], ev[2 * i + 1])) != hipSuccess) {
                release();
                return hip_fail(e, "hipEventElapsedTime");
            }
        const double t = exq_trimmed_mean(samples.data(), reps) * 1e3;   // microseconds
        if (times_us_out) times_us_out[v - first] = (float)t;
        if (best == kVarDefault || t < best_t) {
            best = v;
            best_t = t;
        }
    }
    release();
    L->tuned[M].store((uint8_t)best, std::memory_order_relaxed);
    if (choice_out) *choice_out = best;
    // Leave y holding the chosen kernel's result.
    return run_variant(L, x, M, y, s, best);
}

exq_status exq_gemm_gated(const void* x, int M, exq_layer_t gate, exq_layer_t up, void* h, void* stream) {
    if (!gate || !up) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!x || !h) return fail(EXQ_ERR_INVALID_ARG, "NULL x or h");
    if (M < 1) return fail(EXQ_ERR_INVALID_ARG, "M=%d must be >= 1", M);
    if (gate->K != up->K || gate->N != up->N)
        return fail(EXQ_ERR_INVALID_ARG, "gate (K=%d, N=%d) and up (K=%d, N=%d) differ in shape", gate->K, gate->N,
                    up->K, up->N);
    if (gate->qs != up->qs) return fail(EXQ_ERR_INVALID_ARG, "gate and up differ in scale storage");
    if (!aligned16(x) || !aligned16(h)) return fail(EXQ_ERR_INVALID_ARG, "x and h must be 16-byte aligned");
    if (overlap(x, 2 * (size_t)M * gate->K, h, 2 * (size_t)M * gate->N))
        return fail(EXQ_ERR_INVALID_ARG, "h overlaps x");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M > kTuneMaxM) {
        // Gate product into h, then the up product's epilogue combines in place.
        exq_status st = ensure_scales(gate, s);
        if (st == EXQ_OK) st = ensure_scales(up, s);
        if (st == EXQ_OK) st = exq_prefill_launch(gate, x, M, h, s);
        return st != EXQ_OK ? st : exq_prefill_launch_gated(up, x, M, h, s);
    }
    // Decode in 16-row slices; the tile width follows exq_gemm's rule.  (16-
    // column tiles for the 28672-column feed-forward pair, which fills only 448
    // of the 512 slots with 64-column tiles, measured twice as slow.)
    for (int r0 = 0; r0 < M; r0 += kMaxDecodeM) {
        const int m = std::min(kMaxDecodeM, M - r0);
        const void* xs = static_cast<const uint16_t*>(x) + (size_t)r0 * gate->K;
        void* hs = static_cast<uint16_t*>(h) + (size_t)r0 * gate->N;
        const LinearDev g = linear_dev(gate, xs, hs), u = linear_dev(up, xs, nullptr);
        if (tile_cols_for(gate->N, m) == 64) launch_gated_mb<64>(g, u, m, s);
        else launch_gated_mb<16>(g, u, m, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "gated decode launch");
    }
    return EXQ_OK;
}

exq_status exq_dequant(exq_layer_t L, void* w_out, void* stream) {
    if (!L) return fail(EXQ_ERR_INVALID_ARG, "layer is NULL");
    if (!w_out) return fail(EXQ_ERR_INVALID_ARG, "w_out is NULL");
    if (!aligned16(w_out)) return fail(EXQ_ERR_INVALID_ARG, "w_out must be 16-byte aligned");
    exq_status st = ensure_scales(L, static_cast<hipStream_t>(stream));
    if (st != EXQ_OK) return st;
    LinearDev d = linear_dev(L, nullptr, nullptr);
    hipLaunchKernelGGL(dequant_kernel, dim3(L->N / kTileCols, L->G), dim3(64), 0, static_cast<hipStream_t>(stream), d,
                       static_cast<uint16_t*>(w_out));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "dequant launch");
}

exq_status exq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words, void* stream) {
    if (!buf || !sink) return fail(EXQ_ERR_INVALID_ARG, "NULL buffer");
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return fail(EXQ_ERR_INVALID_ARG, "buf must be 16-byte and sink 4-byte aligned");
    if (bytes == 0 || bytes % 16) return fail(EXQ_ERR_INVALID_ARG, "bytes=%zu is not a positive multiple of 16", bytes);
    if (sink_words < 1 || sink_words > (1 << 20)) return fail(EXQ_ERR_INVALID_ARG, "sink_words=%d not in [1, 2^20]", sink_words);
    const size_t n16 = bytes / 16, chunk = (n16 + sink_words - 1) / sink_words;
    hipLaunchKernelGGL(stream_read_kernel, dim3(sink_words), dim3(512), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u4v*>(buf), n16, chunk, sink);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "stream read launch");
}

exq_status exq_plan_create(int count, const exq_layer_t* layers, const void* const* xs, const void* const* ys, int M,
                           exq_plan_t* out) {
    if (!out) return fail(EXQ_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (count < 1 || !layers || !xs || !ys) return fail(EXQ_ERR_INVALID_ARG, "empty or NULL plan arrays");
    if (M < 1) return fail(EXQ_ERR_INVALID_ARG, "plan M=%d must be >= 1", M);
    const bool prefill = M > kMaxDecodeM;
    if (count > 65535) return fail(EXQ_ERR_UNSUPPORTED, "plan of %d linears (at most 65535)", count);
    for (int i = 0; i < count; ++i)
        if (!layers[i] || !xs[i] || !ys[i]) return fail(EXQ_ERR_INVALID_ARG, "plan entry %d is NULL", i);
    std::vector<LinearDev> list(count);
    std::vector<int> work(count);
    long total_tiles = 0;
    for (int i = 0; i < count; ++i) {
        const exq_layer* L = layers[i];
        if (!aligned16(xs[i]) || !aligned16(ys[i])) return fail(EXQ_ERR_INVALID_ARG, "plan entry %d misaligned", i);
        for (int j = 0; j < count; ++j) {
            if (overlap(ys[i], 2 * (size_t)M * L->N, xs[j], 2 * (size_t)M * layers[j]->K))
                return fail(EXQ_ERR_INVALID_ARG, "output %d overlaps input %d", i, j);
            if (j != i && overlap(ys[i], 2 * (size_t)M * L->N, ys[j], 2 * (size_t)M * layers[j]->N))
                return fail(EXQ_ERR_INVALID_ARG, "outputs %d and %d overlap", i, j);
        }
        if (!prefill && L->qs != layers[0]->qs)
            return fail(EXQ_ERR_INVALID_ARG, "a decode plan needs one scale storage for all linears (entry %d differs)", i);
        if (prefill) {
            if (exq_prefill_tiles(L, M) == 0)
                return fail(EXQ_ERR_UNSUPPORTED, "entry %d: K or M too large for a prefill plan", i);
        } else if (L->N % 64) {
            return fail(EXQ_ERR_UNSUPPORTED, "entry %d: decode plans use 64-column tiles, N=%d", i, L->N);
        } else if (L->N / 64 >= 65536) {
            return fail(EXQ_ERR_UNSUPPORTED, "entry %d has too many tiles", i);
        }
        total_tiles += prefill ? exq_prefill_tiles(L, M) : L->N / 64;
    }
    // A prefill map is padded to 8 equal XCD queues: at most 8x the tiles.
    if (total_tiles > (long)(INT32_MAX / kXcds)) return fail(EXQ_ERR_UNSUPPORTED, "plan too large");
    // Every argument is valid: only now expand quantized scales (a prefill
    // plan's kernels read fp16 scales), so a failed call launches nothing.
    for (int i = 0; i < count && prefill; ++i) {
        exq_status st = ensure_scales(layers[i], nullptr);
        if (st != EXQ_OK) return st;
    }
    for (int i = 0; i < count; ++i) {
        const exq_layer* L = layers[i];
        list[i] = linear_dev(L, xs[i], const_cast<void*>(ys[i]));
        if (prefill) {
            list[i].tiles = exq_prefill_tiles(L, M);
            work[i] = L->K;   // per-workgroup cost: one tile over all of K
        } else {
            list[i].tiles = L->N / 64;
            int words = 0;
            for (int g = 0; g < L->G; ++g) words += L->widths[g];
            work[i] = words + L->G;   // per-workgroup cost, as in the wave plan
        }
    }
    // Longest workgroups first, so the launch does not end on a tail of
    // long-K tiles; within a linear, tiles in order.
    std::vector<int> byw(count);
    for (int i = 0; i < count; ++i) byw[i] = i;
    std::stable_sort(byw.begin(), byw.end(), [&](int a, int b) { return work[a] > work[b]; });
    std::vector<uint32_t> wg_map, part_map;
    uint32_t split_slots = 0;
    if (!prefill) {
        for (int i : byw)
            for (int t = 0; t < list[i].tiles; ++t) wg_map.push_back((uint32_t)i | ((uint32_t)t << 16));
    } else {
        // Workgroup ids are dispatched to the 8 XCDs round-robin (id % 8).  Each
        // block of a linear's tiles (xcd_block: 2 row groups x 4 column
        // groups) goes, whole, to the least-loaded XCD with its rows varying
        // fastest, so the tiles running together on an XCD share a column tile
        // of W and the row tiles of x through its L2.  W is then fetched about
        // twice and x four times instead of W eight times (one row tile per
        // XCD): 21 % less HBM traffic on the 70B block at M = 2048, at the same
        // speed.  Entry i is the next tile queued for XCD i % 8; short queues
        // are padded with empty entries (kPlanEmpty: the workgroup exits).
        std::vector<std::vector<uint32_t>> queue(kXcds);
        std::vector<long> load(kXcds, 0);
        for (int i : byw) {
            const int col_tiles = (layers[i]->N + 255) / 256, row_tiles = list[i].tiles / col_tiles;
            for (int blk = 0; blk < kXcds; ++blk) {
                const XcdBlock b = xcd_block(row_tiles, col_tiles, blk);
                if (b.nr == 0 || b.nc == 0) continue;
                const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
                for (int ct = b.c0; ct < b.c0 + b.nc; ++ct)
                    for (int r = b.r0; r < b.r0 + b.nr; ++r)
                        queue[x].push_back((uint32_t)i | ((uint32_t)(r * col_tiles + ct) << 16));
                load[x] += (long)b.nr * b.nc * work[i];
            }
        }
        // An XCD runs its queue on its compute units (one prefill workgroup
        // each), in order.  When the tiles after its first round do not fill
        // the last round, the tiles of that partial round are cut along K
        // into up to kPlanParts pieces, so the pieces fill it.  (Measured on
        // the 70B block at M = 2048: each XCD ran 32 long tiles, then 9
        // rounds of 32 short ones and a last round of 8.)
        int dev = 0, cus = 0;
        hipError_t e;
        if ((e = hipGetDevice(&dev)) != hipSuccess ||
            (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return hip_fail(e, "compute unit count");
        const int per_xcd = std::max(1, cus / kXcds);
        std::vector<std::vector<uint32_t>> parts(kXcds);
        for (int x = 0; x < kXcds; ++x) {
            const int n = (int)queue[x].size();
            const int r = n > per_xcd ? (n - per_xcd) % per_xcd : 0;
            const int np = r > 0 ? std::min(kPlanParts, per_xcd / r) : 1;
            std::vector<uint32_t> q2, p2;
            for (int k = 0; k < n; ++k) {
                const uint32_t ent = queue[x][k];
                const int G = layers[ent & 0xFFFFu]->G;
                const int pieces = (k >= n - r && np > 1 && G >= np) ? np : 1;
                const uint32_t slot = pieces > 1 ? split_slots++ : 0u;
                for (int pc = 0; pc < pieces; ++pc) {
                    q2.push_back(ent);
                    p2.push_back((uint32_t)pc | ((uint32_t)pieces << 4) | (slot << 8));
                }
            }
            queue[x].swap(q2);
            parts[x].swap(p2);
        }
        size_t longest = 0;
        for (const auto& q : queue) longest = std::max(longest, q.size());
        for (size_t k = 0; k < longest; ++k)
            for (int x = 0; x < kXcds; ++x) {
                wg_map.push_back(k < queue[x].size() ? queue[x][k] : kPlanEmpty);
                part_map.push_back(k < queue[x].size() ? parts[x][k] : 1u << 4);
            }
    }
    exq_plan* P = new (std::nothrow) exq_plan();
    if (!P) return fail(EXQ_ERR_OOM, "host allocation");
    P->count = count;
    P->M = M;
    P->prefill = prefill;
    P->qs = !prefill && layers[0]->qs;
    P->total_wgs = (int)wg_map.size();
    hipError_t e;
    if (!prefill && M <= 4) {
        int dev = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess ||
            (e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) {
            exq_plan_destroy(P);
            return hip_fail(e, "compute unit count");
        }
        P->wide = P->total_wgs >= kWideWgsPerCu * cus;
    }
    if ((e = hipMalloc(&P->d_list, sizeof(LinearDev) * count)) != hipSuccess ||
        (e = hipMalloc(&P->d_wg_map, sizeof(uint32_t) * wg_map.size())) != hipSuccess) {
        exq_plan_destroy(P);
        return fail(EXQ_ERR_OOM, "hipMalloc plan");
    }
    if ((e = hipMemcpy(P->d_list, list.data(), sizeof(LinearDev) * count, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(P->d_wg_map, wg_map.data(), sizeof(uint32_t) * wg_map.size(), hipMemcpyHostToDevice)) !=
            hipSuccess) {
        exq_plan_destroy(P);
        return hip_fail(e, "hipMemcpy plan");
    }
    if (prefill) {
        const size_t ws_floats = (size_t)std::max<uint32_t>(split_slots, 1) * kPlanParts * 256 * 256;
        const size_t ncnt = std::max<uint32_t>(split_slots, 1);
        if ((e = hipMalloc(&P->d_part_map, sizeof(uint32_t) * part_map.size())) != hipSuccess ||
            (e = hipMalloc(&P->d_ws, sizeof(float) * ws_floats)) != hipSuccess ||
            (e = hipMalloc(&P->d_counters, sizeof(uint32_t) * ncnt)) != hipSuccess) {
            exq_plan_destroy(P);
            return fail(EXQ_ERR_OOM, "hipMalloc plan");
        }
        if ((e = hipMemcpy(P->d_part_map, part_map.data(), sizeof(uint32_t) * part_map.size(),
                           hipMemcpyHostToDevice)) != hipSuccess ||
            (e = hipMemset(P->d_counters, 0, sizeof(uint32_t) * ncnt)) != hipSuccess ||
            (e = hipDeviceSynchronize()) != hipSuccess) {
            exq_plan_destroy(P);
            return hip_fail(e, "hipMemcpy plan");
        }
    }
    *out = P;
    return EXQ_OK;
}

exq_status exq_plan_run(exq_plan_t P, void* stream) {
    if (!P) return fail(EXQ_ERR_INVALID_ARG, "plan is NULL");
    if (P->prefill)
        return exq_prefill_plan_launch(P->d_list, P->d_wg_map, P->d_part_map, P->d_ws, P->d_counters, P->total_wgs, P->M,
                                       static_cast<hipStream_t>(stream));
    launch_plan(P, static_cast<hipStream_t>(stream));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : hip_fail(e, "plan launch");
}

void exq_plan_destroy(exq_plan_t P) {
    if (!P) return;
    if (P->d_list) (void)hipFree(P->d_list);
    if (P->d_wg_map) (void)hipFree(P->d_wg_map);
    if (P->d_part_map) (void)hipFree(P->d_part_map);
    if (P->d_ws) (void)hipFree(P->d_ws);
    if (P->d_counters) (void)hipFree(P->d_counters);
    delete P;
}

}  // extern "C"
