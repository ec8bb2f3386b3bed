// Prefill GEMM (M > 16) for gfx950: y = x * W_hat^T on the matrix cores.
//
// The pages place the dequantization inside the matmul kernel (the Q-GEMM
// of the exllamav2 repository report, section "solution philosophy"); at
// large M the product is compute-bound, so here the dequantized tile is
// built once per workgroup in LDS and consumed by fp16 MFMA:
//   * a workgroup of 4 waves owns a 256 (rows of x) x 256 (output columns)
//     tile of y over all of K; each wave computes a 128 x 128 quarter of it
//     with v_mfma_f32_32x32x16_f16 into 16 fp32 accumulator blocks;
//   * K advances in stages of 64 (half a group), double-buffered in LDS: an
//     x tile [256 rows][64] and a W_hat tile [256 columns][64], both fp16
//     and k-contiguous, rows padded to 72 halves so that the 16-byte operand
//     reads of 8 or 16 consecutive rows fall in distinct banks;
//   * thread t stages column t of the W_hat tile: it loads the packed words
//     of its half group through fixed load slots (a slot the width does not
//     use reads an out-of-range offset: zeros, no memory traffic) and
//     dequantizes them exactly -- a code placed in the mantissa of an fp16
//     whose exponent makes its value 2^(10-o) + c, one packed subtract gives
//     c - z exactly and one packed multiply by the scale gives
//     fp16_RNE((c - z) * s), the bits of the dequantization definition;
//   * while the matrix cores work on stage s, the workgroup dequantizes
//     stage s+1 (loaded during stage s-1) into the other buffer and issues
//     the loads of stage s+2; one barrier per stage;
//   * workgroup ids are mapped to tiles XCD-aware: the ids one XCD receives
//     form a contiguous run of tiles in row-major order, so the x rows of a
//     tile are shared through that XCD's L2.
#include <hip/hip_runtime.h>

#include <climits>

#include "exq_device_common.h"
#include "exq_internal.h"

namespace exq {
namespace {

constexpr int kPT = 256;        // tile rows of x and tile columns of W
constexpr int kPK = 64;         // K per stage: half a group
constexpr int kPLd = kPK + 8;   // padded LDS row length, halves
constexpr int kPThreads = 256;  // 4 waves

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// Packed weights of one stage for this thread's column.
struct WRegs {
    uint32_t q[16];   // plane-0 dwords of the half group: up to 4 words
    uint32_t h[4];    // plane-1 dwords: up to 2 pieces of 2 dwords
    uint32_t s;       // fp16 scale in the low half
};

struct PrefillCtx {
    __amdgpu_buffer_rsrc_t rw, rs, rx;
    int tid, lane, wn0, wm0;
    uint32_t n;       // the column this thread stages
    bool n_ok;
};

// Where stage st comes from: half h = st % 2 of group g = st / 2.  A stage
// past the last one reloads the last (L2 hits, never used): a uniform test
// on it would split the stage into branches.
struct StageSrc {
    uint32_t g, P, h;
    int b;
};

__device__ __forceinline__ StageSrc stage_src(const LinearDev& L, int st, int S) {
    st = min(st, S - 1);
    StageSrc r;
    r.g = (uint32_t)(st >> 1);
    r.h = (uint32_t)(st & 1);
    const uint32_t meta = gptr<uint32_t>(L.meta)[r.g];
    r.P = meta >> 4;
    r.b = (int)(meta & 15u);
    return r;
}

// Packed words and scale of a stage.  Slots a width does not use read an
// out-of-range offset: zeros, no memory traffic, fixed load count.
__device__ __forceinline__ void issue_w(const LinearDev& L, const PrefillCtx& c, const StageSrc& src, WRegs& W) {
    const int b = src.b;
    const int p0 = b <= 3 ? 2 : (b == 8 ? 8 : 4), p1 = b - p0, nw0 = p0 >> 1;
    const uint32_t N16 = 16u * (uint32_t)L.N, h = src.h;
    const bool ok = c.n_ok;
    const uint32_t base = 16u * ((uint32_t)L.N * src.P + c.n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t off = (ok && i < nw0) ? base + ((uint32_t)nw0 * h + (uint32_t)i) * N16 : kBufOOB;
        const u4v v = __builtin_amdgcn_raw_buffer_load_b128(c.rw, off, 0, 0);
        W.q[4 * i + 0] = v[0];
        W.q[4 * i + 1] = v[1];
        W.q[4 * i + 2] = v[2];
        W.q[4 * i + 3] = v[3];
    }
    // plane 1: p1 = 1 -> dwords 2h, 2h+1 of word p0; p1 = 2 -> word p0 + h
    const uint32_t w1 = base + ((uint32_t)p0 + (p1 == 2 ? h : 0u)) * N16 + (p1 == 1 ? 8u * h : 0u);
    const uint32_t off0 = (ok && p1 > 0) ? w1 : kBufOOB;
    const uint32_t off1 = (ok && p1 == 2) ? w1 + 8u : kBufOOB;
    const u2v v0 = __builtin_amdgcn_raw_buffer_load_b64(c.rw, off0, 0, 0);
    const u2v v1 = __builtin_amdgcn_raw_buffer_load_b64(c.rw, off1, 0, 0);
    W.h[0] = v0[0];
    W.h[1] = v0[1];
    W.h[2] = v1[0];
    W.h[3] = v1[1];
    const uint32_t soff = ok ? 2u * (src.g * (uint32_t)L.N + c.n) : kBufOOB;
    W.s = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(c.rs, soff, 0, 0);
}

// x chunk `it` of a stage: row it * 32 + tid / 8 of the tile, k chunk tid % 8.
// Rows past M are outside the x buffer: zeros.
__device__ __forceinline__ u4v issue_x(const LinearDev& L, const PrefillCtx& c, const StageSrc& src, int it) {
    const uint32_t r = (uint32_t)(it * 32 + (c.tid >> 3)), kc = (uint32_t)(c.tid & 7);
    const uint32_t off = 2u * (r * (uint32_t)L.K + 128u * src.g + 64u * src.h + 8u * kc);
    return __builtin_amdgcn_raw_buffer_load_b128(c.rx, off, 0, 0);
}

// Width-generic decoding.  For unit U (codes 4U .. 4U+3 of the half group)
// the plane-0 field of code 4U + e sits at bit o + 8 e2 + 16 e1 of dword
// U p0 / 8 of the half's plane-0 dwords (o = (U p0) mod 8, e = e1 + 2 e2),
// and its plane-1 field at bit o + p1 ((U p0 / 8) mod R) + 8 e2 + 16 e1 of
// plane-1 dword U / 8 (p1 = 1) or U / 4 (p1 = 2) -- the EXQ1 layout restated
// per half group.  Shifting the plane-0 dword right by o and rotating the
// plane-1 dword right to bit p0, then merging under the plane-0 mask, leaves
// code 4U + e in bits [0, b) of byte e2 + 2 e1 ("canonical" dword).  Every
// width-dependent amount is a wave-uniform operand taken from this table.
struct DqRow {
    uint32_t shr[4];    // o for units U = 0..3 mod 4 (o repeats every 4 units)
    uint32_t rot[8];    // right rotation bringing the plane-1 field to bit p0 (repeats every 8)
    uint32_t mask0;     // bits [0, p0) of every byte
    uint32_t maskb;     // bits [0, b) of every byte
    uint32_t negc;      // fp16 pair -(1024 + z)
    uint32_t sel4;      // all ones when p0 == 4: plane-0 dword U / 2
    uint32_t sel8;      // all ones when p0 == 8: plane-0 dword U
    uint32_t sel6;      // all ones when p1 == 2: plane-1 dword U / 4
    uint32_t pad[2];
};

constexpr uint16_t f16_bits_of_int(int v) {
    // |v| < 2048: exact in fp16
    uint32_t a = (uint32_t)(v < 0 ? -v : v);
    if (a == 0) return v < 0 ? 0x8000u : 0u;
    int e = 0;
    while ((a >> e) > 1) ++e;
    const uint32_t mant = ((a << 10) >> e) & 0x3FFu;
    return (uint16_t)((v < 0 ? 0x8000u : 0u) | ((uint32_t)(e + 15) << 10) | mant);
}

constexpr DqRow dq_row(int b) {
    DqRow r{};
    if (!(b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8)) return r;
    const int p0 = b <= 3 ? 2 : (b == 8 ? 8 : 4), p1 = b - p0;
    const int R = p1 ? p0 / p1 : 1;
    for (int U = 0; U < 8; ++U) {
        const int o = (U * p0) % 8;
        const int sh1 = o + p1 * (((U * p0) / 8) % R);
        if (U < 4) r.shr[U] = (uint32_t)o;
        r.rot[U] = (uint32_t)((sh1 - p0 + 32) % 32);
    }
    r.mask0 = ((1u << p0) - 1u) * 0x01010101u;
    r.maskb = ((1u << b) - 1u) * 0x01010101u;
    const uint32_t nc = f16_bits_of_int(-(1024 + (1 << (b - 1))));
    r.negc = nc | (nc << 16);
    r.sel4 = p0 == 4 ? ~0u : 0u;
    r.sel8 = p0 == 8 ? ~0u : 0u;
    r.sel6 = p1 == 2 ? ~0u : 0u;
    return r;
}

__constant__ DqRow kDq[9] = {dq_row(0), dq_row(1), dq_row(2), dq_row(3), dq_row(4),
                             dq_row(5), dq_row(6), dq_row(7), dq_row(8)};

__device__ __forceinline__ uint32_t pick(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

// Part KK (units 4KK .. 4KK+3, k in [16KK, 16KK+16)) of the dequantization
// of this thread's column of a half group into its LDS row: each code goes
// into the low byte of an fp16 with high byte 0x64, whose value is then
// 1024 + c; subtracting 1024 + z is exact and the multiply by the scale
// rounds once, giving fp16_RNE((c - z) * s).
template <int KK>
__device__ __forceinline__ void dequant_part(const WRegs& W, const DqRow& T, uint16_t* wrow) {
    const h2 s2 = as_h2(W.s | (W.s << 16));
    const h2 nc = as_h2(T.negc);
    uint32_t out[8];
    static_for<0, 4>([&](auto VC) {
        constexpr int V = decltype(VC)::value;
        constexpr int U = 4 * KK + V;
        uint32_t q = W.q[U >> 2];
        if constexpr ((U >> 1) != (U >> 2)) q = pick(T.sel4, W.q[U >> 1], q);
        if constexpr (U != (U >> 2)) q = pick(T.sel8, W.q[U], q);
        uint32_t hv = W.h[U >> 3];
        if constexpr ((U >> 2) != (U >> 3)) hv = pick(T.sel6, W.h[U >> 2], hv);
        const uint32_t lo = q >> T.shr[U & 3];
        const uint32_t hi = __builtin_amdgcn_alignbit(hv, hv, T.rot[U & 7]);
        const uint32_t canon = pick(T.mask0, lo, hi) & T.maskb;
        const uint32_t b0 = __builtin_amdgcn_perm(0x64646464u, canon, 0x04020400u);   // codes 4U, 4U+1
        const uint32_t b1 = __builtin_amdgcn_perm(0x64646464u, canon, 0x04030401u);   // codes 4U+2, 4U+3
        out[2 * V] = __builtin_bit_cast(uint32_t, (as_h2(b0) + nc) * s2);
        out[2 * V + 1] = __builtin_bit_cast(uint32_t, (as_h2(b1) + nc) * s2);
    });
    *reinterpret_cast<u4v*>(wrow + 16 * KK) = u4v{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<u4v*>(wrow + 16 * KK + 8) = u4v{out[4], out[5], out[6], out[7]};
}

__device__ __forceinline__ void store_x_chunk(const u4v& v, uint16_t* sx, int tid, int it) {
    *reinterpret_cast<u4v*>(sx + (it * 32 + (tid >> 3)) * kPLd + 8 * (tid & 7)) = v;
}

// MFMA operands of K-step kk (16 k) for this wave's 128 x 128 quarter.
// Operand A is W_hat (rows = output columns n), operand B is x (columns =
// rows m of x); lane l holds row l % 32 of a 32-block, k 8 (l / 32) .. +8.
struct Frags {
    h8 a[4], b[4];
};

__device__ __forceinline__ void load_frags(const uint16_t* sw, const uint16_t* sx, const PrefillCtx& c, int kk,
                                           Frags& f) {
    const int r = c.lane & 31, kh = (c.lane >> 5) * 8;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
        f.a[ib] = *reinterpret_cast<const h8*>(sw + (c.wn0 + 32 * ib + r) * kPLd + 16 * kk + kh);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
        f.b[jb] = *reinterpret_cast<const h8*>(sx + (c.wm0 + 32 * jb + r) * kPLd + 16 * kk + kh);
}

__device__ __forceinline__ void mfma_frags(const Frags& f, f16v (&acc)[4][4]) {
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[ib], f.b[jb], acc[ib][jb], 0, 0, 0);
}

// Issue pattern of one region: each of its 16 MFMAs followed by up to four
// VALU operations, one LDS operation and one global load, so that the
// dequantization and staging run in the shadow of the matrix cores.
__device__ __forceinline__ void region_schedule() {
    static_for<0, 16>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);   // LDS
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
    });
}

// Stage st: multiply LDS buffer (rd_w, rd_x); stage st+1 (weights in Wn, x
// chunks in xr, width row T) into buffer (wr_w, wr_x); load stage st+2 (src)
// into Wf and, chunk by chunk as they are freed, into xr.
//
// Four regions, one per K-step, separated by sched_barrier so the scheduler
// interleaves a region's dequantization with its MFMAs without hoisting a
// whole stage's operands.  Region r reads the operands of K-step r and
// multiplies K-step r - 1; region 0 multiplies the previous stage's last
// K-step (`carry`, read before the barrier), so no MFMA waits for an operand
// read issued in its own region.  On return `carry` holds K-step 3.
//
// The scalars of the next stage (src_n: stage st+3, T_n: the width row of
// stage st+2) are loaded at the very end and first used after the closing
// barrier, whose wait covers them: scalar loads return out of order, so
// while one is outstanding every wait for an operand read would have to
// drain all of them.
__device__ __forceinline__ void stage_body(const LinearDev& L, const PrefillCtx& c, int st, int S,
                                           const uint16_t* rd_w, const uint16_t* rd_x, uint16_t* wr_w,
                                           uint16_t* wr_x, const WRegs& Wn, WRegs& Wf, u4v (&xr)[8],
                                           const StageSrc& src, const DqRow& T, StageSrc& src_n, DqRow& T_n,
                                           Frags& carry, Frags& other, f16v (&acc)[4][4]) {
    issue_w(L, c, src, Wf);
    static_for<0, 4>([&](auto KC) {
        constexpr int KK = decltype(KC)::value;
        Frags& rd = (KK & 1) ? carry : other;     // K-step KK lands here
        Frags& mul = (KK & 1) ? other : carry;    // K-step KK - 1 (previous stage's 3 for KK = 0)
        load_frags(rd_w, rd_x, c, KK, rd);
        dequant_part<KK>(Wn, T, wr_w + c.tid * kPLd);
        store_x_chunk(xr[2 * KK], wr_x, c.tid, 2 * KK);
        store_x_chunk(xr[2 * KK + 1], wr_x, c.tid, 2 * KK + 1);
        xr[2 * KK] = issue_x(L, c, src, 2 * KK);
        xr[2 * KK + 1] = issue_x(L, c, src, 2 * KK + 1);
        mfma_frags(mul, acc);
        region_schedule();
        __builtin_amdgcn_sched_barrier(0);
    });
    // Last, so that no wait inside the regions has a scalar load to cover.
    src_n = stage_src(L, st + 3, S);
    T_n = kDq[src.b];
}

__global__ __launch_bounds__(kPThreads) void prefill_kernel(LinearDev L, int M, int row_tiles, int col_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t sw0[kPT * kPLd];
    __shared__ __attribute__((aligned(16))) uint16_t sw1[kPT * kPLd];
    __shared__ __attribute__((aligned(16))) uint16_t sx0[kPT * kPLd];
    __shared__ __attribute__((aligned(16))) uint16_t sx1[kPT * kPLd];

    // XCD-aware tile order: ids i, i+8, i+16, ... (one XCD) take consecutive tiles.
    const int T = row_tiles * col_tiles;
    const int i = blockIdx.x, xcd = i & 7, per = T >> 3, rem = T & 7;
    const int t = xcd * per + min(xcd, rem) + (i >> 3);
    const int m0 = (t / col_tiles) * kPT, n0 = (t % col_tiles) * kPT;

    PrefillCtx c;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    const int wave = c.tid >> 6;
    c.wn0 = (wave & 1) * 128;
    c.wm0 = (wave >> 1) * 128;
    c.n = (uint32_t)(n0 + c.tid);
    c.n_ok = (int)c.n < L.N;
    c.rw = buffer_rsrc(L.qweight, L.qbytes);
    c.rs = buffer_rsrc(L.scales, L.sbytes);
    const int rows = min(M - m0, kPT);
    c.rx = buffer_rsrc(L.x + (size_t)m0 * L.K, 2u * (uint32_t)rows * (uint32_t)L.K);

    const int S = 2 * L.G;
    f16v acc[4][4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[ib][jb][e] = 0.f;

    WRegs W0, W1;
    u4v xr[8];
    StageSrc srcA, srcB;   // stage st+2 for the even / odd stage of an iteration
    DqRow TA, TB;          // width row of stage st+1, likewise
    {
        // Stage 0 is staged alone; from then on every stage stages the next.
        const StageSrc s0 = stage_src(L, 0, S), s1 = stage_src(L, 1, S);
        srcA = stage_src(L, 2, S);
        TA = kDq[s1.b];
        issue_w(L, c, s0, W0);
        issue_w(L, c, s1, W1);
#pragma unroll
        for (int it = 0; it < 8; ++it) xr[it] = issue_x(L, c, s0, it);
        const DqRow& T0 = kDq[s0.b];
        static_for<0, 4>([&](auto KC) { dequant_part<decltype(KC)::value>(W0, T0, sw0 + c.tid * kPLd); });
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            store_x_chunk(xr[it], sx0, c.tid, it);
            xr[it] = issue_x(L, c, s1, it);
        }
    }
    // Zero operands: the first stage's region 0 adds exact zeros.
    Frags carry, other;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        carry.a[i] = h8{};
        carry.b[i] = h8{};
    }
    __syncthreads();
    for (int st = 0; st < S; st += 2) {
        stage_body(L, c, st, S, sw0, sx0, sw1, sx1, W1, W0, xr, srcA, TA, srcB, TB, carry, other, acc);
        __syncthreads();
        stage_body(L, c, st + 1, S, sw1, sx1, sw0, sx0, W0, W1, xr, srcB, TB, srcA, TA, carry, other, acc);
        __syncthreads();
    }
    mfma_frags(carry, acc);

    // Epilogue: lane holds rows m = 32 jb + lane % 32 and, per a, four
    // consecutive columns n = 32 ib + 8 a + 4 (lane / 32) + [0, 4).
    const int lr = c.lane & 31, lh = c.lane >> 5;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const int m = m0 + c.wm0 + 32 * jb + lr;
        if (m >= M) continue;
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int n = n0 + c.wn0 + 32 * ib + 8 * a + 4 * lh;
                if (n >= L.N) continue;
                const uint32_t lo = (uint32_t)f32_to_f16_bits(acc[ib][jb][4 * a]) |
                                    ((uint32_t)f32_to_f16_bits(acc[ib][jb][4 * a + 1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_f16_bits(acc[ib][jb][4 * a + 2]) |
                                    ((uint32_t)f32_to_f16_bits(acc[ib][jb][4 * a + 3]) << 16);
                const u2v v = {lo, hi};
                *gptr_w<u2v>(L.y + (size_t)m * L.N + n) = v;
            }
    }
}

}  // namespace
}  // namespace exq

using namespace exq;

exq_status exq_prefill_launch(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream) {
    // Offsets into one tile's rows of x are 32-bit: 2 * 256 * K bytes must stay below 2^31.
    if ((size_t)2 * kPT * (size_t)L->K >= (size_t)kBufOOB)
        return fail(EXQ_ERR_UNSUPPORTED, "K=%d is too large for the prefill kernel", L->K);
    const long row_tiles = (M + kPT - 1) / kPT, col_tiles = (L->N + kPT - 1) / kPT;
    if (row_tiles * col_tiles > INT_MAX) return fail(EXQ_ERR_UNSUPPORTED, "M=%d gives too many tiles", M);
    LinearDev d = linear_dev(L, x, y);
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)(row_tiles * col_tiles)), dim3(kPThreads), 0, stream, d, M,
                       (int)row_tiles, (int)col_tiles);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : fail(EXQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
}
