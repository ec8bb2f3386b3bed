// Prefill GEMM (M > 16) for gfx950: y = x * W_hat^T on the matrix cores.
//
// The pages place the dequantization inside the matmul kernel (the Q-GEMM
// of the exllamav2 repository report, section "solution philosophy"); at
// large M the product is compute-bound, so the codes are expanded once per
// workgroup tile straight into MFMA operands:
//   * a workgroup of 4 waves owns a 256 (rows of x) x 256 (output columns)
//     tile of y over all of K; wave w owns columns [64 w, 64 w + 64) of it and
//     all 256 rows, 16 blocks of v_mfma_f32_32x32x16_f16 accumulators;
//   * K advances in stages of 64 (half a group).  Within a stage the order of
//     k is free as long as x follows it: MFMA k-slot 8 j + i of K-step kk is
//     code 32 j + 8 kk + i of the half group, so lane l (j = l / 32) consumes
//     exactly EXQ1 quarter 2 h + j of its column -- the 4 b bytes the decode
//     kernel reads -- and decodes it itself, into its own A operands, with
//     wave-uniform shifts and register picks.  W_hat never goes through LDS
//     and no dequantized value is computed twice;
//   * x is copied from global memory straight into LDS (buffer loads with
//     the LDS flag: no registers, no LDS store instructions), [256 rows]
//     [64 k] per stage, 4 buffers so that a stage's copy has two stages to
//     land; 16-byte chunks are XOR-swizzled within a row so that operand
//     reads of 16 consecutive rows fall in distinct banks; one barrier per
//     stage;
//   * decoding is exact and width-generic: a code goes into the low byte of
//     an fp16 whose high byte is 0x64, which reads 1024 + c; one packed
//     subtract of 1024 + z and one packed multiply by the scale give
//     fp16_RNE((c - z) * s), the bits of the dequantization definition;
//   * workgroup ids are mapped to tiles XCD-aware: the ids one XCD receives
//     form a contiguous run of tiles in row-major order, so the x rows of a
//     tile are shared through that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>

#include "exq_device_common.h"
#include "exq_internal.h"

namespace exq {
namespace {

constexpr int kPT = 256;        // tile rows of x and tile columns of W
constexpr int kPK = 64;         // K per stage: half a group
constexpr int kPXBytes = kPT * kPK * 2;   // one stage's x tile in LDS: 256 rows of 128 bytes
constexpr int kPThreads = 256;  // 4 waves

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

struct PrefillCtx {
    __amdgpu_buffer_rsrc_t rw, rs, rx;
    int tid, lane, wave;
    uint32_t q;        // K-quarter of the half group this lane decodes (lane / 32)
    uint32_t col[2];   // its two columns (clamped into [0, N): extra columns are never stored)
    uint32_t xo[4];    // LDS byte offset of the lane's x operand of K-step kk in row block 0
    uint32_t xv[8];    // x buffer offset of the 16 bytes the lane copies in copy `it` of a stage
};

// x tile rows are 128 bytes (8 slots of 16 bytes); k chunk kc of row r sits in
// slot kc ^ xswz(r), so that 16-byte operand reads of 16 consecutive rows at
// one kc touch 16 distinct slot / row-parity pairs: no bank conflicts.
__device__ __forceinline__ uint32_t xswz(uint32_t r) { return (r & 7u) ^ ((r >> 3) & 1u); }

// Where stage st of a tile's stage range [lo, hi) comes from: half h = st % 2
// of group g = st / 2.  A stage past the last one reloads the last (cache
// hits, never used): a uniform test on it would split the stage into
// branches.  Stages lo - 2 and lo - 1 (run first when the range holds 2 mod 4
// stages) read stage lo's words with an out-of-range scale offset: scale 0,
// so every weight they decode is a zero.
struct StageSrc {
    uint32_t g, P, h, so;   // so: byte offset of the group's scales (out of range: zeros)
    int b;
};

__device__ __forceinline__ StageSrc stage_src(const LinearDev& L, int st, int lo, int hi) {
    const uint32_t null_scale = st < lo ? kBufOOB : 0u;
    st = max(min(st, hi - 1), lo);
    StageSrc r;
    r.g = (uint32_t)(st >> 1);
    r.h = (uint32_t)(st & 1);
    r.so = null_scale + 2u * r.g * (uint32_t)L.N;
    // Read-only for the kernel: a constant-space load keeps it scalar although
    // the LDS copies count as memory writes.
    const uint32_t meta = ((const __attribute__((address_space(4))) uint32_t*)L.meta)[r.g];
    r.P = meta >> 4;
    r.b = (int)(meta & 15u);
    return r;
}

// Packed words of one K-quarter of one column, and its scale.
struct QRegs {
    uint32_t q[8];   // plane-0 dwords (p0 of them)
    uint32_t h[2];   // plane-1 dwords (p1 of them)
    uint32_t s;      // fp16 scale in the low half
};

// Loads quarter 2h + j of the lane's two columns through fixed slots; a slot
// the width does not use reads an out-of-range offset (zeros, no traffic).
// Column-local dword m of group g sits at byte 16 (N P_g + (m / 4) N + n) + 4 (m % 4).
// SAME_GROUP: the stage is the second half of the group `prev` was loaded
// for (stages run in pairs from an even one), so its scale is prev's.
template <bool SAME_GROUP>
__device__ __forceinline__ void issue_w(const LinearDev& L, const PrefillCtx& c, const StageSrc& src,
                                        QRegs (&W)[2], const QRegs (&prev)[2]) {
    const int b = src.b;
    const uint32_t p0 = b <= 3 ? 2u : (b == 8 ? 8u : 4u), p1 = (uint32_t)b - p0;
    const uint32_t N16 = 16u * (uint32_t)L.N, qq = 2u * src.h + c.q;
    const uint32_t m0 = p0 * qq, m1 = 4u * p0 + p1 * qq;
    const uint32_t offA = (m0 >> 2) * N16 + 4u * (m0 & 3u);
    const uint32_t offC = (m1 >> 2) * N16 + 4u * (m1 & 3u);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t base = 16u * ((uint32_t)L.N * src.P + c.col[i]);
        const u4v a = __builtin_amdgcn_raw_buffer_load_b128(c.rw, base + offA, 0, 0);
        const u4v bq = __builtin_amdgcn_raw_buffer_load_b128(c.rw, p0 == 8 ? base + offA + N16 : kBufOOB, 0, 0);
        const u2v hh = __builtin_amdgcn_raw_buffer_load_b64(c.rw, p1 >= 1 ? base + offC : kBufOOB, 0, 0);
        W[i].q[0] = a[0];
        W[i].q[1] = a[1];
        W[i].q[2] = a[2];
        W[i].q[3] = a[3];
        W[i].q[4] = bq[0];
        W[i].q[5] = bq[1];
        W[i].q[6] = bq[2];
        W[i].q[7] = bq[3];
        W[i].h[0] = hh[0];
        W[i].h[1] = hh[1];
        if constexpr (SAME_GROUP)
            W[i].s = prev[i].s;   // the second half of a group: the first half's scale
        else
            W[i].s = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(c.rs, src.so + 2u * c.col[i], 0, 0);
    }
}

// Copy `it` of a stage: the wave's 64 lanes move rows 64 w + 8 it .. + 8 of
// the stage's x tile (1 KiB) straight into LDS, lane i writing bytes
// [16 i, 16 i + 16) of that KiB, so lane i fetches k chunk
// (i % 8) ^ xswz(row) of row 64 w + 8 it + i / 8.  The stage's position in K
// goes in the scalar offset; rows past M fail the range check of the
// vector offset and read zeros.
__device__ __forceinline__ void copy_x(const PrefillCtx& c, const StageSrc& src, uint16_t* sx, int it) {
    const uint32_t soff = 256u * src.g + 128u * src.h;
    char* dst = reinterpret_cast<char*>(sx) + 1024 * (8 * c.wave + it);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_ptr_t)dst, 16, (int)c.xv[it], (int)soff, 0, 0);
}

// Width-generic decoding.  For unit U (codes 4U .. 4U+3 of a K-quarter) the
// plane-0 field of code 4U + e sits at bit o + 8 e2 + 16 e1 of dword U p0 / 8
// of the quarter's plane-0 dwords (o = (U p0) mod 8, e = e1 + 2 e2), and its
// plane-1 field at bit o + p1 ((U p0 / 8) mod R) + 8 e2 + 16 e1 of plane-1
// dword U p1 / 8 -- the EXQ1 layout restated per quarter.  Shifting the plane-0 dword right by o and rotating the
// plane-1 dword right to bit p0, then merging under the plane-0 mask, leaves
// code 4U + e in bits [0, b) of byte e2 + 2 e1 ("canonical" dword).  Every
// width-dependent amount is a wave-uniform operand taken from this table.
struct DqRow {
    uint32_t shr[4];    // o for units U = 0..3 mod 4 (o repeats every 4 units)
    uint32_t rot[8];    // right rotation bringing the plane-1 field to bit p0 (repeats every 8)
    uint32_t mask0;     // bits [0, p0) of every byte
    uint32_t maskb;     // bits [0, b) of every byte
    uint32_t negc;      // fp16 pair -(1024 + z)
    uint32_t sel4;      // all ones when p0 == 4: plane-0 dword U / 2 (else U / 4)
    uint32_t sel8;      // all ones when p0 == 8: plane-0 dword U
    uint32_t sel6;      // all ones when p1 == 2: plane-1 dword U / 4 (else 0)
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

// A operand of K-step kk for one column: units 2 kk and 2 kk + 1 of the
// lane's quarter, i.e. codes 8 kk .. 8 kk + 7 as fp16_RNE((c - z) * s).  Each
// code goes into the low byte of an fp16 with high byte 0x64 (value 1024 + c);
// subtracting 1024 + z is exact and the multiply by the scale rounds once.
template <int KK>
__device__ __forceinline__ h8 dequant_operand(const QRegs& W, const DqRow& T) {
    const h2 s2 = as_h2(W.s | (W.s << 16));
    const h2 nc = as_h2(T.negc);
    uint32_t out[4];
    static_for<0, 2>([&](auto VC) {
        constexpr int V = decltype(VC)::value;
        constexpr int U = 2 * KK + V;
        uint32_t q = W.q[U >> 2];
        if constexpr ((U >> 1) != (U >> 2)) q = pick(T.sel4, W.q[U >> 1], q);
        if constexpr (U != (U >> 2)) q = pick(T.sel8, W.q[U], q);
        uint32_t hv = W.h[0];
        if constexpr ((U >> 2) != 0) hv = pick(T.sel6, W.h[U >> 2], hv);
        const uint32_t lo = q >> T.shr[U & 3];
        const uint32_t hi = __builtin_amdgcn_alignbit(hv, hv, T.rot[U & 7]);
        const uint32_t canon = pick(T.mask0, lo, hi) & T.maskb;
        const uint32_t b0 = __builtin_amdgcn_perm(0x64646464u, canon, 0x04020400u);   // codes 4U, 4U+1
        const uint32_t b1 = __builtin_amdgcn_perm(0x64646464u, canon, 0x04030401u);   // codes 4U+2, 4U+3
        out[2 * V] = __builtin_bit_cast(uint32_t, (as_h2(b0) + nc) * s2);
        out[2 * V + 1] = __builtin_bit_cast(uint32_t, (as_h2(b1) + nc) * s2);
    });
    const u4v v = {out[0], out[1], out[2], out[3]};
    return __builtin_bit_cast(h8, v);
}

// Operands of one K-step: the wave's two W blocks (A) and eight x blocks (B).
struct Ops {
    h8 a[2], x[8];
};

// x operand of K-step kk: lane l holds row 32 jb + l % 32 of the tile and the
// x values that meet its k-slots, k = 32 (l / 32) + 8 kk + [0, 8).
__device__ __forceinline__ void load_x_ops(const uint16_t* sx, const PrefillCtx& c, int kk, Ops& o) {
    const char* base = reinterpret_cast<const char*>(sx) + c.xo[kk];
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) o.x[jb] = *reinterpret_cast<const h8*>(base + jb * 32 * 128);
}

__device__ __forceinline__ void mfma_ops(const Ops& o, f16v (&acc)[2][8]) {
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[ib], o.x[jb], acc[ib][jb], 0, 0, 0);
}

// Issue pattern of one region: each of its 16 MFMAs followed by one LDS
// operation, one global load and up to four VALU operations, so that
// decoding and staging run in the shadow of the matrix cores.  Memory
// operations right behind each MFMA measured 1.2 % faster than after the
// VALU operations.
__device__ __forceinline__ void region_schedule() {
    static_for<0, 16>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x080, 1, 0);   // LDS
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
    });
}

// Stage st.  On entry LDS buffer rd_x holds stage st's x tile, Wc its packed
// words, `carry` the operands of the previous stage's last K-step; stage
// st + 1's x tile is landing in another buffer.  Region r reads and decodes
// the operands of K-step r and multiplies K-step r - 1 (region 0: `carry`,
// prepared before the barrier), so no MFMA waits for work issued in its own
// region; it also starts two of the wave's copies of stage st + 2's x tile
// into wr_x, the buffer stage st - 2 read.  Stage st+1's packed words go into
// Wn.  sched_barrier keeps the regions apart so the scheduler interleaves
// within a region without hoisting a whole stage's operands.
//
// The scalars of the next stage (src3: stage st+3, T_n: the width row of
// stage st+1) are loaded at the very end and first used after the closing
// barrier, whose wait covers them: scalar loads return out of order, so
// while one is outstanding every wait for an operand read would drain all.
template <bool NEXT_SAME_GROUP>
__device__ __forceinline__ void stage_body(const LinearDev& L, const PrefillCtx& c, int st, int lo, int hi,
                                           const uint16_t* rd_x, uint16_t* wr_x, const QRegs (&Wc)[2],
                                           QRegs (&Wn)[2], const StageSrc& src1, const StageSrc& src2,
                                           const DqRow& T, StageSrc& src3, DqRow& T_n, Ops& carry, Ops& other,
                                           f16v (&acc)[2][8]) {
    issue_w<NEXT_SAME_GROUP>(L, c, src1, Wn, Wc);
    static_for<0, 4>([&](auto KC) {
        constexpr int KK = decltype(KC)::value;
        Ops& rd = (KK & 1) ? carry : other;     // K-step KK lands here
        Ops& mul = (KK & 1) ? other : carry;    // K-step KK - 1 (previous stage's 3 for KK = 0)
        load_x_ops(rd_x, c, KK, rd);
        rd.a[0] = dequant_operand<KK>(Wc[0], T);
        rd.a[1] = dequant_operand<KK>(Wc[1], T);
        copy_x(c, src2, wr_x, 2 * KK);
        copy_x(c, src2, wr_x, 2 * KK + 1);
        mfma_ops(mul, acc);
        region_schedule();
        __builtin_amdgcn_sched_barrier(0);
    });
    // Last, so that no wait inside the regions has a scalar load to cover.
    src3 = stage_src(L, st + 3, lo, hi);
    T_n = kDq[src1.b];
}

// Closes a stage.  A stage issues at least 14 vector memory operations (6 or
// 8 packed-word and scale loads, 8 copies), so waiting until at most 8 are
// outstanding completes every one issued before it -- in particular the
// copies of the x tile the next stage reads; then the barrier makes the
// copies of all waves visible.
// The copies write LDS behind the compiler's back as far as __syncthreads is
// concerned (its fence would wait for all of them), hence the explicit wait
// and a bare barrier; sched_barrier keeps the next stage's reads below it.
__device__ __forceinline__ void stage_end() {
    __builtin_amdgcn_s_waitcnt((8 & 15) | ((8 >> 4) << 14) | (7 << 4) | (15 << 8));   // vmcnt(8)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// SiLU(g) * u in fp32 (g read back as fp16): g / (1 + e^-g) * u.
__device__ __forceinline__ float silu_mul_h(uint16_t g16, float u) {
    const float g = (float)__builtin_bit_cast(_Float16, g16);
    return g / (1.0f + expf(-g)) * u;
}

// A tile of a prefill plan cut along K into nparts pieces (part in K order):
// each piece stores its fp32 sums to the plan's workspace and counts itself;
// the last to arrive adds all pieces in K order and stores y.
struct TilePart {
    int part, nparts;
    float* ws;               // nparts x [256 accumulators][256 threads] floats of this tile
    uint32_t* counter;       // arrivals of this tile (zero between launches)
};

// One 256 x 256 output tile (rows m0.., columns n0..) over K-stages [lo, hi)
// (a stage is half a group).  GATED: y already holds the gate product g
// (fp16) of the same tile, and the tile stores SiLU(g) * acc over it.
template <bool GATED>
__device__ __forceinline__ void prefill_tile(const LinearDev& L, int M, int m0, int n0, int lo, int hi,
                                             const TilePart& tp, uint16_t* sxa, uint16_t* sxb, uint16_t* sxc,
                                             uint16_t* sxd) {
    PrefillCtx c;
    c.tid = threadIdx.x;
    c.lane = c.tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
    c.q = (uint32_t)(c.lane >> 5);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) c.col[ib] = (uint32_t)min(n0 + 64 * c.wave + 32 * ib + (c.lane & 31), L.N - 1);
    c.rw = buffer_rsrc(L.qweight, L.qbytes);
    c.rs = buffer_rsrc(L.scales, L.sbytes);
    const int rows = min(M - m0, kPT);
    c.rx = buffer_rsrc(L.x + (size_t)m0 * L.K, 2u * (uint32_t)rows * (uint32_t)L.K);
    {
        // Operand reads: row lane % 32 of each row block, k chunk 4 (lane / 32) + kk.
        const uint32_t r = (uint32_t)(c.lane & 31), s0 = (4u * c.q) ^ xswz(r);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) c.xo[kk] = 128u * r + 16u * (s0 ^ (uint32_t)kk);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const uint32_t R = (uint32_t)(64 * c.wave + 8 * it + (c.lane >> 3));
            c.xv[it] = 2u * (uint32_t)L.K * R + 16u * ((uint32_t)(c.lane & 7) ^ xswz(R));
        }
    }

    f16v acc[2][8];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[ib][jb][e] = 0.f;

    QRegs W0[2], W1[2];
    StageSrc s1, s2;
    DqRow T0;
    // The loop runs 4 stages per trip, each with its own x buffer; a stage
    // count of 2 mod 4 starts two stages early on zero x tiles and zero scales.
    const int st0 = ((hi - lo) & 2) ? lo - 2 : lo;
    {
        const StageSrc s0 = stage_src(L, st0, lo, hi);
        s1 = stage_src(L, st0 + 1, lo, hi);
        s2 = stage_src(L, st0 + 2, lo, hi);
        T0 = kDq[s0.b];
        if (st0 == lo) {
#pragma unroll
            for (int it = 0; it < 8; ++it) copy_x(c, s0, sxa, it);
#pragma unroll
            for (int it = 0; it < 8; ++it) copy_x(c, s1, sxb, it);
        } else {
            const u4v z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int k = 0; k < kPXBytes / 16 / kPThreads; ++k) {
                *reinterpret_cast<u4v*>(reinterpret_cast<char*>(sxa) + 16 * (k * kPThreads + c.tid)) = z;
                *reinterpret_cast<u4v*>(reinterpret_cast<char*>(sxb) + 16 * (k * kPThreads + c.tid)) = z;
            }
        }
        issue_w<false>(L, c, s0, W0, W0);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    // Zero operands: the first stage's region 0 adds exact zeros.
    Ops carry, other;
#pragma unroll
    for (int k = 0; k < 8; ++k) carry.x[k] = h8{};
    carry.a[0] = h8{};
    carry.a[1] = h8{};
    __syncthreads();
    for (int st = st0; st < hi; st += 4) {
        StageSrc s3, s4, s5, s6;
        DqRow T1, T2, T3, T4;
        stage_body<true>(L, c, st, lo, hi, sxa, sxc, W0, W1, s1, s2, T0, s3, T1, carry, other, acc);
        stage_end();
        stage_body<false>(L, c, st + 1, lo, hi, sxb, sxd, W1, W0, s2, s3, T1, s4, T2, carry, other, acc);
        stage_end();
        stage_body<true>(L, c, st + 2, lo, hi, sxc, sxa, W0, W1, s3, s4, T2, s5, T3, carry, other, acc);
        stage_end();
        stage_body<false>(L, c, st + 3, lo, hi, sxd, sxb, W1, W0, s4, s5, T3, s6, T4, carry, other, acc);
        stage_end();
        s1 = s5;
        s2 = s6;
        T0 = T4;
    }
    mfma_ops(carry, acc);
    // The last stages' copies (of clamped stages, never read) land before
    // the tile ends, so none can reach the LDS of the next workgroup.
    __builtin_amdgcn_s_waitcnt((0 & 15) | ((0 >> 4) << 14) | (7 << 4) | (15 << 8));   // vmcnt(0)

    if constexpr (!GATED) {
        if (tp.nparts > 1) {
            // Piece of a tile cut along K.  Accumulator k (= 16 (8 ib + jb) + e)
            // of thread t goes to ws[part][k][t]: agent-scope stores, each
            // thread waiting for its own before the barrier (a workgroup
            // barrier does not wait for global stores), then one release count.
            __shared__ uint32_t last;
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int jb = 0; jb < 8; ++jb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __hip_atomic_store(tp.ws + ((size_t)tp.part * 256 + (16 * (8 * ib + jb) + e)) * kPThreads + c.tid,
                                           acc[ib][jb][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt((0 & 15) | ((0 >> 4) << 14) | (7 << 4) | (15 << 8));   // vmcnt(0)
            __syncthreads();
            if (c.tid == 0)
                last = __hip_atomic_fetch_add(tp.counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(tp.nparts - 1);
            __syncthreads();
            if (!last) return;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            // The last piece adds the stored pieces (its own among them) in K
            // order, whatever the arrival order, four outputs at a time.
            const int lr = c.lane & 31, lh = c.lane >> 5;
            for (int jb = 0; jb < 8; ++jb) {
                const int m = m0 + 32 * jb + lr;
                if (m >= M) continue;
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int n = n0 + 64 * c.wave + 32 * ib + 8 * a + 4 * lh;
                        if (n >= L.N) continue;
                        float o[4];
                        for (int p = 0; p < tp.nparts; ++p) {
                            const float* src = tp.ws + ((size_t)p * 256 + 16 * (8 * ib + jb) + 4 * a) * kPThreads + c.tid;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v = __hip_atomic_load(src + e * kPThreads, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT);
                                o[e] = p == 0 ? v : o[e] + v;
                            }
                        }
                        const uint32_t lo16 = (uint32_t)f32_to_f16_bits(o[0]) | ((uint32_t)f32_to_f16_bits(o[1]) << 16);
                        const uint32_t hi16 = (uint32_t)f32_to_f16_bits(o[2]) | ((uint32_t)f32_to_f16_bits(o[3]) << 16);
                        const u2v v = {lo16, hi16};
                        *gptr_w<u2v>(L.y + (size_t)m * L.N + n) = v;
                    }
            }
            if (c.tid == 0) __hip_atomic_store(tp.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }

    // Epilogue: lane holds rows m = 32 jb + lane % 32 and, per a, four
    // consecutive columns n = 64 wave + 32 ib + 8 a + 4 (lane / 32) + [0, 4).
    const int lr = c.lane & 31, lh = c.lane >> 5;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
        const int m = m0 + 32 * jb + lr;
        if (m >= M) continue;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int n = n0 + 64 * c.wave + 32 * ib + 8 * a + 4 * lh;
                if (n >= L.N) continue;
                float o[4] = {acc[ib][jb][4 * a], acc[ib][jb][4 * a + 1], acc[ib][jb][4 * a + 2],
                              acc[ib][jb][4 * a + 3]};
                if constexpr (GATED) {
                    const u2v g = *gptr_w<u2v>(L.y + (size_t)m * L.N + n);
                    o[0] = silu_mul_h((uint16_t)(g[0] & 0xFFFFu), o[0]);
                    o[1] = silu_mul_h((uint16_t)(g[0] >> 16), o[1]);
                    o[2] = silu_mul_h((uint16_t)(g[1] & 0xFFFFu), o[2]);
                    o[3] = silu_mul_h((uint16_t)(g[1] >> 16), o[3]);
                }
                const uint32_t lo = (uint32_t)f32_to_f16_bits(o[0]) | ((uint32_t)f32_to_f16_bits(o[1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_f16_bits(o[2]) | ((uint32_t)f32_to_f16_bits(o[3]) << 16);
                const u2v v = {lo, hi};
                *gptr_w<u2v>(L.y + (size_t)m * L.N + n) = v;
            }
    }
}

template <bool GATED>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(LinearDev L, int M, int row_tiles, int col_tiles) {
    __shared__ __attribute__((aligned(1024))) uint16_t sxa[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxb[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxc[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxd[kPXBytes / 2];
    // XCD-aware tile order: ids x, x+8, x+16, ... (XCD x) take block x of
    // xcd_block, rows varying fastest; ids past a smaller block exit.
    const int j = (int)(blockIdx.x >> 3);
    const XcdBlock b = xcd_block(row_tiles, col_tiles, (int)(blockIdx.x & 7));
    if (j >= b.nr * b.nc) return;
    const TilePart whole{0, 1, nullptr, nullptr};
    prefill_tile<GATED>(L, M, (b.r0 + j % b.nr) * kPT, (b.c0 + j / b.nr) * kPT, 0, 2 * L.G, whole, sxa, sxb, sxc,
                        sxd);
}

// Several linears in one launch: workgroup i takes entry i of wg_map
// (linear | tile << 16, tiles numbered row-major, or all ones: no tile); the
// host orders the map longest-K first and XCD-aware.  part_map[i] is
// part | nparts << 4 | slot << 8: the tile's K-stages are cut into nparts
// pieces of whole groups, this workgroup takes piece `part`, and a cut tile
// uses workspace block `slot` (kPlanParts x 256 x 256 floats) and counter `slot`.
__global__ __launch_bounds__(kPThreads) void prefill_plan_kernel(const LinearDev* __restrict__ list,
                                                                  const uint32_t* __restrict__ wg_map,
                                                                  const uint32_t* __restrict__ part_map,
                                                                  float* __restrict__ ws,
                                                                  uint32_t* __restrict__ counters, int M) {
    __shared__ __attribute__((aligned(1024))) uint16_t sxa[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxb[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxc[kPXBytes / 2];
    __shared__ __attribute__((aligned(1024))) uint16_t sxd[kPXBytes / 2];
    const uint32_t e = gptr<uint32_t>(wg_map)[blockIdx.x];
    if (e == 0xFFFFFFFFu) return;   // padding entry: no tile
    LinearDev L;
    {
        static_assert(sizeof(LinearDev) % 4 == 0, "descriptor copy");
        const EXQ_GLOBAL uint32_t* src = gptr<uint32_t>(list + (e & 0xFFFFu));
        uint32_t* dst = reinterpret_cast<uint32_t*>(&L);
#pragma unroll
        for (int k = 0; k < (int)(sizeof(LinearDev) / 4); ++k)
            dst[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)src[k]);   // uniform: SGPRs
    }
    const int col_tiles = (L.N + kPT - 1) / kPT, t = (int)(e >> 16);
    const uint32_t pm = gptr<uint32_t>(part_map)[blockIdx.x];
    const int part = (int)(pm & 15u), nparts = (int)((pm >> 4) & 15u);
    const uint32_t slot = pm >> 8;
    // Piece `part` of nparts: groups [G part / nparts, G (part + 1) / nparts).
    const int lo = 2 * (L.G * part / nparts), hi = 2 * (L.G * (part + 1) / nparts);
    const TilePart tp{part, nparts, ws + (size_t)slot * kPlanParts * 256 * kPThreads, counters + slot};
    prefill_tile<false>(L, M, (t / col_tiles) * kPT, (t % col_tiles) * kPT, lo, hi, tp, sxa, sxb, sxc, sxd);
}

}  // namespace
}  // namespace exq

using namespace exq;

namespace {

template <bool GATED>
exq_status prefill_launch_dev(const LinearDev& d, int M, hipStream_t stream) {
    // Offsets into one tile's rows of x are 32-bit: 2 * 256 * K bytes must stay below 2^31.
    if ((size_t)2 * kPT * (size_t)d.K >= (size_t)kBufOOB)
        return fail(EXQ_ERR_UNSUPPORTED, "K=%d is too large for the prefill kernel", d.K);
    const long row_tiles = (M + kPT - 1) / kPT, col_tiles = (d.N + kPT - 1) / kPT;
    if (row_tiles * col_tiles > INT_MAX) return fail(EXQ_ERR_UNSUPPORTED, "M=%d gives too many tiles", M);
    long per_xcd = 0;   // the largest block: 8 of them cover every tile
    for (int blk = 0; blk < 8; ++blk) {
        const XcdBlock b = xcd_block((int)row_tiles, (int)col_tiles, blk);
        per_xcd = std::max(per_xcd, (long)b.nr * b.nc);
    }
    hipLaunchKernelGGL(prefill_kernel<GATED>, dim3((unsigned)(8 * per_xcd)), dim3(kPThreads), 0, stream, d, M,
                       (int)row_tiles, (int)col_tiles);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : fail(EXQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
}

}  // namespace

exq_status exq_prefill_launch(const exq_layer* L, const void* x, int M, void* y, hipStream_t stream) {
    return prefill_launch_dev<false>(linear_dev(L, x, y), M, stream);
}

// A descriptor whose fp16 scales the caller provides (the allocation-free entry point).
exq_status exq_prefill_launch_desc(const LinearDev& d, int M, hipStream_t stream) {
    return prefill_launch_dev<false>(d, M, stream);
}

// h holds the gate product; writes SiLU(h) * (x W_up^T) over it.
exq_status exq_prefill_launch_gated(const exq_layer* U, const void* x, int M, void* h, hipStream_t stream) {
    return prefill_launch_dev<true>(linear_dev(U, x, h), M, stream);
}

// Tiles of one linear in a prefill plan (0 if the linear cannot be planned).
int exq_prefill_tiles(const exq_layer* L, int M) {
    if ((size_t)2 * kPT * (size_t)L->K >= (size_t)kBufOOB) return 0;
    const long t = (long)((M + kPT - 1) / kPT) * ((L->N + kPT - 1) / kPT);
    return t < 65536 ? (int)t : 0;
}

exq_status exq_prefill_plan_launch(const LinearDev* d_list, const uint32_t* d_wg_map, const uint32_t* d_part_map,
                                   float* d_ws, uint32_t* d_counters, int total_wgs, int M, hipStream_t stream) {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3((unsigned)total_wgs), dim3(kPThreads), 0, stream, d_list, d_wg_map,
                       d_part_map, d_ws, d_counters, M);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? EXQ_OK : fail(EXQ_ERR_HIP, "prefill plan launch: %s", hipGetErrorString(e));
}
