// Internal declarations shared by the host (HIP-free) and device halves of libexq.
#pragma once

#include <atomic>
#include <cstddef>
#include <mutex>
#include <cstdint>
#include <vector>

#include "../../include/exq.h"

namespace exq {

constexpr int kGroup = 128;     // input channels per group
constexpr int kTileCols = 16;   // output columns per decode workgroup (lane % 16)
constexpr int kWaves = 8;       // waves per decode workgroup, each takes a share of the groups
constexpr int kMaxDecodeM = 16; // largest M served by the decode kernel
constexpr int kTuneMaxM = 64;   // row counts a layer keeps a tuned kernel choice for

// Prefill tiles of one linear by XCD: block b of 8 is rows [r0, r0 + nr) x
// columns [c0, c0 + nc) of the (row tiles x column tiles) grid, from 2 row
// groups x 4 column groups (1 x 8 for a single row tile).  Tiles of one
// block run on one XCD, rows varying fastest, and share W and x in its L2.
struct XcdBlock {
    int r0, nr, c0, nc;
};
constexpr XcdBlock xcd_block(int row_tiles, int col_tiles, int b) {
    const int rgs = row_tiles < 2 ? 1 : 2, cgs = 8 / rgs, rg = b / cgs, cg = b % cgs;
    const int r0 = row_tiles * rg / rgs, r1 = row_tiles * (rg + 1) / rgs;
    const int c0 = col_tiles * cg / cgs, c1 = col_tiles * (cg + 1) / cgs;
    return XcdBlock{r0, r1 - r0, c0, c1 - c0};
}

// Most pieces a prefill plan cuts one tile into along K (to fill the last
// round of an XCD's queue).
constexpr int kPlanParts = 4;

// Kernel choices of exq_gemm (a layer's tuned entry for M, 0 = the default rule).
enum Variant : uint8_t { kVarDefault = 0, kVarDecode16 = 1, kVarDecode64 = 2, kVarPrefill = 3, kNumVariants = 4 };

// Records a message for exq_last_error() and returns `s`.
exq_status fail(exq_status s, const char* fmt, ...);

bool width_supported(int b);

// Validation shared by every entry point that describes a layer.
exq_status check_layer_shape(int K, int N, int group_size, const uint8_t* widths);

// How the kWaves waves of a decode workgroup share a layer's groups.  All
// groups are sorted by (width, index) and cut into kWaves contiguous chunks
// of balanced decode instruction counts, so each wave streams one or two runs
// of equal-width groups with a fixed number of loads per group.
//   order[i] = g | (P_g << 16) in that sorted order;
//   bounds[w] .. bounds[w+1] is wave w's chunk of `order`;
//   runs[w*6 + i] counts its groups of width kWidthOrder[i].
constexpr int kNumWidths = 6;
constexpr int kWidthOrder[kNumWidths] = {2, 3, 4, 5, 6, 8};

struct WavePlan {
    std::vector<uint32_t> order;
    std::vector<uint16_t> bounds;
    std::vector<uint16_t> runs;
};

WavePlan plan_waves(int K, const uint8_t* widths);

// Per-group metadata word read by the kernels: (P_g << 4) | b_g.
std::vector<uint32_t> group_meta(int K, const uint8_t* widths);

}  // namespace exq

// A packed layer resident in device memory (the exq_layer_t handle).
struct exq_layer {
    int K, N, G;
    std::vector<uint8_t> widths;
    const void* qweight;      // borrowed
    const void* scales;       // borrowed fp16 [G][N]; for quantized scales the owned expansion, once made
    bool qs = false;          // quantized group scales (4-bit codes + column references)
    const void* qscale = nullptr;     // borrowed 4-bit codes [G][N/2]
    const void* ref = nullptr;        // borrowed fp16 [N]
    // fp16 expansion of the quantized scales for the prefill and dequant
    // kernels, made on the first call that needs it (ensure_scales).
    std::atomic<uint16_t*> d_scales_own{nullptr};
    std::mutex expand_mu;
    exq::WavePlan plan;
    uint32_t* d_meta = nullptr;
    uint32_t* d_order = nullptr;
    uint16_t* d_bounds = nullptr;
    uint16_t* d_runs = nullptr;
    // Kernel choice per row count M (0 = default rule), set by exq_autotune or
    // exq_set_variant; read without locking by exq_gemm.
    std::atomic<uint8_t> tuned[exq::kTuneMaxM + 1] = {};
};
