// Internal declarations shared by the host (HIP-free) and device halves of libexq.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/exq.h"

namespace exq {

constexpr int kGroup = 128;     // input channels per group
constexpr int kTileCols = 64;   // output columns per workgroup tile (one per lane)
constexpr int kWaves = 4;       // waves per decode workgroup, each takes a slice of K
constexpr int kMaxDecodeM = 16; // largest M served by the decode kernel
constexpr int kMaxSplitGroups = 1024;

// Records a message for exq_last_error() and returns `s`.
exq_status fail(exq_status s, const char* fmt, ...);

bool width_supported(int b);

// Validation shared by every entry point that describes a layer.
exq_status check_layer_shape(int K, int N, int group_size, const uint8_t* widths);

// Split of a layer's K range: S workgroups per column tile, each of which
// gives its kWaves waves contiguous, byte-balanced runs of groups.
// bounds has S*kWaves + 1 entries; run (s, w) = [bounds[s*kWaves+w], bounds[s*kWaves+w+1]).
struct SplitPlan {
    int S = 1;
    std::vector<uint16_t> bounds;
    int max_split_groups = 0;   // largest number of groups in one split
};

SplitPlan plan_splits(int K, int N, const uint8_t* widths, int forced_splits);

// Per-group metadata word read by the kernels: (P_g << 4) | b_g.
std::vector<uint32_t> group_meta(int K, const uint8_t* widths);

}  // namespace exq
