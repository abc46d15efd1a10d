// Internal interface between the C ABI (sgmv_api.cpp) and the kernel
// launchers (sgmv_kernels.hip). Not installed; callers use include/sgmv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace sgmv {

enum DType { kF32 = 0, kBF16 = 1 };

struct ShrinkArgs {
    float *V;
    const void *X;
    const uint64_t *A_ptrs;
    int num_adapters;
    const int32_t *seg_start;
    const int32_t *seg_adapter;
    int num_segments, M, d_in, r, dtype;
    void *workspace;
};

struct ExpandArgs {
    void *Y;
    const float *V;
    const uint64_t *B_ptrs;
    int num_adapters;
    const int32_t *seg_start;
    const int32_t *seg_adapter;
    int num_segments, M, d_out, r, dtype;
    float scale;
};

struct FusedArgs {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    int num_adapters;
    const int32_t *seg_start;
    const int32_t *seg_adapter;
    int num_segments, M, d_in, d_out, r, dtype;
    float scale;
    void *workspace;
};

constexpr int kSubTileRows = 16;   // rows of an MFMA shrink tile
constexpr int kTileRows64 = 64;    // rows of an MFMA expand tile (and of a fused handoff)
constexpr int kMacroSteps = 128;   // d_in elements per MFMA shrink macro step

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// How many workgroups split d_in for each 16-row MFMA shrink tile. One
// workgroup streams only about 100 GB/s, so a batch with very few long rows
// (at most 8 tiles of 16) spreads each tile over up to 4 workgroups, each
// keeping at least four 128-wide macro steps per wave; larger batches
// already have enough tiles to fill the chip and are not split.
inline int shrink_ksplit(int M, int d_in) {
    const int subtiles = (M + kSubTileRows - 1) / kSubTileRows;
    const int nmacro = (d_in + kMacroSteps - 1) / kMacroSteps;
    if (subtiles > 8) return 1;
    return std::max(1, std::min(4, nmacro / 16));
}

// Shrink workspace (bf16 only, when the split is more than one part): one
// arrival counter per 16-row tile, then the tiles' partial results
// (tile x part x 16 x r fp32). Every launch leaves it all zero.
struct ShrinkLayout {
    size_t counters, partials, total;
    int subtiles, ks;
};

inline ShrinkLayout shrink_layout(int M, int d_in, int r, int dtype) {
    ShrinkLayout L;
    L.subtiles = dtype == kBF16 ? (M + kSubTileRows - 1) / kSubTileRows : 0;
    L.ks = dtype == kBF16 ? shrink_ksplit(M, d_in) : 1;
    L.counters = 0;
    L.partials = align256(sizeof(uint32_t) * (size_t)L.subtiles);
    L.total = L.ks > 1 ? align256(L.partials + sizeof(float) * (size_t)L.subtiles * L.ks *
                                                   kSubTileRows * (size_t)r)
                       : 0;
    return L;
}

// Fused workspace: one 128-byte line of counters per segment (expand
// workgroups departed) and per 64-row tile (MFMA shrink tiles arrived,
// expand workgroups departed), so that consumers polling one tile do not
// contend with another's; then one counter per 16-row shrink tile, V of the
// MFMA path (M x r fp32), the split partials as above, and V of the vector
// path as M x r flagged 64-bit pairs. Every launch leaves it all zero.
constexpr int kCounterStride = 32;  // uint32 words per counter line
struct FusedLayout {
    size_t seg_counters, tile_counters, sub_counters, v, partials, vpairs, total;
    int tiles, subtiles, ks;
};

inline FusedLayout fused_layout(int num_segments, int M, int d_in, int r, int dtype) {
    FusedLayout L;
    L.tiles = dtype == kBF16 ? (M + kTileRows64 - 1) / kTileRows64 : 0;
    L.subtiles = dtype == kBF16 ? (M + kSubTileRows - 1) / kSubTileRows : 0;
    L.ks = dtype == kBF16 ? shrink_ksplit(M, d_in) : 1;
    L.seg_counters = 0;
    L.tile_counters = kCounterStride * sizeof(uint32_t) * (size_t)num_segments;
    L.sub_counters = L.tile_counters + kCounterStride * sizeof(uint32_t) * (size_t)L.tiles;
    L.v = align256(L.sub_counters + sizeof(uint32_t) * (size_t)L.subtiles);
    L.partials = align256(L.v + sizeof(float) * (size_t)M * (size_t)r);
    L.vpairs = align256(L.partials + (L.ks > 1 ? sizeof(float) * (size_t)L.subtiles * L.ks *
                                                     kSubTileRows * (size_t)r
                                               : 0));
    L.total = align256(L.vpairs + sizeof(uint64_t) * (size_t)M * (size_t)r);
    return L;
}

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream);
hipError_t launch_fused(const FusedArgs &a, hipStream_t stream);

}  // namespace sgmv
