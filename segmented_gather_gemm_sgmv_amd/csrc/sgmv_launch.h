// Internal interface between the C ABI (sgmv_api.cpp) and the kernel
// launchers (sgmv_kernels.hip). Not installed; callers use include/sgmv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

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
    const int32_t *rows = nullptr;  // gathered call: token row of each segment row
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
    const int32_t *rows = nullptr;  // scattered call: token row of each segment row
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
    const int32_t *rows = nullptr;  // gathered call: token row of each segment row
};

constexpr int kTileRows64 = 64;    // rows of an MFMA expand tile (and of a fused arrival counter)
constexpr int kShrinkRows16 = 16;  // rows of an MFMA shrink tile

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Every workspace starts with one 256-byte header line. Word 0 is the sticky
// status of the calls that use the workspace (bits of enum sgmv_ws_status in
// sgmv.h); the rest of the line is reserved and stays zero.
constexpr size_t kHeaderBytes = 256;

// Bounded waits: how many times a waiting workgroup polls before it gives
// up, and where it reports that it did. `status` is NULL for a call without
// a workspace (such a call has no cross-workgroup wait). A workgroup that
// finds the status non-zero when it starts does nothing.
struct WaitCtl {
    uint32_t *status;
    uint32_t limit;
};
constexpr uint32_t kDefaultWaitLimit = 1u << 15;
constexpr uint32_t kStatusTimeout = 1;      // a bounded wait gave up
constexpr uint32_t kStatusBadOffsets = 2;   // seg_start decreases somewhere
uint32_t wait_limit();
uint32_t set_wait_limit(uint32_t polls);

constexpr int kCounterStride = 32;  // uint32 words per counter line (128 bytes)

// Which MFMA shrink tile a bf16 launch takes: 16-row tiles for batches of
// up to kSmallBatchRows rows (few tiles: a handful of mid-length segments),
// 64-row tiles above (many tiles: prefill batches), where sharing each A_k
// chunk among 64 rows keeps the L1 traffic near the HBM bytes.
constexpr int kSmallBatchRows = 2048;
inline bool small_tiles(int M) { return M <= kSmallBatchRows; }

// 16-row tiles: how many workgroups split d_in for each work item. Within a
// workgroup the four waves already split d_in, so one workgroup per item is
// the rule: no partial tiles, no combine. Only batches whose items each
// stream more than about 320 KB (X rows plus their columns of A_k: a very
// long d_in) split further, up to 8 parts, keeping about one workgroup per
// CU over the batch and at least 4 steps (one per wave) per part. The cost
// of a split is a partial tile per part, summed in a fixed order by the
// parts themselves.
inline int shrink_ksplit16(int M, int d_in, int r) {
    const int tiles = (M + kShrinkRows16 - 1) / kShrinkRows16;
    if (tiles == 0) return 1;
    const int nsteps = (d_in + 127) / 128;
    const double bytes = 2.0 * d_in * (kShrinkRows16 + std::max(std::min(r, 32), 16));
    int ks = (int)std::ceil(bytes / (320.0 * 1024.0));
    ks = std::min(ks, 8);
    ks = std::min(ks, std::max(1, 256 / tiles));
    ks = std::min(ks, std::max(1, nsteps / 4));
    return std::max(ks, 1);
}

// 64-row tiles: d_in is split over up to 8 workgroups per tile, enough for
// about two workgroups per CU over the batch's tiles, with at least four
// 128-wide macro steps per part. (One workgroup streams only a few tens of
// GB/s, so long segments need the whole chip.)
constexpr int kShrinkTargetWorkgroups = 512;
inline int shrink_ksplit64(int M, int d_in) {
    const int tiles = (M + kTileRows64 - 1) / kTileRows64;
    const int nmacro = (d_in + 127) / 128;
    if (tiles == 0) return 1;
    int ks = (kShrinkTargetWorkgroups + tiles - 1) / tiles;
    ks = std::min(ks, 8);
    ks = std::min(ks, nmacro / 4);
    return std::max(ks, 1);
}

// A 16-row shrink tile meets at most two long segments (each has 16 rows or
// more, and segments do not overlap); each (tile, piece, column group), a
// shrink unit, is a work item of its own, so that a tile that meets two
// segments does not run d_in twice in one workgroup. A 64-row tile is one
// unit (its workgroup takes all of its pieces).
constexpr int kShrinkPieces = 2;

// MFMA shrink items of a launch: one per unit rounded up to a multiple of 8
// (units are dealt to the XCDs in contiguous runs), or one per (unit, part)
// when d_in is split.
__host__ __device__ inline int mfma_shrink_items(int num_units, int ks) {
    return ks == 1 ? (num_units + 7) / 8 * 8 : num_units * ks;
}

// Column groups of a 16-row tile: one workgroup computes at most 32 columns
// of V, so r = 64 takes two.
inline int shrink_groups(int r) { return r > 32 ? r / 32 : 1; }

// The shrink work of a bf16 launch: tile kind, units, parts, and the bytes
// of one part's partial tile (16 or 64 rows x the columns of one workgroup,
// at least 16: the MFMA tile is 16 columns wide, fp32).
struct ShrinkPlan {
    int small, units, ks;
    size_t part_bytes;
};

inline ShrinkPlan shrink_plan(int M, int d_in, int r, int dtype) {
    ShrinkPlan P{1, 0, 1, 0};
    if (dtype != kBF16) return P;
    P.small = small_tiles(M) ? 1 : 0;
    if (P.small) {
        P.units = kShrinkPieces * shrink_groups(r) * ((M + kShrinkRows16 - 1) / kShrinkRows16);
        P.ks = shrink_ksplit16(M, d_in, r);
        P.part_bytes = sizeof(float) * kShrinkRows16 * (size_t)std::max(std::min(r, 32), 16);
    } else {
        P.units = (M + kTileRows64 - 1) / kTileRows64;
        P.ks = shrink_ksplit64(M, d_in);
        P.part_bytes = sizeof(float) * kTileRows64 * (size_t)std::max(r, 16);
    }
    return P;
}

// Shrink workspace (bf16 only, when the split is more than one part): the
// header line, then one 128-byte counter line per shrink unit (its parts
// arrived, then departed), then the units' partial results (unit x part).
// Every launch leaves it all zero.
struct ShrinkLayout {
    size_t counters, partials, total;
    ShrinkPlan plan;
};

inline ShrinkLayout shrink_layout(int M, int d_in, int r, int dtype) {
    ShrinkLayout L;
    L.plan = shrink_plan(M, d_in, r, dtype);
    L.counters = kHeaderBytes;
    L.partials = align256(L.counters + kCounterStride * sizeof(uint32_t) * (size_t)L.plan.units);
    L.total = L.plan.ks > 1 ? align256(L.partials + L.plan.part_bytes * (size_t)L.plan.units * L.plan.ks) : 0;
    return L;
}

// Columns of Y one vector-path expand workgroup covers: 256 threads, one
// 16-byte vector each.
inline int vector_col_tiles(int d_out, int dtype) {
    const int cols = 256 * (dtype == kBF16 ? 8 : 4);
    return (d_out + cols - 1) / cols;
}

// Fused workspace: the header line, then one 128-byte line of counters per
// 64-row expand tile (shrink parts arrived, expand workgroups departed), so
// that consumers polling one tile do not contend with another's; then, when
// d_in is split, one counter line per shrink unit; then V of the MFMA
// path (M x r fp32), the split partials, and V of the vector path as flagged
// 64-bit pairs, one M x r copy per vector expand column tile (each expand
// workgroup reads and clears its own copy). Every launch leaves it all zero.
struct FusedLayout {
    size_t tile_counters, split_counters, v, partials, vpairs, total;
    int tiles, copies;
    ShrinkPlan plan;
};

inline FusedLayout fused_layout(int M, int d_in, int d_out, int r, int dtype) {
    FusedLayout L;
    L.tiles = dtype == kBF16 ? (M + kTileRows64 - 1) / kTileRows64 : 0;
    L.plan = shrink_plan(M, d_in, r, dtype);
    L.copies = vector_col_tiles(d_out, dtype);
    L.tile_counters = kHeaderBytes;
    L.split_counters = align256(L.tile_counters + kCounterStride * sizeof(uint32_t) * (size_t)L.tiles);
    L.v = align256(L.split_counters +
                   (L.plan.ks > 1 ? kCounterStride * sizeof(uint32_t) * (size_t)L.plan.units : 0));
    L.partials = align256(L.v + sizeof(float) * (size_t)M * (size_t)r);
    L.vpairs = align256(L.partials +
                        (L.plan.ks > 1 ? L.plan.part_bytes * (size_t)L.plan.units * L.plan.ks : 0));
    L.total = align256(L.vpairs + sizeof(uint64_t) * (size_t)M * (size_t)r * (size_t)L.copies);
    return L;
}

// Layer-batched fused launch: up to kMaxProjections projections of one batch
// (shared rows, segments, rank, scale and dtype), each with its own X, Y,
// pools and d_in / d_out, in one launch. The descriptors travel in the
// kernel arguments.
constexpr int kMaxProjections = 8;

struct LayerProj {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    uint32_t *tile_counters, *split_counters;
    float *Vws, *Vpairs, *partials;
    int num_adapters, d_in, d_out;
    int ntiles_g, ntiles_m, num_tiles, num_units, ks, small;
    int base;   // first workgroup id of the projection's region (a multiple of 8)
    int items;  // items of its own fused launch
};

struct LayerArgs {
    LayerProj p[kMaxProjections];
    int num_projections;
    WaitCtl wc;  // one status word for the whole call: the first projection's header
};

struct LayerProjIn {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    int num_adapters, d_in, d_out;
};

struct LayerCall {
    LayerProjIn p[kMaxProjections];
    int num_projections;
    const int32_t *seg_start;
    const int32_t *seg_adapter;
    int num_segments, M, r, dtype;
    float scale;
    void *workspace;
    const int32_t *rows = nullptr;  // gathered call: token row of each segment row
};

// A layer call's workspace: each projection's fused workspace, back to back
// at 256-byte aligned offsets, in projection order.
inline size_t layer_workspace_total(const LayerProjIn *p, int num_projections, int num_segments, int M, int r,
                                    int dtype) {
    size_t total = 0;
    for (int q = 0; q < num_projections; ++q)
        total += align256(fused_layout(M, p[q].d_in, p[q].d_out, r, dtype).total);
    return total;
}

// Per-rank entry points, one translation unit each (R = 8, 16, 32, 64).
template <int R>
hipError_t launch_shrink_rank(const ShrinkArgs &a, hipStream_t stream);
template <int R>
hipError_t launch_expand_rank(const ExpandArgs &a, hipStream_t stream);
template <int R>
hipError_t launch_fused_rank(const FusedArgs &a, hipStream_t stream);
template <int R>
hipError_t launch_fused_layer_rank(const LayerCall &a, hipStream_t stream);

// The fused call on the library's own per-device scratch array (a.workspace
// is ignored): for callers that cannot allocate. The batch's fused workspace
// must fit in kScratchBytes.
constexpr size_t kScratchBytes = (size_t)16 << 20;
hipError_t launch_fused_noalloc(FusedArgs a, hipStream_t stream);

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream);
hipError_t launch_fused(const FusedArgs &a, hipStream_t stream);
hipError_t launch_fused_layer(const LayerCall &a, hipStream_t stream);
hipError_t launch_stream_probe(const void *src, size_t vecs, uint32_t *sink, int num_blocks, hipStream_t stream);
hipError_t launch_set_slot(uint64_t *A_ptrs, uint64_t *B_ptrs, int slot, uint64_t a, uint64_t b,
                           hipStream_t stream);

}  // namespace sgmv
