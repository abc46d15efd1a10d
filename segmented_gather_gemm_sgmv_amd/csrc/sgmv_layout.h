// Launch geometry and workspace layouts of the SGMV kernels: plain host
// arithmetic, shared by the kernel launchers, the C ABI's size queries and
// checks, and the kernels themselves (the few functions marked
// SGMV_HOST_DEVICE). Free of HIP types, so that the host-only part of the
// library also builds with a host compiler alone (the sanitizer build).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#ifdef __HIPCC__
#define SGMV_HOST_DEVICE __host__ __device__
#else
#define SGMV_HOST_DEVICE
#endif

namespace sgmv {

enum DType { kF32 = 0, kBF16 = 1 };

constexpr int kTileRows64 = 64;    // rows of an MFMA expand tile (and of a fused arrival counter)
constexpr int kShrinkRows16 = 16;  // rows of an MFMA shrink tile

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ceil(a / b) for a >= 0 and b > 0, for every int a (no overflow).
inline int ceil_div(int a, int b) { return (int)(((int64_t)a + b - 1) / b); }

constexpr int kLaunchThreads = 256;  // threads per workgroup of every SGMV kernel (4 waves)
constexpr int kExpandCols = 128;     // d_out columns per MFMA expand tile

// Every workspace starts with one 256-byte header line. Word 0 is the sticky
// status of the calls that use the workspace (bits of enum sgmv_ws_status in
// sgmv.h); the rest of the line is reserved and stays zero.
constexpr size_t kHeaderBytes = 256;

constexpr uint32_t kDefaultWaitLimit = 1u << 15;
constexpr uint32_t kStatusTimeout = 1;      // a bounded wait gave up
constexpr uint32_t kStatusBadOffsets = 2;   // seg_start decreases somewhere

constexpr int kCounterStride = 32;  // uint32 words per counter line (128 bytes)

// Which MFMA shrink tile a bf16 launch takes: 16-row tiles for batches of
// few tiles (a handful of mid-length segments), 64-row tiles for larger
// ones (prefill batches), where sharing each A_k chunk among 64 rows keeps
// the L1 traffic near the HBM bytes. The bound is where the two measured
// even on MI355X (fused calls of 2 to 16 long segments): about 12 tiles of
// 64 rows at r = 64, where a 16-row unit re-reads its 64 rank rows of A_k
// for every 16 rows, and 16 tiles at smaller ranks.
inline int small_batch_rows(int r) { return r >= 64 ? 768 : 1024; }
inline bool small_tiles(int M, int r) { return M <= small_batch_rows(r); }

// 16-row tiles: how many workgroups split d_in for each work item. Within a
// workgroup the four waves already split d_in, so one workgroup per item is
// the rule: no partial tiles, no combine. Only batches whose items each
// stream more than about 320 KB (X rows plus their columns of A_k: a very
// long d_in) split further, up to 8 parts, keeping about one workgroup per
// CU over the batch and at least 4 steps (one per wave) per part. The cost
// of a split is a partial tile per part, summed in a fixed order by the
// parts themselves.
inline int shrink_ksplit16(int M, int d_in, int r) {
    const int tiles = ceil_div(M, kShrinkRows16);
    if (tiles == 0) return 1;
    const int nsteps = ceil_div(d_in, 128);
    const double bytes = 2.0 * d_in * (kShrinkRows16 + std::max(std::min(r, 32), 16));
    int ks = (int)std::ceil(bytes / (320.0 * 1024.0));
    ks = std::min(ks, 8);
    ks = std::min(ks, std::max(1, 256 / tiles));
    ks = std::min(ks, std::max(1, nsteps / 4));
    return std::max(ks, 1);
}

// 64-row tiles: d_in is split over up to 8 workgroups per tile, enough for
// about `target` workgroups over the batch's tiles, with at least four
// 128-wide macro steps per part. (One workgroup streams only a few tens of
// GB/s, so long segments need the whole chip.) A shrink launch aims at two
// workgroups per CU; the fused launch at fewer, which leaves slots to expand
// workgroups, whose Y and B loads are then in flight while the shrink runs.
constexpr int kShrinkTargetWorkgroups = 512;
constexpr int kFusedShrinkTargetWorkgroups = 204;
inline int shrink_ksplit64(int M, int d_in, int target = kShrinkTargetWorkgroups) {
    const int tiles = ceil_div(M, kTileRows64);
    const int nmacro = ceil_div(d_in, 128);
    if (tiles == 0) return 1;
    int ks = (target + tiles - 1) / tiles;
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
SGMV_HOST_DEVICE inline int mfma_shrink_items(int num_units, int ks) {
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
    P.small = small_tiles(M, r) ? 1 : 0;
    if (P.small) {
        P.units = kShrinkPieces * shrink_groups(r) * ceil_div(M, kShrinkRows16);
        P.ks = shrink_ksplit16(M, d_in, r);
        P.part_bytes = sizeof(float) * kShrinkRows16 * (size_t)std::max(std::min(r, 32), 16);
    } else {
        P.units = ceil_div(M, kTileRows64);
        P.ks = shrink_ksplit64(M, d_in);
        P.part_bytes = sizeof(float) * kTileRows64 * (size_t)std::max(r, 16);
    }
    return P;
}

// The shrink work of a fused launch: as in a shrink launch, with the fused
// launch's split of d_in for 64-row tiles (never more parts than a shrink
// launch takes, so a shrink launch's item count bounds it).
inline ShrinkPlan fused_shrink_plan(int M, int d_in, int r, int dtype) {
    ShrinkPlan P = shrink_plan(M, d_in, r, dtype);
    if (P.units && !P.small) P.ks = shrink_ksplit64(M, d_in, kFusedShrinkTargetWorkgroups);
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
    return ceil_div(d_out, kLaunchThreads * (dtype == kBF16 ? 8 : 4));
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
    L.tiles = dtype == kBF16 ? ceil_div(M, kTileRows64) : 0;
    L.plan = fused_shrink_plan(M, d_in, r, dtype);
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

struct LayerProjIn {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    int num_adapters, d_in, d_out;
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

// Workgroups of the largest launch one projection of a call makes (the
// fused launch: vector shrink, MFMA shrink, vector expand and MFMA expand
// items, each region padded to a multiple of 8), counted in 64 bits. The
// kernels number their workgroups with int, and one dispatch holds at most
// 2^32 work-items, 2^24 workgroups: calls beyond kMaxWorkgroups are refused.
constexpr int64_t kMaxWorkgroups = (int64_t)1 << 24;
inline int64_t launch_workgroups(int M, int num_segments, int d_in, int d_out, int r, int dtype) {
    auto pad8 = [](int64_t n) { return (n + 7) / 8 * 8; };
    const ShrinkPlan P = shrink_plan(M, d_in, r, dtype);
    const int64_t mfma_shrink = P.units == 0 ? 0 : P.ks == 1 ? pad8(P.units) : (int64_t)P.units * P.ks;
    const int64_t tiles = dtype == kBF16 ? ceil_div(M, kTileRows64) : 0;
    return pad8(num_segments) * (r / 4) + mfma_shrink + (int64_t)num_segments * vector_col_tiles(d_out, dtype) +
           pad8(tiles * ceil_div(d_out, kExpandCols));
}

constexpr size_t kScratchBytes = (size_t)16 << 20;  // the no-allocation entry point's scratch array

}  // namespace sgmv
