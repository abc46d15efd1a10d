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

constexpr int kTileRows64 = 64;    // rows of an MFMA shrink or expand tile (and of a fused handoff)
constexpr int kMacroSteps = 128;   // d_in elements per MFMA shrink macro step

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

// How many workgroups split d_in for each 64-row MFMA shrink tile: enough for
// about two workgroups per CU over the batch's tiles, at most 8 parts and at
// least four 128-wide macro steps per part. One workgroup streams only a few
// tens of GB/s, so long segments need the whole chip; the cost is a 64 x r
// fp32 partial tile per part, summed by the last part to arrive.
inline int shrink_ksplit(int M, int d_in) {
    const int tiles = (M + kTileRows64 - 1) / kTileRows64;
    const int nmacro = (d_in + kMacroSteps - 1) / kMacroSteps;
    if (tiles == 0) return 1;
    int ks = (512 + tiles - 1) / tiles;
    ks = std::min(ks, 8);
    ks = std::min(ks, nmacro / 4);
    return std::max(ks, 1);
}

// Shrink workspace (bf16 only, when the split is more than one part): the
// header line, then one 128-byte counter line per 64-row tile (its parts arrived, then departed),
// then the tiles' partial results (tile x part x 64 x max(r, 16) fp32: the
// MFMA tile is at least 16 columns wide). Every launch leaves it all zero.
struct ShrinkLayout {
    size_t counters, partials, total;
    int tiles, ks;
};

inline ShrinkLayout shrink_layout(int M, int d_in, int r, int dtype) {
    ShrinkLayout L;
    L.tiles = dtype == kBF16 ? (M + kTileRows64 - 1) / kTileRows64 : 0;
    L.ks = dtype == kBF16 ? shrink_ksplit(M, d_in) : 1;
    L.counters = kHeaderBytes;
    L.partials = align256(L.counters + kCounterStride * sizeof(uint32_t) * (size_t)L.tiles);
    L.total = L.ks > 1 ? align256(L.partials + sizeof(float) * (size_t)L.tiles * L.ks *
                                                   kTileRows64 * (size_t)std::max(r, 16))
                       : 0;
    return L;
}

// Columns of Y one vector-path expand workgroup covers: 256 threads, one
// 16-byte vector each.
inline int vector_col_tiles(int d_out, int dtype) {
    const int cols = 256 * (dtype == kBF16 ? 8 : 4);
    return (d_out + cols - 1) / cols;
}

// Fused workspace: the header line, then one 128-byte line of counters per
// 64-row tile (V
// complete, expand workgroups departed, split shrink parts arrived), so
// that consumers polling one tile do not contend with another's; then V of
// the MFMA path (M x r fp32), the split partials as above, and V of the
// vector path as flagged 64-bit pairs, one M x r copy per vector expand
// column tile (each expand workgroup reads and clears its own copy). Every
// launch leaves it all zero.
struct FusedLayout {
    size_t tile_counters, v, partials, vpairs, total;
    int tiles, ks, copies;
};

inline FusedLayout fused_layout(int M, int d_in, int d_out, int r, int dtype) {
    FusedLayout L;
    L.tiles = dtype == kBF16 ? (M + kTileRows64 - 1) / kTileRows64 : 0;
    L.ks = dtype == kBF16 ? shrink_ksplit(M, d_in) : 1;
    L.copies = vector_col_tiles(d_out, dtype);
    L.tile_counters = kHeaderBytes;
    L.v = align256(L.tile_counters + kCounterStride * sizeof(uint32_t) * (size_t)L.tiles);
    L.partials = align256(L.v + sizeof(float) * (size_t)M * (size_t)r);
    L.vpairs = align256(L.partials + (L.ks > 1 ? sizeof(float) * (size_t)L.tiles * L.ks *
                                                     kTileRows64 * (size_t)std::max(r, 16)
                                               : 0));
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
    uint32_t *tile_counters;
    float *Vws, *Vpairs, *partials;
    int num_adapters, d_in, d_out;
    int ntiles_g, ntiles_m, num_tiles, ks;
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
