// Internal interface between the C ABI (sgmv_api.cpp) and the kernel
// launchers (sgmv_kernels.hip): the kernels' argument blocks and the
// launchers. Not installed; callers use include/sgmv.h. Sizes and workspace
// layouts are in sgmv_layout.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sgmv_layout.h"

namespace sgmv {

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

// Bounded waits: how many times a waiting workgroup polls before it gives
// up, and where it reports that it did. `status` is NULL for a call without
// a workspace (such a call has no cross-workgroup wait). A workgroup that
// finds the status non-zero when it starts does nothing.
struct WaitCtl {
    uint32_t *status;
    uint32_t limit;
};
uint32_t wait_limit();
uint32_t set_wait_limit(uint32_t polls);

struct LayerProj {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    uint32_t *tile_counters, *split_counters;
    float *Vws, *Vpairs, *partials;
    int num_adapters, d_in, d_out;
    int ntiles_g, ntiles_m, num_tiles, num_units, ks;
    int base;   // first workgroup id of the projection's region (a multiple of 8)
    int items;  // items of its own fused launch
};

struct LayerArgs {
    LayerProj p[kMaxProjections];
    int num_projections;
    WaitCtl wc;  // one status word for the whole call: the first projection's header
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
hipError_t launch_fused_noalloc(FusedArgs a, hipStream_t stream);

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream);
hipError_t launch_fused(const FusedArgs &a, hipStream_t stream);
hipError_t launch_fused_layer(const LayerCall &a, hipStream_t stream);
hipError_t launch_stream_probe(const void *src, size_t vecs, uint32_t *sink, int num_blocks, hipStream_t stream);
hipError_t launch_set_slot(uint64_t *A_ptrs, uint64_t *B_ptrs, int slot, uint64_t a, uint64_t b,
                           hipStream_t stream);

}  // namespace sgmv
