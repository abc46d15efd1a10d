// Internal interface between the C ABI (sgmv_api.cpp) and the kernel
// launchers (sgmv_kernels.hip). Not installed; callers use include/sgmv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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

// Workspace of the fused kernel: two counters per segment (vector-path shrink
// workgroups arrived, expand workgroups departed), two per MFMA row tile,
// then V (M x r fp32). Every launch leaves all of it zero.
constexpr int kFusedTileRows = 64;

struct FusedLayout {
    size_t seg_counters, tile_counters, v, total;
    int tiles;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline FusedLayout fused_layout(int num_segments, int M, int r) {
    FusedLayout L;
    L.tiles = (M + kFusedTileRows - 1) / kFusedTileRows;
    L.seg_counters = 0;
    L.tile_counters = 2 * sizeof(uint32_t) * (size_t)num_segments;
    L.v = align256(L.tile_counters + 2 * sizeof(uint32_t) * (size_t)L.tiles);
    L.total = align256(L.v + sizeof(float) * (size_t)M * (size_t)r);
    return L;
}

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t stream);
hipError_t launch_expand(const ExpandArgs &a, hipStream_t stream);
hipError_t launch_fused(const FusedArgs &a, hipStream_t stream);

}  // namespace sgmv
