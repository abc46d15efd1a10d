// The launching entry points of the C ABI declared in include/sgmv.h:
// argument checks, then dispatch to the gfx950 kernels. The host-only entry
// points (size queries, metadata helpers) are in sgmv_host.cpp.
#include "sgmv.h"

#include <hip/hip_runtime.h>

#include "sgmv_checks.h"
#include "sgmv_launch.h"

using namespace sgmv::abi;

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? SGMV_OK : SGMV_ERR_HIP; }

int check_workspace(const void *workspace, size_t workspace_bytes, size_t need) {
    if (need == 0) return SGMV_OK;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
        return SGMV_ERR_WORKSPACE;
    return SGMV_OK;
}

// The checks and launches shared by the contiguous calls (rows == NULL,
// gathered == false) and the gathered ones (rows required when M > 0).
int shrink_call(float *V, const void *X, const int32_t *rows, bool gathered, const uint64_t *A_ptrs,
                int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                int32_t num_segments, int32_t M, int32_t d_in, int32_t r, int32_t dtype, void *workspace,
                size_t workspace_bytes, void *stream) {
    int st = check_common(num_adapters, num_segments, M, r, dtype);
    if (st != SGMV_OK) return st;
    st = check_sizes(M, num_segments, d_in, 8, r, dtype);
    if (st != SGMV_OK) return st;
    if (M == 0 || num_segments == 0) return SGMV_OK;
    if (!V || !X || !A_ptrs || !seg_start || !seg_adapter || (gathered && !rows)) return SGMV_ERR_NULL;
    if (!aligned16(V) || !aligned16(X)) return SGMV_ERR_ALIGN;
    st = check_workspace(workspace, workspace_bytes, sgmv::shrink_layout(M, d_in, r, dtype).total);
    if (st != SGMV_OK) return st;
    sgmv::ShrinkArgs a{V, X, A_ptrs, num_adapters, seg_start, seg_adapter,
                       num_segments, M, d_in, r, dtype, workspace, gathered ? rows : nullptr};
    return hip_status(sgmv::launch_shrink(a, static_cast<hipStream_t>(stream)));
}

int expand_call(void *Y, const float *V, const int32_t *rows, bool gathered, const uint64_t *B_ptrs,
                int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                int32_t num_segments, int32_t M, int32_t d_out, int32_t r, float alpha, int32_t dtype,
                void *stream) {
    int st = check_common(num_adapters, num_segments, M, r, dtype);
    if (st != SGMV_OK) return st;
    st = check_sizes(M, num_segments, 8, d_out, r, dtype);
    if (st != SGMV_OK) return st;
    if (M == 0 || num_segments == 0) return SGMV_OK;
    if (!Y || !V || !B_ptrs || !seg_start || !seg_adapter || (gathered && !rows)) return SGMV_ERR_NULL;
    if (!aligned16(Y) || !aligned16(V)) return SGMV_ERR_ALIGN;
    sgmv::ExpandArgs a{Y, V, B_ptrs, num_adapters, seg_start, seg_adapter, num_segments,
                       M, d_out, r, dtype, alpha / (float)r, gathered ? rows : nullptr};
    return hip_status(sgmv::launch_expand(a, static_cast<hipStream_t>(stream)));
}

int fused_call(void *Y, const void *X, const int32_t *rows, bool gathered, const uint64_t *A_ptrs,
               const uint64_t *B_ptrs, int32_t num_adapters, const int32_t *seg_start,
               const int32_t *seg_adapter, int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out,
               int32_t r, float alpha, int32_t dtype, void *workspace, size_t workspace_bytes,
               void *stream) {
    int st = check_common(num_adapters, num_segments, M, r, dtype);
    if (st != SGMV_OK) return st;
    st = check_sizes(M, num_segments, d_in, d_out, r, dtype);
    if (st != SGMV_OK) return st;
    if (M == 0 || num_segments == 0) return SGMV_OK;
    if (!Y || !X || !A_ptrs || !B_ptrs || !seg_start || !seg_adapter || (gathered && !rows))
        return SGMV_ERR_NULL;
    if (!aligned16(Y) || !aligned16(X)) return SGMV_ERR_ALIGN;
    st = check_workspace(workspace, workspace_bytes,
                         sgmv::fused_layout(M, d_in, d_out, r, dtype).total);
    if (st != SGMV_OK) return st;
    sgmv::FusedArgs a{Y, X, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter,
                      num_segments, M, d_in, d_out, r, dtype, alpha / (float)r, workspace,
                      gathered ? rows : nullptr};
    return hip_status(sgmv::launch_fused(a, static_cast<hipStream_t>(stream)));
}

// sgmv_fused's checks, then the launch on the library's scratch array.
int fused_noalloc_call(void *Y, const void *X, const uint64_t *A_ptrs, const uint64_t *B_ptrs,
                       int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                       int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out, int32_t r, float alpha,
                       int32_t dtype, void *stream) {
    int st = check_common(num_adapters, num_segments, M, r, dtype);
    if (st != SGMV_OK) return st;
    st = check_sizes(M, num_segments, d_in, d_out, r, dtype);
    if (st != SGMV_OK) return st;
    if (M == 0 || num_segments == 0) return SGMV_OK;
    if (!Y || !X || !A_ptrs || !B_ptrs || !seg_start || !seg_adapter) return SGMV_ERR_NULL;
    if (!aligned16(Y) || !aligned16(X)) return SGMV_ERR_ALIGN;
    if (sgmv::fused_layout(M, d_in, d_out, r, dtype).total > sgmv::kScratchBytes) return SGMV_ERR_SCRATCH;
    sgmv::FusedArgs a{Y, X, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter,
                      num_segments, M, d_in, d_out, r, dtype, alpha / (float)r, nullptr, nullptr};
    return hip_status(sgmv::launch_fused_noalloc(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int sgmv_shrink(float *V, const void *X, const uint64_t *A_ptrs, int32_t num_adapters,
                const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                int32_t M, int32_t d_in, int32_t r, int32_t dtype, void *workspace,
                size_t workspace_bytes, void *stream) {
    return shrink_call(V, X, nullptr, false, A_ptrs, num_adapters, seg_start, seg_adapter, num_segments,
                       M, d_in, r, dtype, workspace, workspace_bytes, stream);
}

int sgmv_expand(void *Y, const float *V, const uint64_t *B_ptrs, int32_t num_adapters,
                const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                int32_t M, int32_t d_out, int32_t r, float alpha, int32_t dtype, void *stream) {
    return expand_call(Y, V, nullptr, false, B_ptrs, num_adapters, seg_start, seg_adapter, num_segments,
                       M, d_out, r, alpha, dtype, stream);
}

int sgmv_fused(void *Y, const void *X, const uint64_t *A_ptrs, const uint64_t *B_ptrs,
               int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
               int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out, int32_t r,
               float alpha, int32_t dtype, void *workspace, size_t workspace_bytes,
               void *stream) {
    return fused_call(Y, X, nullptr, false, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter,
                      num_segments, M, d_in, d_out, r, alpha, dtype, workspace, workspace_bytes, stream);
}

int sgmv_fused_noalloc(void *Y, const void *X, const uint64_t *A_ptrs, const uint64_t *B_ptrs,
                       int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                       int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out, int32_t r, float alpha,
                       int32_t dtype, void *stream) {
    return fused_noalloc_call(Y, X, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter, num_segments, M, d_in,
                              d_out, r, alpha, dtype, stream);
}

int sgmv_shrink_gather(float *V, const void *X, const int32_t *rows, const uint64_t *A_ptrs,
                       int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                       int32_t num_segments, int32_t M, int32_t d_in, int32_t r, int32_t dtype,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return shrink_call(V, X, rows, true, A_ptrs, num_adapters, seg_start, seg_adapter, num_segments, M,
                       d_in, r, dtype, workspace, workspace_bytes, stream);
}

int sgmv_expand_scatter(void *Y, const float *V, const int32_t *rows, const uint64_t *B_ptrs,
                        int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                        int32_t num_segments, int32_t M, int32_t d_out, int32_t r, float alpha,
                        int32_t dtype, void *stream) {
    return expand_call(Y, V, rows, true, B_ptrs, num_adapters, seg_start, seg_adapter, num_segments, M,
                       d_out, r, alpha, dtype, stream);
}

int sgmv_fused_gather(void *Y, const void *X, const int32_t *rows, const uint64_t *A_ptrs,
                      const uint64_t *B_ptrs, int32_t num_adapters, const int32_t *seg_start,
                      const int32_t *seg_adapter, int32_t num_segments, int32_t M, int32_t d_in,
                      int32_t d_out, int32_t r, float alpha, int32_t dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return fused_call(Y, X, rows, true, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter,
                      num_segments, M, d_in, d_out, r, alpha, dtype, workspace, workspace_bytes, stream);
}

int sgmv_fused_layer(const sgmv_projection *projections, int32_t num_projections, const int32_t *rows,
                     const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments, int32_t M,
                     int32_t r, float alpha, int32_t dtype, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (!valid_dtype(dtype)) return SGMV_ERR_DTYPE;
    if (!valid_rank(r)) return SGMV_ERR_RANK;
    sgmv::LayerCall a{};
    int st = layer_inputs(projections, num_projections, num_segments, M, r, dtype, a.p);
    if (st != SGMV_OK) return st;
    if (M < 0 || num_segments < 0) return SGMV_ERR_SHAPE;
    if (num_projections == 0 || M == 0 || num_segments == 0) return SGMV_OK;
    if (!seg_start || !seg_adapter) return SGMV_ERR_NULL;
    for (int32_t q = 0; q < num_projections; ++q) {
        const sgmv::LayerProjIn &p = a.p[q];
        if (!p.Y || !p.X || !p.A_ptrs || !p.B_ptrs) return SGMV_ERR_NULL;
        if (!aligned16(p.Y) || !aligned16(p.X)) return SGMV_ERR_ALIGN;
    }
    st = check_workspace(workspace, workspace_bytes,
                         sgmv::layer_workspace_total(a.p, num_projections, num_segments, M, r, dtype));
    if (st != SGMV_OK) return st;
    a.num_projections = num_projections;
    a.seg_start = seg_start;
    a.seg_adapter = seg_adapter;
    a.num_segments = num_segments;
    a.M = M;
    a.r = r;
    a.dtype = dtype;
    a.scale = alpha / (float)r;
    a.workspace = workspace;
    a.rows = rows;
    return hip_status(sgmv::launch_fused_layer(a, static_cast<hipStream_t>(stream)));
}


int sgmv_admit_adapter(void *A_slot, void *B_slot, const void *A_host, const void *B_host,
                       size_t A_bytes, size_t B_bytes, uint64_t *A_ptrs, uint64_t *B_ptrs,
                       int32_t slot, int32_t num_adapters, void *stream) {
    if (!A_slot || !B_slot || !A_host || !B_host || !A_ptrs || !B_ptrs) return SGMV_ERR_NULL;
    if (slot < 0 || slot >= num_adapters || A_bytes == 0 || B_bytes == 0) return SGMV_ERR_SHAPE;
    if (!aligned16(A_slot) || !aligned16(B_slot)) return SGMV_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(A_slot, A_host, A_bytes, hipMemcpyHostToDevice, st) != hipSuccess) return SGMV_ERR_HIP;
    if (hipMemcpyAsync(B_slot, B_host, B_bytes, hipMemcpyHostToDevice, st) != hipSuccess) return SGMV_ERR_HIP;
    return hip_status(sgmv::launch_set_slot(A_ptrs, B_ptrs, slot, reinterpret_cast<uintptr_t>(A_slot),
                                            reinterpret_cast<uintptr_t>(B_slot), st));
}

int sgmv_stream_probe(const void *src, size_t bytes, uint32_t *sink, int32_t num_blocks, void *stream) {
    if (!src || !sink) return SGMV_ERR_NULL;
    if (num_blocks <= 0 || bytes == 0 || (bytes & 15) != 0) return SGMV_ERR_SHAPE;
    if (!aligned16(src)) return SGMV_ERR_ALIGN;
    return hip_status(sgmv::launch_stream_probe(src, bytes / 16, sink, num_blocks, static_cast<hipStream_t>(stream)));
}

int sgmv_workspace_status(const void *workspace, uint32_t *status, void *stream) {
    if (!workspace || !status) return SGMV_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, st) != hipSuccess) return SGMV_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return SGMV_ERR_HIP;
    *status = word;
    return SGMV_OK;
}

uint32_t sgmv_set_wait_limit(uint32_t polls) { return sgmv::set_wait_limit(polls); }



}  // extern "C"
