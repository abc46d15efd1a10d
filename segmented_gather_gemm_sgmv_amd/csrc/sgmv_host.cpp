// The host-only entry points of the C ABI declared in include/sgmv.h: status
// strings, workspace size queries and the metadata helpers. Plain C++ with no
// HIP dependency, so that a host compiler alone can build them (with the
// sanitizers, for the host-side tests).
#include <algorithm>
#include <numeric>

#include "sgmv.h"
#include "sgmv_checks.h"
#include "sgmv_layout.h"

static_assert(SGMV_NOALLOC_SCRATCH_BYTES == sgmv::kScratchBytes, "scratch size of the header and the library agree");
static_assert(SGMV_WS_WAIT_TIMEOUT == sgmv::kStatusTimeout && SGMV_WS_BAD_OFFSETS == sgmv::kStatusBadOffsets,
              "status bits of the header and the kernels agree");
static_assert(SGMV_MAX_PROJECTIONS == sgmv::kMaxProjections, "projection limit of the header and the library agree");

using namespace sgmv::abi;

extern "C" {

int sgmv_version(void) { return 300; }

const char *sgmv_status_string(int status) {
    switch (status) {
        case SGMV_OK: return "ok";
        case SGMV_ERR_NULL: return "a required pointer is NULL";
        case SGMV_ERR_SHAPE: return "invalid size (negative, not a multiple of 8, or too large)";
        case SGMV_ERR_RANK: return "rank must be 8, 16, 32 or 64";
        case SGMV_ERR_DTYPE: return "dtype must be SGMV_F32 or SGMV_BF16";
        case SGMV_ERR_ALIGN: return "X, Y and V must be 16-byte aligned";
        case SGMV_ERR_WORKSPACE: return "workspace missing or too small";
        case SGMV_ERR_HIP: return "HIP runtime error at launch";
        case SGMV_ERR_ADAPTER: return "adapter id negative or outside the pool";
        case SGMV_ERR_SCRATCH: return "batch needs more workspace than the library's static scratch holds";
        default: return "unknown status";
    }
}

size_t sgmv_workspace_bytes(int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out,
                            int32_t r, int32_t dtype) {
    if (check_common(0, num_segments, M, r, dtype) != SGMV_OK ||
        check_sizes(M, num_segments, d_in, d_out, r, dtype) != SGMV_OK)
        return 0;
    return std::max(sgmv::shrink_layout(M, d_in, r, dtype).total,
                    sgmv::fused_layout(M, d_in, d_out, r, dtype).total);
}

size_t sgmv_layer_workspace_bytes(const sgmv_projection *projections, int32_t num_projections,
                                  int32_t num_segments, int32_t M, int32_t r, int32_t dtype) {
    sgmv::LayerProjIn in[sgmv::kMaxProjections];
    if (layer_inputs(projections, num_projections, num_segments, M, r, dtype, in) != SGMV_OK) return 0;
    return sgmv::layer_workspace_total(in, num_projections, num_segments, M, r, dtype);
}

int sgmv_build_segments(const int32_t *token_adapter, int32_t M, int32_t *perm,
                        int32_t *seg_start, int32_t *seg_adapter, int32_t *num_segments) {
    if (M < 0) return SGMV_ERR_SHAPE;
    if (!num_segments || !seg_start || (M > 0 && (!token_adapter || !perm || !seg_adapter)))
        return SGMV_ERR_NULL;
    for (int32_t i = 0; i < M; ++i)
        if (token_adapter[i] < 0) return SGMV_ERR_ADAPTER;
    std::iota(perm, perm + M, 0);
    std::stable_sort(perm, perm + M, [token_adapter](int32_t a, int32_t b) {
        return token_adapter[a] < token_adapter[b];
    });
    int32_t n = 0;
    for (int32_t p = 0; p < M; ++p) {
        const int32_t id = token_adapter[perm[p]];
        if (p == 0 || id != token_adapter[perm[p - 1]]) {
            seg_start[n] = p;
            seg_adapter[n] = id;
            ++n;
        }
    }
    seg_start[n] = M;
    *num_segments = n;
    return SGMV_OK;
}

int sgmv_check_segments(const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                        int32_t M, int32_t num_adapters) {
    if (num_segments < 0 || M < 0 || num_adapters < 0) return SGMV_ERR_SHAPE;
    if (!seg_start || (num_segments > 0 && !seg_adapter)) return SGMV_ERR_NULL;
    if (seg_start[0] != 0 || seg_start[num_segments] != M) return SGMV_ERR_SHAPE;
    for (int32_t s = 0; s < num_segments; ++s) {
        if (seg_start[s + 1] < seg_start[s]) return SGMV_ERR_SHAPE;
        if (seg_adapter[s] < 0 || seg_adapter[s] >= num_adapters) return SGMV_ERR_ADAPTER;
    }
    return SGMV_OK;
}

int sgmv_pool_pointers(uint64_t *ptrs_host, const void *base, int32_t num_adapters,
                       int64_t slot_bytes) {
    if (num_adapters < 0 || slot_bytes < 0) return SGMV_ERR_SHAPE;
    if (num_adapters == 0) return SGMV_OK;
    if (!ptrs_host || !base) return SGMV_ERR_NULL;
    if ((slot_bytes & 15) != 0 || !aligned16(base)) return SGMV_ERR_ALIGN;
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    for (int32_t k = 0; k < num_adapters; ++k) ptrs_host[k] = b + (uint64_t)k * (uint64_t)slot_bytes;
    return SGMV_OK;
}

}  // extern "C"
