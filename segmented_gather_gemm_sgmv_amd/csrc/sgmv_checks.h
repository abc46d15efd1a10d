// Argument checks of the C ABI, shared by the launching entry points
// (sgmv_api.cpp) and the host-only ones (sgmv_host.cpp). Host code only,
// free of HIP types.
#pragma once

#include <stdint.h>

#include "sgmv.h"
#include "sgmv_layout.h"

namespace sgmv {
namespace abi {

inline bool valid_rank(int32_t r) { return r == 8 || r == 16 || r == 32 || r == 64; }
inline bool valid_dtype(int32_t dt) { return dt == SGMV_F32 || dt == SGMV_BF16; }
inline bool valid_dim(int32_t d) { return d > 0 && d % 8 == 0; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element count one operand may span: indices are formed in 64-bit
// arithmetic, but a segment's row count and a column index stay in int.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

inline int check_common(int32_t num_adapters, int32_t num_segments, int32_t M, int32_t r, int32_t dtype) {
    if (!valid_dtype(dtype)) return SGMV_ERR_DTYPE;
    if (!valid_rank(r)) return SGMV_ERR_RANK;
    if (M < 0 || num_segments < 0 || num_adapters < 0) return SGMV_ERR_SHAPE;
    return SGMV_OK;
}

// Widths and sizes of one projection (call check_common first): d_in and
// d_out positive multiples of 8, X and Y within kMaxElems elements, and the
// launch within kMaxWorkgroups. A shrink-only or expand-only call passes 8
// for the width it does not have.
inline int check_sizes(int32_t M, int32_t num_segments, int32_t d_in, int32_t d_out, int32_t r, int32_t dtype) {
    if (!valid_dim(d_in) || !valid_dim(d_out)) return SGMV_ERR_SHAPE;
    if ((int64_t)M * d_in > kMaxElems || (int64_t)M * d_out > kMaxElems) return SGMV_ERR_SHAPE;
    if (launch_workgroups(M, num_segments, d_in, d_out, r, dtype) > kMaxWorkgroups) return SGMV_ERR_SHAPE;
    return SGMV_OK;
}

// Copies and checks a layer call's host descriptors.
inline int layer_inputs(const sgmv_projection *projections, int32_t num_projections, int32_t num_segments,
                        int32_t M, int32_t r, int32_t dtype, LayerProjIn *out) {
    if (num_projections < 0 || num_projections > SGMV_MAX_PROJECTIONS) return SGMV_ERR_SHAPE;
    if (num_projections > 0 && !projections) return SGMV_ERR_NULL;
    int64_t workgroups = 0;
    for (int32_t q = 0; q < num_projections; ++q) {
        const sgmv_projection &p = projections[q];
        int st = check_common(p.num_adapters, num_segments, M, r, dtype);
        if (st != SGMV_OK) return st;
        st = check_sizes(M, num_segments, p.d_in, p.d_out, r, dtype);
        if (st != SGMV_OK) return st;
        // the layer launch starts each projection's items on a multiple of 8
        workgroups += (launch_workgroups(M, num_segments, p.d_in, p.d_out, r, dtype) + 7) / 8 * 8;
        out[q] = LayerProjIn{p.Y, p.X, p.A_ptrs, p.B_ptrs, p.num_adapters, p.d_in, p.d_out};
    }
    return workgroups > kMaxWorkgroups ? SGMV_ERR_SHAPE : SGMV_OK;
}

}  // namespace abi
}  // namespace sgmv
