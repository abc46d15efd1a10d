// bf16 MFMA tile path for long segments (gfx950).
//
// A segment with at least kLongRows rows is a small dense GEMM per step
// (Punica guide, "Hardware-Level Optimizations in SGMV": the tile shape
// follows the request length, prefill segments taking matrix-core tiles).
// Work is tiled over the batch's rows in tiles of kTileRows rows; a tile's
// workgroup finds the long segments that intersect it (a "piece" each) and
// runs each piece on v_mfma_f32_16x16x32_bf16, one wave per 16 rows.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 as used here (wave64): lane l
// holds A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] for e < 8, and
// receives D[4 (l / 16) + v][l % 16] for v < 4. The k index inside one
// instruction is only a summation index, so each lane may bring any 8
// consecutive elements of the reduction dimension as long as its A and B
// operands agree on which ones.
//
//  * shrink piece: D = X_rows (16 x d_in) . A_k^T (d_in x r). X rows are
//    read straight from HBM into the A operand; A_k is staged through LDS in
//    chunks of kShrinkKStep columns (double-buffered) and shared by the four
//    waves. fp32 accumulation.
//  * expand piece: D = V_rows (16 x r) . B_k (r x 128 columns). V is fp32 and
//    enters the A operand as two bf16 halves, hi = rne(v) and lo = rne(v - hi),
//    so hi + lo carries 16 significant bits; both halves meet the same B
//    operand. B_k is stored r x d_out (columns contiguous), so it is
//    transposed through LDS on its way in; the result is staged through LDS
//    so that Y is read and written in whole 16-byte vectors per lane.
#pragma once

#include "sgmv_common.h"

namespace sgmv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kLongRows = 16;           // segments this long or longer take the MFMA path
constexpr int kTileRows = 64;           // batch rows per MFMA tile (4 waves x 16)
constexpr int kShrinkKStep = 64;        // d_in elements staged per chunk
constexpr int kExpandTileCols = 128;    // d_out columns per expand tile
constexpr int kMaxPieces = 8;           // long segments one window of a tile can meet

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_to(int v, int M) { return v < 0 ? 0 : (v > M ? M : v); }

// Number of offsets p in [0, num_segments] with clamp(seg_start[p]) <= t, by a
// workgroup-wide search that tests 256 pivots per round (offsets are
// non-decreasing). Every thread returns the same value.
template <int kThreads>
__device__ int count_starts_le(const int32_t *seg_start, int num_segments, int M, int t) {
    int base = 0, len = num_segments + 1;
    while (len > 0) {
        const int stride = (len + kThreads - 1) / kThreads;
        const int off = (int)threadIdx.x * stride;
        const bool pred = off < len && clamp_to(seg_start[base + off], M) <= t;
        const int c = __syncthreads_count(pred);
        if (c == 0) break;
        const int last_true = base + (c - 1) * stride;
        const int end = c * stride < len ? base + c * stride : base + len;
        base = last_true + 1;
        len = end - base;
    }
    return base;
}

struct Piece {
    int lo, hi;  // rows of the piece (inside the tile and the segment)
    int seg;     // segment index
    int k;       // adapter
};

struct PieceList {
    Piece p[kMaxPieces];
    int n;
    int starts[kWave + 1];
    int more, next;
};

// Collect into `pl` the long segments (with a valid adapter) that intersect
// rows [t0, t1) of the batch. Offsets are scanned in windows of kWave
// segments from the one holding row t0, until a segment starts at or past
// t1. With valid (non-decreasing) offsets at most five long segments meet a
// tile; pieces beyond kMaxPieces (possible only with invalid offsets) are
// dropped. Call with the whole workgroup; pl is visible to all on return.
__device__ void gather_pieces(PieceList &pl, const int32_t *seg_start, const int32_t *seg_adapter,
                              int num_segments, int num_adapters, int M, int t0, int t1) {
    const int tid = threadIdx.x;
    const int cnt = count_starts_le<kBlockThreads>(seg_start, num_segments, M, t0);
    int first = cnt > 0 ? cnt - 1 : 0;
    if (tid == 0) pl.n = 0;
    while (true) {
        if (tid <= kWave) {
            const int idx = first + tid;
            pl.starts[tid] = idx <= num_segments ? clamp_to(seg_start[idx], M) : M;
        }
        __syncthreads();
        if (tid < kWave) {
            const int s = first + tid;
            if (s < num_segments) {
                const int lo = pl.starts[tid];
                const int hi = max(lo, pl.starts[tid + 1]);
                if (hi - lo >= kLongRows && lo < t1 && hi > t0) {
                    const int k = seg_adapter[s];
                    if (k >= 0 && k < num_adapters) {
                        const int slot = atomicAdd(&pl.n, 1);
                        if (slot < kMaxPieces) pl.p[slot] = Piece{max(lo, t0), min(hi, t1), s, k};
                    }
                }
            }
        }
        if (tid == 0) {
            const int last = min(first + kWave, num_segments);
            pl.more = last < num_segments && pl.starts[last - first] < t1;
            pl.next = last;
        }
        __syncthreads();
        if (!pl.more) break;
        first = pl.next;
        __syncthreads();
    }
    if (tid == 0 && pl.n > kMaxPieces) pl.n = kMaxPieces;
    __syncthreads();
}

// ----------------------------------------------------------------------------
// Shrink piece: V[m, 0:R] = X[m, :] . A_k for rows m in [p0, p1) of tile t0.
// ----------------------------------------------------------------------------
template <int R>
struct ShrinkSmem {
    static constexpr int kNB = R < 16 ? 1 : R / 16;            // 16-column MFMA blocks
    static constexpr int kRows = kNB * 16;                       // staged rows (zero past R)
    static constexpr int kStride = kShrinkKStep + 8;             // bf16 per staged row (padded)
    uint16_t a[2][kRows * kStride];
};

template <int R, bool kCoherent, typename StoreV>
__device__ void shrink_piece_mfma(const bf16_t *X, const bf16_t *Ak, int d_in, int t0, int p0, int p1,
                                  ShrinkSmem<R> &sm, StoreV store_v_fn) {
    constexpr int NB = ShrinkSmem<R>::kNB;
    constexpr int kStride = ShrinkSmem<R>::kStride;
    constexpr int kChunkVecs = R * (kShrinkKStep / 8);          // 16-byte vectors per chunk
    constexpr int kPer = (kChunkVecs + kBlockThreads - 1) / kBlockThreads;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane >> 4;
    const int i = lane & 15;
    const int row = t0 + 16 * wave + i;
    const bool row_ok = row >= p0 && row < p1;
    const bf16_t *xrow = X + (size_t)(row_ok ? row : p0) * d_in;
    const int nsteps = (d_in + kShrinkKStep - 1) / kShrinkKStep;

    // Staged rows past R (only when R < 16) stay zero for the whole piece.
    if (R < 16) {
        for (int idx = tid; idx < 2 * (NB * 16 - R) * kStride; idx += kBlockThreads) {
            const int b = idx / ((NB * 16 - R) * kStride);
            const int rem = idx % ((NB * 16 - R) * kStride);
            sm.a[b][R * kStride + rem] = 0;
        }
    }

    uint4 creg[kPer];
    uint4 xcur[2], xnext[2];
    auto load_chunk = [&](int step) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int idx = tid + q * kBlockThreads;
            const int j = idx >> 3;
            const int k = step * kShrinkKStep + (idx & 7) * 8;
            creg[q] = (idx < kChunkVecs && k < d_in) ? ld16_stream(Ak + (size_t)j * d_in + k)
                                                     : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int idx = tid + q * kBlockThreads;
            if (idx < kChunkVecs)
                *reinterpret_cast<uint4 *>(&sm.a[buf][(idx >> 3) * kStride + (idx & 7) * 8]) = creg[q];
        }
    };
    auto load_x = [&](int step, uint4 (&xr)[2]) {
        const int k = step * kShrinkKStep + 16 * g;
        xr[0] = (row_ok && k < d_in) ? ld16(xrow + k) : make_uint4(0, 0, 0, 0);
        xr[1] = (row_ok && k + 8 < d_in) ? ld16(xrow + k + 8) : make_uint4(0, 0, 0, 0);
    };

    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_chunk(0);
    load_x(0, xcur);
    store_chunk(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nsteps;
        if (more) {
            load_chunk(st + 1);
            load_x(st + 1, xnext);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8_t a = as_bf16x8(xcur[h]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint4 bv = *reinterpret_cast<const uint4 *>(
                    &sm.a[buf][(16 * b + i) * kStride + 16 * g + 8 * h]);
                acc[b] = mfma_bf16(a, as_bf16x8(bv), acc[b]);
            }
        }
        if (more) {
            store_chunk(buf ^ 1);
            xcur[0] = xnext[0];
            xcur[1] = xnext[1];
        }
        __syncthreads();
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = t0 + 16 * wave + 4 * g + v;
            const int j = 16 * b + i;
            if (m >= p0 && m < p1 && j < R) store_v_fn((size_t)m * R + j, acc[b][v]);
        }
    }
}

// ----------------------------------------------------------------------------
// Expand piece: Y[m, n0:n0+128] += scale * V[m, :] . B_k[:, n0:n0+128]
// for rows m in [p0, p1) of tile t0.
// ----------------------------------------------------------------------------
template <int R>
struct ExpandSmem {
    static constexpr int kK = R < 32 ? 32 : R;                  // reduction length, zero-padded
    static constexpr int kBtStride = kK + 8;                     // bf16 per transposed row (padded)
    static constexpr int kYsStride = kExpandTileCols + 4;        // floats per staged output row
    uint16_t bt[kExpandTileCols * kBtStride];                    // B tile, [n][k]
    float ys[kTileRows * kYsStride];                             // delta tile, [m][n]
};

__device__ __forceinline__ uint32_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int R, typename LoadV>
__device__ void expand_piece_mfma(bf16_t *Y, const bf16_t *Bk, int d_out, int t0, int p0, int p1,
                                  int n0, float scale, ExpandSmem<R> &sm, LoadV load_v_fn) {
    constexpr int K = ExpandSmem<R>::kK;
    constexpr int KS = K / 32;                                   // MFMA steps over the rank
    constexpr int kBt = ExpandSmem<R>::kBtStride;
    constexpr int kYs = ExpandSmem<R>::kYsStride;
    constexpr int kColVecs = kExpandTileCols / 8;                // 16 vectors of 8 per row
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane >> 4;
    const int i = lane & 15;

    // Y of this thread's output vectors, fetched early (each thread owns 4).
    constexpr int kYPer = kTileRows * kColVecs / kBlockThreads;
    uint4 yv[kYPer];
#pragma unroll
    for (int q = 0; q < kYPer; ++q) {
        const int idx = tid + q * kBlockThreads;
        const int m = t0 + idx / kColVecs;
        const int n = n0 + (idx % kColVecs) * 8;
        yv[q] = (m >= p0 && m < p1 && n < d_out) ? ld16(Y + (size_t)m * d_out + n) : make_uint4(0, 0, 0, 0);
    }

    // B tile -> LDS, transposed: two rank rows per pass, packed as pairs.
    for (int idx = tid; idx < (R / 2) * kColVecs; idx += kBlockThreads) {
        const int jp = idx / kColVecs;
        const int c8 = idx % kColVecs;
        const int n = n0 + c8 * 8;
        uint4 r0 = make_uint4(0, 0, 0, 0), r1 = make_uint4(0, 0, 0, 0);
        if (n < d_out) {
            r0 = ld16_stream(Bk + (size_t)(2 * jp) * d_out + n);
            r1 = ld16_stream(Bk + (size_t)(2 * jp + 1) * d_out + n);
        }
        const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
        const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t lo16 = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
            const uint32_t hi16 = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xffffu);
            *reinterpret_cast<uint32_t *>(&sm.bt[(c8 * 8 + e) * kBt + 2 * jp]) = lo16 | (hi16 << 16);
        }
    }
    if (R < K) {  // zero the padded part of the reduction
        for (int idx = tid; idx < kExpandTileCols * (K - R); idx += kBlockThreads)
            sm.bt[(idx / (K - R)) * kBt + R + idx % (K - R)] = 0;
    }

    // V rows of this wave as bf16 hi/lo halves (A operand).
    const int row = t0 + 16 * wave + i;
    const bool row_ok = row >= p0 && row < p1;
    bf16x8_t ahi[KS], alo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float v2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = ks * 32 + 8 * g + 2 * e2 + u;
                v2[u] = (row_ok && j < R) ? load_v_fn((size_t)row * R + j) : 0.f;
            }
            const uint32_t hb0 = bf16_bits(v2[0]), hb1 = bf16_bits(v2[1]);
            const float r0 = v2[0] - __uint_as_float(hb0 << 16);
            const float r1 = v2[1] - __uint_as_float(hb1 << 16);
            h[e2] = hb0 | (hb1 << 16);
            l[e2] = bf16_bits(r0) | (bf16_bits(r1) << 16);
        }
        ahi[ks] = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
        alo[ks] = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
    }
    __syncthreads();  // B tile in LDS

#pragma unroll
    for (int b = 0; b < kExpandTileCols / 16; ++b) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t bv = as_bf16x8(
                *reinterpret_cast<const uint4 *>(&sm.bt[(16 * b + i) * kBt + ks * 32 + 8 * g]));
            acc = mfma_bf16(ahi[ks], bv, acc);
            acc = mfma_bf16(alo[ks], bv, acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sm.ys[(16 * wave + 4 * g + v) * kYs + 16 * b + i] = acc[v];
    }
    __syncthreads();  // delta tile in LDS

#pragma unroll
    for (int q = 0; q < kYPer; ++q) {
        const int idx = tid + q * kBlockThreads;
        const int r = idx / kColVecs;
        const int c8 = idx % kColVecs;
        const int m = t0 + r;
        const int n = n0 + c8 * 8;
        if (m >= p0 && m < p1 && n < d_out) {
            const float4 d0 = *reinterpret_cast<const float4 *>(&sm.ys[r * kYs + c8 * 8]);
            const float4 d1 = *reinterpret_cast<const float4 *>(&sm.ys[r * kYs + c8 * 8 + 4]);
            const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            float y[8];
            widen<bf16_t>(yv[q], y);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] + scale * d[e];
            st16(Y + (size_t)m * d_out + n, narrow<bf16_t>(y));
        }
    }
    __syncthreads();  // LDS free for the next piece
}

}  // namespace sgmv
