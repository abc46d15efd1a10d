// SGMV kernels for gfx950 (MI355X): shrink, expand and fused shrink+expand.
//
// What is computed (Punica guide, aifetchly blog, section "The SGMV
// Mathematical Formulation" and the equation for y_i in "The Heterogeneous
// Batching Bottleneck"): for each segment s of rows seg_start[s] ..
// seg_start[s+1]-1 with adapter k = seg_adapter[s],
//     V[m, :] = X[m, :] . A_k          Y[m, :] += (alpha / r) * V[m, :] . B_k
// One launch covers every segment, each workgroup taking one segment's piece
// of work (figure "CUDA Threadblock Tiling": a block per segment gathers the
// segment's rows and streams that adapter's weights).
//
// Vector path. Every byte of an adapter is read once per segment and reused
// across the segment's rows held in registers, so decode segments (a handful
// of rows) run at the rate weights stream in from HBM.
//
//  * shrink: one workgroup per (segment, group of JG rank rows). The group's
//    JG rows of A_k (stored r x d_in, each row contiguous) are streamed in
//    16-byte loads spread over 256 lanes; each lane keeps partial dot products
//    for every (row, rank) pair of the segment, which are then summed across
//    the workgroup: a recursive-halving shuffle reduction inside each wave,
//    then a fixed-order sum over the four waves in LDS. No atomics: the
//    result is bitwise reproducible.
//  * expand: one workgroup per (segment, tile of d_out columns). B_k (stored
//    r x d_out) is streamed row by row, 16 bytes per lane; V of the segment's
//    rows is uniform across the workgroup; Y is read, updated in fp32 and
//    rounded once on store.
//  * fused: one launch whose workgroups take tickets from a counter: all
//    shrink items come first, then all expand items. An expand item waits for
//    its segment's shrink items; because those hold earlier tickets they were
//    already claimed by running workgroups that never wait, so the wait always
//    ends. The last workgroup to finish returns the counters to zero.

#include "sgmv_common.h"
#include "sgmv_launch.h"

namespace sgmv {

constexpr int kShrinkThreads = 256;
constexpr int kShrinkJG = 4;       // rank rows per shrink workgroup
constexpr int kShrinkUnroll = 4;   // 16-byte vectors in flight per lane per rank row
constexpr int kRowBlock = 8;       // rows held in registers at a time
constexpr int kExpandThreads = 64;

// ----------------------------------------------------------------------------
// Shrink, one block of up to ROWS rows of one segment against JG rank rows.
// ----------------------------------------------------------------------------
template <typename T, int R, int JG, int ROWS>
__device__ __forceinline__ void shrink_rows(float *V, const T *__restrict__ X,
                                            const T *__restrict__ Ak, int d_in, int row0,
                                            int nrows, int j0, float (*red)[64]) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int NV = ROWS * JG;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int nvec = d_in / VEC;

    float acc[ROWS][JG];
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
#pragma unroll
        for (int jj = 0; jj < JG; ++jj) acc[m][jj] = 0.f;

    for (int base = 0; base < nvec; base += kShrinkThreads * kShrinkUnroll) {
        uint4 a[kShrinkUnroll][JG];
#pragma unroll
        for (int u = 0; u < kShrinkUnroll; ++u) {
            const int v = base + u * kShrinkThreads + tid;
#pragma unroll
            for (int jj = 0; jj < JG; ++jj)
                a[u][jj] = v < nvec ? ld16_stream(Ak + (size_t)(j0 + jj) * d_in + (size_t)v * VEC)
                                    : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < ROWS; ++m) {
            if (m < nrows) {
                const T *xrow = X + (size_t)(row0 + m) * d_in;
#pragma unroll
                for (int u = 0; u < kShrinkUnroll; ++u) {
                    const int v = base + u * kShrinkThreads + tid;
                    if (v < nvec) {
                        float xf[VEC];
                        widen<T>(ld16(xrow + (size_t)v * VEC), xf);
#pragma unroll
                        for (int jj = 0; jj < JG; ++jj) {
                            float af[VEC];
                            widen<T>(a[u][jj], af);
#pragma unroll
                            for (int e = 0; e < VEC; ++e) acc[m][jj] = fmaf(xf[e], af[e], acc[m][jj]);
                        }
                    }
                }
            }
        }
    }

    float vals[NV];
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
#pragma unroll
        for (int jj = 0; jj < JG; ++jj) vals[m * JG + jj] = acc[m][jj];
    wave_reduce_transpose<NV>(vals, lane);
    constexpr int kSpread = kWave / NV;  // lanes that hold the same value index
    if ((lane & (kSpread - 1)) == 0) red[wave][lane / kSpread] = vals[0];
    __syncthreads();
    if (tid < NV) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kShrinkThreads / kWave; ++w) sum += red[w][tid];
        const int m = tid / JG;
        const int jj = tid % JG;
        if (m < nrows) V[(size_t)(row0 + m) * R + j0 + jj] = sum;
    }
    __syncthreads();
}

// All rows of one segment for rank rows j0 .. j0+JG-1.
template <typename T, int R, int JG>
__device__ __forceinline__ void shrink_segment(float *V, const T *__restrict__ X,
                                               const T *__restrict__ Ak, int d_in, int lo,
                                               int hi, int j0, float (*red)[64]) {
    for (int row0 = lo; row0 < hi; row0 += kRowBlock) {
        const int nrows = min(kRowBlock, hi - row0);
        if (nrows == 1)
            shrink_rows<T, R, JG, 1>(V, X, Ak, d_in, row0, nrows, j0, red);
        else if (nrows <= 2)
            shrink_rows<T, R, JG, 2>(V, X, Ak, d_in, row0, nrows, j0, red);
        else if (nrows <= 4)
            shrink_rows<T, R, JG, 4>(V, X, Ak, d_in, row0, nrows, j0, red);
        else
            shrink_rows<T, R, JG, 8>(V, X, Ak, d_in, row0, nrows, j0, red);
    }
}

template <typename T, int R>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(
    float *__restrict__ V, const T *__restrict__ X, const uint64_t *__restrict__ A_ptrs,
    int num_adapters, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ seg_adapter, int M, int d_in) {
    constexpr int JG = R < kShrinkJG ? R : kShrinkJG;
    constexpr int groups = R / JG;
    __shared__ float red[kShrinkThreads / kWave][64];
    const int s = blockIdx.x / groups;
    const int g = blockIdx.x % groups;
    int lo, hi;
    segment_rows(seg_start, s, M, lo, hi);
    const int k = seg_adapter[s];
    if (lo >= hi || k < 0 || k >= num_adapters) return;
    const T *Ak = reinterpret_cast<const T *>(A_ptrs[k]);
    shrink_segment<T, R, JG>(V, X, Ak, d_in, lo, hi, g * JG, red);
}

// ----------------------------------------------------------------------------
// Expand, one block of up to RB rows of one segment, VEC columns per lane.
// ----------------------------------------------------------------------------
// kCoherentV: V was written by other workgroups of this same launch (fused
// path), so it is read with device-coherent vector loads; otherwise it came
// from an earlier launch and may be read through any cache.
template <bool kCoherentV>
__device__ __forceinline__ float load_v(const float *p) {
    if constexpr (kCoherentV)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

template <typename T, int R, int RB, bool kCoherentV>
__device__ __forceinline__ void expand_rows(T *Y, const float *V, const T *__restrict__ Bk,
                                            int d_out, int row0, int nrows, int n0,
                                            bool active, float scale) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int JC = R < 8 ? R : 8;  // rank rows of B held in registers at a time
    float acc[RB][VEC];
#pragma unroll
    for (int m = 0; m < RB; ++m)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[m][e] = 0.f;

    // Up to 16 rank rows are unrolled so all their loads are in flight at
    // once; larger ranks stream 8 rows at a time to bound register use.
    constexpr int kChunks = R <= 16 ? R / JC : 1;
#pragma unroll kChunks
    for (int jc = 0; jc < R; jc += JC) {
        uint4 b[JC];
#pragma unroll
        for (int jj = 0; jj < JC; ++jj)
            b[jj] = active ? ld16_stream(Bk + (size_t)(jc + jj) * d_out + n0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
            float bf[VEC];
            widen<T>(b[jj], bf);
#pragma unroll
            for (int m = 0; m < RB; ++m) {
                if (m < nrows) {
                    const float v = load_v<kCoherentV>(V + (size_t)(row0 + m) * R + jc + jj);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[m][e] = fmaf(v, bf[e], acc[m][e]);
                }
            }
        }
    }
    if (!active) return;
#pragma unroll
    for (int m = 0; m < RB; ++m) {
        if (m < nrows) {
            T *yp = Y + (size_t)(row0 + m) * d_out + n0;
            float y[VEC];
            widen<T>(ld16(yp), y);
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = y[e] + scale * acc[m][e];
            st16(yp, narrow<T>(y));
        }
    }
}

template <typename T, int R, bool kCoherentV>
__device__ __forceinline__ void expand_segment(T *Y, const float *V, const T *__restrict__ Bk,
                                               int d_out, int lo, int hi, int n0, bool active,
                                               float scale) {
    for (int row0 = lo; row0 < hi; row0 += kRowBlock) {
        const int nrows = min(kRowBlock, hi - row0);
        if (nrows == 1)
            expand_rows<T, R, 1, kCoherentV>(Y, V, Bk, d_out, row0, nrows, n0, active, scale);
        else if (nrows <= 2)
            expand_rows<T, R, 2, kCoherentV>(Y, V, Bk, d_out, row0, nrows, n0, active, scale);
        else if (nrows <= 4)
            expand_rows<T, R, 4, kCoherentV>(Y, V, Bk, d_out, row0, nrows, n0, active, scale);
        else
            expand_rows<T, R, 8, kCoherentV>(Y, V, Bk, d_out, row0, nrows, n0, active, scale);
    }
}

template <typename T, int R>
__global__ __launch_bounds__(kExpandThreads) void expand_kernel(
    T *__restrict__ Y, const float *__restrict__ V, const uint64_t *__restrict__ B_ptrs,
    int num_adapters, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ seg_adapter, int M, int d_out, int ntiles, float scale) {
    constexpr int VEC = Elem<T>::kPerVec;
    const int s = blockIdx.x / ntiles;
    const int tile = blockIdx.x % ntiles;
    int lo, hi;
    segment_rows(seg_start, s, M, lo, hi);
    const int k = seg_adapter[s];
    if (lo >= hi || k < 0 || k >= num_adapters) return;
    const T *Bk = reinterpret_cast<const T *>(B_ptrs[k]);
    const int n0 = (tile * kExpandThreads + (int)threadIdx.x) * VEC;
    expand_segment<T, R, false>(Y, V, Bk, d_out, lo, hi, n0, n0 < d_out, scale);
}

// ----------------------------------------------------------------------------
// Fused: shrink items, then expand items, ordered by tickets.
// ----------------------------------------------------------------------------
struct FusedControl {
    uint32_t ticket;  // next item to hand out
    uint32_t done;    // workgroups finished
    uint32_t pad[62];
};

template <typename T, int R>
__global__ __launch_bounds__(kShrinkThreads) void fused_kernel(
    T *__restrict__ Y, const T *__restrict__ X, const uint64_t *__restrict__ A_ptrs,
    const uint64_t *__restrict__ B_ptrs, int num_adapters,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_adapter,
    int num_segments, int M, int d_in, int d_out, int ntiles, float scale,
    FusedControl *ctl, uint32_t *ready, float *Vws) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int JG = R < kShrinkJG ? R : kShrinkJG;
    constexpr int groups = R / JG;
    __shared__ float red[kShrinkThreads / kWave][64];
    __shared__ uint32_t s_item;
    __shared__ int s_flag;
    const int tid = threadIdx.x;
    const uint32_t shrink_items = (uint32_t)num_segments * groups;
    const uint32_t total = gridDim.x;

    if (tid == 0) s_item = atomicAdd(&ctl->ticket, 1u);
    __syncthreads();
    const uint32_t item = s_item;

    if (item < shrink_items) {
        const int s = item / groups;
        const int g = item % groups;
        int lo, hi;
        segment_rows(seg_start, s, M, lo, hi);
        const int k = seg_adapter[s];
        if (lo < hi && k >= 0 && k < num_adapters) {
            const T *Ak = reinterpret_cast<const T *>(A_ptrs[k]);
            shrink_segment<T, R, JG>(Vws, X, Ak, d_in, lo, hi, g * JG, red);
            __threadfence();  // this lane's V stores are visible device-wide
            __syncthreads();
            if (tid == 0)
                __hip_atomic_fetch_add(&ready[s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        const uint32_t e = item - shrink_items;
        const int s = e / ntiles;
        const int tile = e % ntiles;
        int lo, hi;
        segment_rows(seg_start, s, M, lo, hi);
        const int k = seg_adapter[s];
        if (lo < hi && k >= 0 && k < num_adapters) {
            if (tid == 0) {
                // Bounded wait: the producers hold earlier tickets and never
                // wait, so this ends; the bound only guards against a broken
                // workspace (counters not zero on entry).
                uint32_t spins = 0;
                int ok = 1;
                while (__hip_atomic_load(&ready[s], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
                       (uint32_t)groups) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++spins > (1u << 26)) {
                        ok = 0;
                        break;
                    }
                }
                s_flag = ok;
            }
            __syncthreads();
            __threadfence();
            if (s_flag) {
                const T *Bk = reinterpret_cast<const T *>(B_ptrs[k]);
                const int n0 = (tile * kShrinkThreads + tid) * VEC;
                expand_segment<T, R, true>(Y, Vws, Bk, d_out, lo, hi, n0, n0 < d_out, scale);
            }
        }
    }

    // Retire: the last workgroup out returns the control words to zero.
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&ctl->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = (prev == total - 1);
    }
    __syncthreads();
    if (s_flag) {
        for (int i = tid; i < num_segments; i += kShrinkThreads) ready[i] = 0;
        if (tid == 0) {
            ctl->ticket = 0;
            ctl->done = 0;
        }
    }
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------
template <typename T, int R>
static hipError_t launch_shrink_t(const ShrinkArgs &a, hipStream_t st) {
    constexpr int JG = R < kShrinkJG ? R : kShrinkJG;
    const unsigned grid = (unsigned)a.num_segments * (R / JG);
    hipLaunchKernelGGL((shrink_kernel<T, R>), dim3(grid), dim3(kShrinkThreads), 0, st, a.V,
                       reinterpret_cast<const T *>(a.X), a.A_ptrs, a.num_adapters, a.seg_start,
                       a.seg_adapter, a.M, a.d_in);
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_expand_t(const ExpandArgs &a, hipStream_t st) {
    constexpr int VEC = Elem<T>::kPerVec;
    const int tile_cols = kExpandThreads * VEC;
    const int ntiles = (a.d_out + tile_cols - 1) / tile_cols;
    const unsigned grid = (unsigned)a.num_segments * ntiles;
    hipLaunchKernelGGL((expand_kernel<T, R>), dim3(grid), dim3(kExpandThreads), 0, st,
                       reinterpret_cast<T *>(a.Y), a.V, a.B_ptrs, a.num_adapters, a.seg_start,
                       a.seg_adapter, a.M, a.d_out, ntiles, a.scale);
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t st) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int JG = R < kShrinkJG ? R : kShrinkJG;
    const int tile_cols = kShrinkThreads * VEC;
    const int ntiles = (a.d_out + tile_cols - 1) / tile_cols;
    const unsigned grid = (unsigned)a.num_segments * (R / JG) + (unsigned)a.num_segments * ntiles;
    const FusedLayout L = fused_layout(a.num_segments, a.M, a.r);
    char *ws = static_cast<char *>(a.workspace);
    hipLaunchKernelGGL((fused_kernel<T, R>), dim3(grid), dim3(kShrinkThreads), 0, st,
                       reinterpret_cast<T *>(a.Y), reinterpret_cast<const T *>(a.X), a.A_ptrs,
                       a.B_ptrs, a.num_adapters, a.seg_start, a.seg_adapter, a.num_segments, a.M,
                       a.d_in, a.d_out, ntiles, a.scale,
                       reinterpret_cast<FusedControl *>(ws + L.control),
                       reinterpret_cast<uint32_t *>(ws + L.ready),
                       reinterpret_cast<float *>(ws + L.v));
    return hipGetLastError();
}

#define SGMV_RANK_SWITCH(FN, T, args, st)           \
    switch ((args).r) {                             \
        case 8: return FN<T, 8>((args), (st));      \
        case 16: return FN<T, 16>((args), (st));    \
        case 32: return FN<T, 32>((args), (st));    \
        case 64: return FN<T, 64>((args), (st));    \
        default: return hipErrorInvalidValue;       \
    }

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t st) {
    if (a.dtype == kF32) SGMV_RANK_SWITCH(launch_shrink_t, float, a, st)
    SGMV_RANK_SWITCH(launch_shrink_t, bf16_t, a, st)
}

hipError_t launch_expand(const ExpandArgs &a, hipStream_t st) {
    if (a.dtype == kF32) SGMV_RANK_SWITCH(launch_expand_t, float, a, st)
    SGMV_RANK_SWITCH(launch_expand_t, bf16_t, a, st)
}

hipError_t launch_fused(const FusedArgs &a, hipStream_t st) {
    if (a.dtype == kF32) SGMV_RANK_SWITCH(launch_fused_t, float, a, st)
    SGMV_RANK_SWITCH(launch_fused_t, bf16_t, a, st)
}

}  // namespace sgmv
