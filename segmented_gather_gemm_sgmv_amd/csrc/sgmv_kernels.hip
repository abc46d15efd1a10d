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
//  * shrink: one workgroup per (segment, group of four rank rows). For a
//    segment of one or two rows each wave takes one rank row j: row j of
//    A_k (stored r x d_in, each row contiguous) is streamed in 16-byte
//    loads, all in flight at once for d_in = 4096; each lane keeps a partial
//    dot product per segment row, and one recursive-halving shuffle
//    reduction per wave finishes them. For a longer segment the four waves
//    split d_in instead, each covering the four rank rows for a block of
//    rows, and their sums meet in LDS in wave order. No atomics: results are
//    bitwise reproducible.
//  * expand: one workgroup per (segment, tile of d_out columns). B_k (stored
//    r x d_out) is streamed row by row, 16 bytes per lane (once per segment
//    for r <= 16); V of the segment's rows is uniform across the workgroup;
//    Y is read, updated in fp32 and rounded once on store.
//  * fused: one launch; workgroups with the lowest ids do the shrink work,
//    the rest the expand work. An expand workgroup requests its B and Y,
//    then waits for V from its segment's shrink workgroups, which have lower
//    ids and so were dispatched first and never wait for an expand
//    workgroup. V crosses
//    workgroups only through device-scope (agent) atomic stores and loads,
//    performed at the device's point of coherence, so no cache writeback or
//    invalidation is needed. On the vector path each V value travels with a
//    ready flag in one 64-bit store, into one copy per expand column tile;
//    each expand workgroup polls the values of its own copy and clears them
//    once it has read them. On the MFMA path each part of a shrink tile
//    waits until its V stores have completed, then increments the tile's
//    arrival counter, and a consumer reads V once it has seen every part; a
//    departure counter per tile lets the last consumer return V and the
//    tile's counters to zero. Every launch leaves the whole workspace zero.

#include <atomic>
#include <mutex>
#include <type_traits>

#include "sgmv_common.h"
#include "sgmv_launch.h"
#include "sgmv_mfma.h"

namespace sgmv {

constexpr int kBlock = kBlockThreads;  // threads per workgroup (4 waves)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kShrinkUnroll = 8;       // 16-byte A vectors in flight per lane
constexpr int kRowBlock = 8;           // segment rows held in registers at a time

// V written by one launch and read by another may use any cache; V handed
// between workgroups of one launch uses device-coherent atomics.
template <bool kCoherent>
__device__ __forceinline__ void store_v(float *p, float v) {
    if constexpr (kCoherent)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

template <bool kCoherent>
__device__ __forceinline__ float load_v(const float *p) {
    if constexpr (kCoherent)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        return *p;
}

// Wait until every vector memory operation this wave issued has completed
// (s_waitcnt with vmcnt = 0 and the other counters left alone).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// V handed from the vector shrink to the vector expand within one launch
// travels as 64-bit pairs {value bits, ready flag}, each written by one
// device-scope atomic store: a consumer polls the values themselves, so the
// handoff costs one memory round trip after the store, with no counter and
// no barrier. `V` then points at M x r such pairs.
__device__ __forceinline__ void store_v_flagged(float *V, size_t idx, float v) {
    const uint64_t w = (1ull << 32) | __float_as_uint(v);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(V) + idx, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The workspace's sticky status word (NULL when the call has no workspace),
// as earlier calls left it: read at a workgroup's start with a plain load
// (the kernel boundary makes earlier launches' writes visible; a plain load
// may be served by the L2 its XCD shares, where a device-scope one would go
// to memory from every workgroup).
__device__ __forceinline__ uint32_t read_status(const WaitCtl &wc) {
    return wc.status ? *wc.status : 0u;
}

// The status word as it is now, failures of this launch included.
__device__ __forceinline__ uint32_t read_status_now(const WaitCtl &wc) {
    return wc.status ? __hip_atomic_load(wc.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
}

// Sets a status bit (call from one lane).
__device__ __forceinline__ void report(const WaitCtl &wc, uint32_t bit) {
    if (wc.status) __hip_atomic_fetch_or(wc.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// After unsuccessful poll number `spins` (0-based, uniform): whether the wait
// ends. It ends once `limit` polls have failed (reported as a timeout), or
// early when another wait has already failed: every 32nd poll rereads the
// status, so one failed wait does not leave the rest to run to their bounds.
// `lead`: this lane reports.
__device__ __forceinline__ bool give_up(const WaitCtl &wc, uint32_t spins, bool lead) {
    if (spins >= wc.limit) {
        if (lead) report(wc, kStatusTimeout);
        return true;
    }
    if ((spins & 31) == 31) return __builtin_amdgcn_readfirstlane((int)read_status_now(wc)) != 0;
    return false;
}

// Wave-wide: lane t < RB * JC fetches V[row0 + min(t / JC, nrows - 1)][jc + t % JC]
// from flagged pairs, polling until every one carries its flag. Returns false
// if the wait gave up (then `out` is meaningless).
template <int RB, int JC>
__device__ __forceinline__ bool poll_v_block(const float *V, int row0, int nrows, int R, int jc,
                                             float &out, const WaitCtl &wc) {
    static_assert(RB * JC <= kWave, "one pair per lane");
    const int lane = threadIdx.x & (kWave - 1);
    const int t = lane < RB * JC ? lane : 0;
    const uint64_t *p = reinterpret_cast<const uint64_t *>(V) +
                        (size_t)(row0 + min(t / JC, nrows - 1)) * R + jc + t % JC;
    for (uint32_t spins = 0;; ++spins) {
        const uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__all((uint32_t)(w >> 32) != 0)) {
            out = __uint_as_float((uint32_t)w);
            return true;
        }
        if (give_up(wc, spins, lane == 0)) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// ----------------------------------------------------------------------------
// Shrink: one wave, rank row j, up to ROWS rows of one segment.
//
// Every load is unconditional: an address past the end of a row is clamped
// back onto the row and its value masked to zero, and rows past the end of
// the block repeat the last row and are simply not stored. Straight-line
// loads let the compiler keep all of them in flight at once.
// ----------------------------------------------------------------------------
// kFlagged: V holds `copies` copies of M x r flagged pairs, `copy_stride`
// pairs apart, and each result goes to every copy.
template <typename T, int R, int ROWS, bool kFlagged, typename ArowFn, typename RM>
__device__ __forceinline__ void shrink_wave(float *V, const T *X, ArowFn arow_fn, int d_in,
                                            int row0, int nrows, int j, int lane, RM rm, int copies,
                                            size_t copy_stride) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int U = ROWS <= 2 ? kShrinkUnroll : (ROWS <= 4 ? kShrinkUnroll / 2 : kShrinkUnroll / 4);
    const int nvec = d_in / VEC;
    float acc[ROWS];
    const T *xrow[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        acc[m] = 0.f;
        xrow[m] = X + (size_t)rm(row0 + min(m, nrows - 1)) * d_in;
    }

    const T *Arow = nullptr;
    for (int base = 0; base < nvec; base += kWave * U) {
        uint4 a[U];
        uint4 x[ROWS][U];
        bool ok[U];
        int vc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            ok[u] = v < nvec;
            vc[u] = ok[u] ? v : nvec - 1;
        }
        // X first: its address is known before the adapter's
#pragma unroll
        for (int m = 0; m < ROWS; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) x[m][u] = ld16(xrow[m] + (size_t)vc[u] * VEC);
        // once, in the first pass: asked for on every pass, the address would
        // make each pass wait for the previous pass's loads
        if (base == 0) Arow = arow_fn();
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = ld16_stream(Arow + (size_t)vc[u] * VEC);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!ok[u]) a[u] = make_uint4(0, 0, 0, 0);
            float af[VEC];
            widen<T>(a[u], af);
#pragma unroll
            for (int m = 0; m < ROWS; ++m) {
                float xf[VEC];
                widen<T>(x[m][u], xf);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[m] = fmaf(xf[e], af[e], acc[m]);
            }
        }
    }
    wave_reduce_transpose<ROWS>(acc, lane);
    constexpr int kSpread = kWave / ROWS;  // lanes holding the same row's total
    if ((lane & (kSpread - 1)) == 0) {
        const int m = lane / kSpread;
        const size_t idx = (size_t)(row0 + m) * R + j;
        if (m < nrows) {
            if constexpr (kFlagged) {
                for (int c = 0; c < copies; ++c) store_v_flagged(V, idx + (size_t)c * copy_stride, acc[0]);
            } else
                V[idx] = acc[0];
        }
    }
}

// Segments of kSplitRows rows or more take the shrink a workgroup at a
// time: the four waves split d_in, and each covers a block of up to 8 rows
// (4 in some launches, see shrink_segment_split) and the workgroup's four
// rank rows j0 .. j0 + 3. A wave then streams its quarter of the block's X
// rows and of the four A_k rows, so X crosses the L1 once per workgroup
// instead of once per rank row, and a wave's loads fit in flight at once
// (d_in = 4096: two 16-byte vectors per lane and row). The partial sums
// meet in LDS and are added in wave order.
constexpr int kSplitRows = 3;

struct ShrinkSplitSmem {
    float part[kWavesPerBlock][8 * kWavesPerBlock];  // [wave][row * 4 + rank row]
};

template <typename T, int R, int ROWS, bool kFlagged, typename RM>
__device__ __forceinline__ void shrink_block_split(float *V, const T *X, const T *Ak, int d_in, int row0,
                                                   int nrows, int j0, RM rm, int copies, size_t copy_stride,
                                                   ShrinkSplitSmem &sm) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int J = kWavesPerBlock;
    constexpr int NV = ROWS * J;
    constexpr int U = 2;  // (ROWS + 4) * U vectors in flight per lane
    static_assert(ROWS * J <= 8 * kWavesPerBlock, "one block's partial sums fit the LDS buffer");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nvec = d_in / VEC;
    const int quarter = (nvec + J - 1) / J;
    const int vbeg = wave * quarter, vend = min(nvec, vbeg + quarter);
    float acc[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) acc[q] = 0.f;
    const T *xrow[ROWS];
#pragma unroll
    for (int m = 0; m < ROWS; ++m) xrow[m] = X + (size_t)rm(row0 + min(m, nrows - 1)) * d_in;
    // Loads are unconditional: a vector past the wave's range reads a clamped
    // address and is zeroed; rows past the block repeat its last row and are
    // never stored.
    for (int base = vbeg; base < vend; base += kWave * U) {
        uint4 x[ROWS][U], a[J][U];
        bool ok[U];
        int vc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = base + u * kWave + lane;
            ok[u] = v < vend;
            vc[u] = ok[u] ? v : vend - 1;
        }
#pragma unroll
        for (int m = 0; m < ROWS; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) x[m][u] = ld16(xrow[m] + (size_t)vc[u] * VEC);
#pragma unroll
        for (int jj = 0; jj < J; ++jj)
#pragma unroll
            for (int u = 0; u < U; ++u) a[jj][u] = ld16_stream(Ak + (size_t)(j0 + jj) * d_in + (size_t)vc[u] * VEC);
        // the four A_k vectors of a column widened once, each X vector widened
        // where it is used: few values live at a time
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float af[J][VEC];
#pragma unroll
            for (int jj = 0; jj < J; ++jj) {
                if (!ok[u]) a[jj][u] = make_uint4(0, 0, 0, 0);
                widen<T>(a[jj][u], af[jj]);
            }
#pragma unroll
            for (int m = 0; m < ROWS; ++m) {
                float xf[VEC];
                widen<T>(x[m][u], xf);
#pragma unroll
                for (int jj = 0; jj < J; ++jj)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[m * J + jj] = fmaf(xf[e], af[jj][e], acc[m * J + jj]);
            }
        }
    }
    wave_reduce_transpose<NV>(acc, lane);
    constexpr int kSpread = kWave / NV;  // lanes holding the same value's total
    if ((lane & (kSpread - 1)) == 0) sm.part[wave][lane / kSpread] = acc[0];
    __syncthreads();
    if (threadIdx.x < NV) {
        const int q = threadIdx.x;
        const float v = ((sm.part[0][q] + sm.part[1][q]) + sm.part[2][q]) + sm.part[3][q];
        const int m = q / J;
        if (m < nrows) {
            const size_t idx = (size_t)(row0 + m) * R + j0 + q % J;
            if constexpr (kFlagged) {
                for (int c = 0; c < copies; ++c) store_v_flagged(V, idx + (size_t)c * copy_stride, v);
            } else
                V[idx] = v;
        }
    }
    __syncthreads();  // sm is rewritten by the next block
}

template <typename T, int R, bool kFlagged, typename RM>
__device__ __forceinline__ void shrink_segment_split(float *V, const T *X, const T *Ak, int d_in, int lo, int hi,
                                                     int j0, RM rm, int copies, size_t copy_stride,
                                                     ShrinkSplitSmem &sm) {
    // Blocks of up to 8 rows take half the passes of blocks of 4. Launches
    // for batches with no segment of 16 rows or more keep blocks of 4: they
    // have little room for segments of several rows, and the registers of
    // 8-row blocks would cost their other items (segments of one or two
    // rows) a workgroup per CU at some ranks.
    constexpr int kRows = std::is_same<T, bf16_short_t>::value ? 4 : 8;
    for (int row0 = lo; row0 < hi; row0 += kRows) {
        const int nrows = min(kRows, hi - row0);
        if (nrows <= 4)
            shrink_block_split<T, R, 4, kFlagged>(V, X, Ak, d_in, row0, nrows, j0, rm, copies, copy_stride, sm);
        else
            shrink_block_split<T, R, 8, kFlagged>(V, X, Ak, d_in, row0, nrows, j0, rm, copies, copy_stride, sm);
    }
}

// All rows of one segment, rank row j, one wave. `arow_fn()` returns the
// address of row j of the segment's A_k; rm(p) the row of X behind segment
// row p.
template <typename T, int R, bool kFlagged, typename ArowFn, typename RM>
__device__ __forceinline__ void shrink_segment_wave(float *V, const T *X, ArowFn arow_fn, int d_in,
                                                    int lo, int hi, int j, int lane, RM rm, int copies,
                                                    size_t copy_stride) {
    for (int row0 = lo; row0 < hi; row0 += kRowBlock) {
        const int nrows = min(kRowBlock, hi - row0);
        if (nrows == 1)
            shrink_wave<T, R, 1, kFlagged>(V, X, arow_fn, d_in, row0, nrows, j, lane, rm, copies,
                                                copy_stride);
        else if (nrows <= 2)
            shrink_wave<T, R, 2, kFlagged>(V, X, arow_fn, d_in, row0, nrows, j, lane, rm, copies,
                                                copy_stride);
        else if (nrows <= 4)
            shrink_wave<T, R, 4, kFlagged>(V, X, arow_fn, d_in, row0, nrows, j, lane, rm, copies,
                                                copy_stride);
        else
            shrink_wave<T, R, 8, kFlagged>(V, X, arow_fn, d_in, row0, nrows, j, lane, rm, copies,
                                                copy_stride);
    }
}

template <typename T>
__device__ __forceinline__ bool takes_mfma(int rows) {
    return Elem<T>::kMfma && rows >= kLongRows;
}

// Whether the vector path owns a segment: rows present, a valid adapter, and
// too short for the MFMA path. Evaluated without short-circuits, so that the
// compiler requests the adapter id together with the row bounds instead of
// after them.
template <typename T>
__device__ __forceinline__ bool vector_segment(int lo, int hi, int k, int num_adapters) {
    return (lo < hi) & (k >= 0) & (k < num_adapters) & !takes_mfma<T>(hi - lo);
}

// One vector-path shrink item: rank row j of segment s, one wave (a segment
// of kSplitRows rows or more: rank rows j0 .. j0 + 3, the workgroup, so
// every wave of the workgroup must call this with the same segment). Returns
// false if the segment is empty, names no valid adapter or belongs to the
// MFMA path (then nothing is written).
// Offsets that decrease at this segment (so that other segments may overlap)
// are reported, once. In a separate shrink launch a non-zero workspace
// status (an earlier failure) makes the item a no-op; in the fused launch
// (kFlagged) the consumers check it instead, where their check costs no
// latency: a producer's V in a failed workspace is never read.
template <typename T, int R, bool kFlagged, bool kSpec, typename RM>
__device__ __forceinline__ bool shrink_vector_item(float *V, const T *X, const uint64_t *A_ptrs,
                                                   int num_adapters, const int32_t *seg_start,
                                                   const int32_t *seg_adapter, int s, int j, int M,
                                                   int d_in, int lane, RM rm, const WaitCtl &wc,
                                                   ShrinkSplitSmem &split_sm, int copies = 1) {
    AdapterTable<kSpec> tab;
    tab.load(A_ptrs, num_adapters, lane);
    int lo, hi;
    const uint32_t st = kFlagged ? 0u : read_status(wc);
    const int k = seg_adapter[s];
    const bool inverted = segment_rows(seg_start, s, M, lo, hi);
    if (inverted && j == 0 && lane == 0) report(wc, kStatusBadOffsets);
    if (!vector_segment<T>(lo, hi, k, num_adapters) | (st != 0)) return false;
    if (hi - lo >= kSplitRows) {  // uniform across the workgroup
        const T *Ak = reinterpret_cast<const T *>(tab.address(A_ptrs, k));
        shrink_segment_split<T, R, kFlagged>(V, X, Ak, d_in, lo, hi, j - (int)threadIdx.x / kWave, rm, copies,
                                             (size_t)M * R, split_sm);
        return true;
    }
    auto arow = [&]() { return reinterpret_cast<const T *>(tab.address(A_ptrs, k)) + (size_t)j * d_in; };
    shrink_segment_wave<T, R, kFlagged>(V, X, arow, d_in, lo, hi, j, lane, rm, copies, (size_t)M * R);
    return true;
}

// Thread 0 waits (bounded) until *counter reaches `target`. Returns 1 to
// every thread of the workgroup on success; loads issued after it see what
// the counted workgroups stored before counting themselves in (device-scope
// atomics on both sides, see the top of the file). Each caller explains why
// the workgroups it waits for are dispatched; the bound only guards against
// a workspace whose counters were not zero on entry or invalid metadata, and
// a wait that gives up is reported in the status word.
__device__ __forceinline__ int wait_for(uint32_t *counter, uint32_t target, int *s_flag, const WaitCtl &wc) {
    if (threadIdx.x == 0) {
        int ok = 1;
        for (uint32_t spins = 0;
             __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++spins) {
            if (give_up(wc, spins, true)) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(4);  // about 256 clocks between polls
        }
        *s_flag = ok;
    }
    __syncthreads();
    return *s_flag;
}

// Publish this workgroup's results: every wave waits until its stores
// (device-scope atomics) have completed, then thread 0 increments the
// counter.
__device__ __forceinline__ void publish(uint32_t *counter) {
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup out; returns 1 to every thread if it was the last of
// `expected` (all of them have finished reading V by then).
__device__ __forceinline__ int depart_last(uint32_t *counter, uint32_t expected, int *s_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev == expected - 1;
    }
    __syncthreads();
    return *s_flag;
}

__device__ __forceinline__ void zero_rows(float *Vws, int lo, int hi, int R) {
    for (int i = threadIdx.x; i < (hi - lo) * R; i += kBlock) store_v<true>(Vws + (size_t)lo * R + i, 0.f);
}

__device__ __forceinline__ void zero_pairs(float *Vpairs, int lo, int hi, int R) {
    uint64_t *p = reinterpret_cast<uint64_t *>(Vpairs) + (size_t)lo * R;
    for (int i = threadIdx.x; i < (hi - lo) * R; i += kBlock)
        __hip_atomic_store(p + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_pair(uint32_t *a, uint32_t *b) {
    if (threadIdx.x == 0) {
        __hip_atomic_store(a, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One MFMA shrink item: part `kp` (of `ks`) of d_in for column group `cg` of
// piece `pi` of the 16-row tile `t` (the shrink unit u; see
// mfma_shrink_item). With ks == 1 the result goes straight to V. Otherwise each part leaves its 16 x R partial
// tile in the workspace, in the MFMA D layout (fragment f = 64 b + lane holds
// four values, 16 bytes), counts itself in at *split_counter and waits for
// the other parts. Then every part finishes its own share of the fragments:
// it sums them over the parts in the order 0 .. ks-1, writes those V entries
// and clears those fragments in every part, so the tile's combine is spread
// over ks workgroups. The counter's return to zero is described below.
//
// The wait ends: the parts of a tile have consecutive workgroup ids,
// workgroups are dispatched in id order, and at most one tile straddles the
// dispatch front, with fewer parts than the device has slots, so every part
// of a waiting tile is dispatched. If the bound runs out all the same (a
// corrupt counter), the part skips its share and returns 0. Returns 1 (to
// all threads) once this workgroup's V entries are stored.
// kSelfReset: a second count lets the last part out return the split
// counter to zero. Without it (the fused kernel) the counter is left at ks
// for the tile's last expand workgroup to reset: the expand workgroups start
// only once every part has published, i.e. has passed its wait, and the
// part's own departure round trip stays off the path to its V handoff.
template <int R, bool kCoherent, bool kSelfReset, typename AkOf, typename RM>
__device__ int shrink_mfma_item(float *V, const bf16_t *X, AkOf ak_of,
                                const Piece &pc, int d_in, int t, int cg, int u, int kp, int ks,
                                uint32_t *split_counter, float *partials, ShrinkSmem<R> &sm,
                                int *s_flag, RM rm, const WaitCtl &wc) {
    constexpr int NB = ShrinkSmem<R>::kNBW;
    constexpr int kFrags = NB * kWave;  // 16-byte fragments per partial tile
    constexpr uint32_t kTileBytes = kFrags * 16;
    static_assert(kFrags <= kBlock, "one fragment per thread");
    const int t0 = t * kShrinkRows;
    const int nsteps = (d_in + ShrinkSmem<R>::kStepK - 1) / ShrinkSmem<R>::kStepK;
    const int per = (nsteps + ks - 1) / ks;
    const int s0 = min(nsteps, kp * per);
    const int s1 = min(nsteps, s0 + per);
    f32x4_t res = {0.f, 0.f, 0.f, 0.f};
    shrink_tile_mfma<R>(X, ak_of(pc.k), d_in, t0, pc.lo, pc.hi, cg, s0, s1, sm, res, rm);
    auto in_pieces = [&](int m) { return m >= pc.lo && m < pc.hi; };
    // fragment f = 64 b + lane, lane = (i, g): rows t0 + 4 g + v (v < 4),
    // column 16 (NB cg + b) + i
    auto store_frag = [&](int f, const f32x4_t &val) {
        const int lane = f % kWave, b = f / kWave;
        const int j = 16 * (NB * cg + b) + (lane & 15);
        if (j >= R) return;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = t0 + 4 * (lane >> 4) + v;
            if (in_pieces(m)) store_v<kCoherent>(V + (size_t)m * R + j, val[v]);
        }
    };
    const int tid = threadIdx.x;
    if (ks == 1) {
        if (tid < kFrags) store_frag(tid, res);
        return 1;
    }
    float *tile_parts = partials + (size_t)u * ks * (kTileBytes / 4);
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(tile_parts, (uint32_t)ks * kTileBytes);
    if (tid < kFrags) store4_coherent(rs, (uint32_t)kp * kTileBytes + (uint32_t)tid * 16, res);
    publish(split_counter);
    if (!wait_for(split_counter, (uint32_t)ks, s_flag, wc)) return 0;
    // This part's share: fragments [f0, f1). Every part of a fragment is
    // requested before it is summed or cleared: a load placed after a store
    // to the same buffer would wait for that store.
    constexpr int kMaxParts = 8;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const int f0 = kp * kFrags / ks, f1 = (kp + 1) * kFrags / ks;
    for (int f = f0 + tid; f < f1; f += kBlock) {
        f32x4_t pv[kMaxParts];
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) pv[k] = load4_coherent(rs, (uint32_t)k * kTileBytes + (uint32_t)f * 16);
        f32x4_t sum = zero;
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) sum += pv[k];
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) store4_coherent(rs, (uint32_t)k * kTileBytes + (uint32_t)f * 16, zero);
        store_frag(f, sum);
    }
    // every part has seen the full count once all of them have counted out
    if constexpr (kSelfReset) {
        if (depart_last(split_counter, 2u * (uint32_t)ks, s_flag) && threadIdx.x == 0)
            __hip_atomic_store(split_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return 1;
}

// One MFMA shrink item of a 64-row tile: part `kp` (of `ks`) of d_in for the
// 64-row tile `t`.
// With ks == 1 the result goes straight to V. Otherwise each part leaves its
// 64 x R partial tile in the workspace, in the MFMA D layout (fragment f =
// (wave * NB + b) * 64 + lane holds four values, 16 bytes), counts itself in
// at *split_counter and waits for the other parts. Then every part finishes
// its own share of the fragments: it sums them over the parts in the order
// 0 .. ks-1, writes those V entries and clears those fragments in every
// part, so the tile's combine is spread over ks workgroups instead of
// resting on one. The counter's return to zero is described below.
//
// The wait ends: the parts of a tile have consecutive workgroup ids,
// workgroups are dispatched in id order, and at most one tile straddles the
// dispatch front, with fewer parts than the device has slots, so every part
// of a waiting tile is dispatched. If the bound runs
// out all the same (a corrupt counter), the part skips its share and
// returns 0. Returns 1 (to all threads) once this workgroup's V entries are
// stored.
// kSelfReset: a second count lets the last part out return the split
// counter to zero. Without it (the fused kernel) the counter is left at ks
// for the tile's last expand workgroup to reset: the expand workgroups start
// only once every part has published, i.e. has passed its wait, and the
// part's own departure round trip stays off the path to its V handoff.
template <int R, bool kCoherent, bool kSelfReset, typename AkOf, typename RM>
__device__ int shrink_mfma_item64(float *V, const bf16_t *X, AkOf ak_of,
                                const PieceList &pl, int d_in, int t, int kp, int ks,
                                uint32_t *split_counter, float *partials, Shrink64Smem<R> &sm,
                                int *s_flag, RM rm, const WaitCtl &wc) {
    constexpr int NB = Shrink64Smem<R>::kNB;
    constexpr int kFrags = kWavesPerBlock * NB * kWave;  // 16-byte fragments per partial tile
    constexpr uint32_t kTileBytes = kFrags * 16;
    const int t0 = t * kShrinkTileRows;
    const int nmacro = (d_in + kMacroK - 1) / kMacroK;
    const int per = (nmacro + ks - 1) / ks;
    const int ms0 = min(nmacro, kp * per);
    const int ms1 = min(nmacro, ms0 + per);
    f32x4_t res[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) res[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // pieces kPassPieces at a time: one pass over this part of d_in each
    constexpr int PP = Shrink64Smem<R>::kPassPieces;
    for (int q = 0; q < pl.n; q += PP) {
        const Piece p0 = pl.p[q];
        bool two = false;
        if constexpr (PP == 2) {
            if (q + 1 < pl.n) {
                const Piece p1 = pl.p[q + 1];
                const bf16_t *const ak[2] = {ak_of(p0.k), ak_of(p1.k)};
                const int lo[2] = {p0.lo, p1.lo}, hi[2] = {p0.hi, p1.hi};
                shrink_tile64_mfma<R, 2>(X, ak, d_in, t0, lo, hi, ms0, ms1, sm, res, rm);
                two = true;
            }
        }
        if (!two) {
            const bf16_t *const ak[1] = {ak_of(p0.k)};
            const int lo[1] = {p0.lo}, hi[1] = {p0.hi};
            shrink_tile64_mfma<R, 1>(X, ak, d_in, t0, lo, hi, ms0, ms1, sm, res, rm);
        }
    }
    auto in_pieces = [&](int m) {
        bool in = false;
        for (int q = 0; q < pl.n; ++q) in |= m >= pl.p[q].lo && m < pl.p[q].hi;
        return in;
    };
    // fragment f: wave w = f / (NB * 64), block b, lane (i, g): rows
    // t0 + 16 w + 4 g + v (v < 4), column 16 b + i
    auto store_frag = [&](int f, const f32x4_t &val) {
        const int lane = f % kWave, b = (f / kWave) % NB, w = f / (kWave * NB);
        const int j = 16 * b + (lane & 15);
        if (j >= R) return;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = t0 + 16 * w + 4 * (lane >> 4) + v;
            if (in_pieces(m)) store_v<kCoherent>(V + (size_t)m * R + j, val[v]);
        }
    };
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    if (ks == 1) {
#pragma unroll
        for (int b = 0; b < NB; ++b) store_frag((wave * NB + b) * kWave + lane, res[b]);
        return 1;
    }
    float *tile_parts = partials + (size_t)t * ks * (kTileBytes / 4);
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(tile_parts, (uint32_t)ks * kTileBytes);
#pragma unroll
    for (int b = 0; b < NB; ++b)
        store4_coherent(rs, (uint32_t)kp * kTileBytes + (uint32_t)((wave * NB + b) * kWave + lane) * 16, res[b]);
    publish(split_counter);
    if (!wait_for(split_counter, (uint32_t)ks, s_flag, wc)) return 0;
    // This part's share: fragments [f0, f1), one per thread at most while
    // kFrags / ks <= kBlock. Every part of a fragment is requested before it
    // is summed or cleared: a load placed after a store to the same buffer
    // would wait for that store.
    constexpr int kMaxParts = 8;
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    const int f0 = kp * kFrags / ks, f1 = (kp + 1) * kFrags / ks;
    for (int f = f0 + (int)threadIdx.x; f < f1; f += kBlock) {
        f32x4_t pv[kMaxParts];
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) pv[k] = load4_coherent(rs, (uint32_t)k * kTileBytes + (uint32_t)f * 16);
        f32x4_t sum = zero;
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) sum += pv[k];
#pragma unroll
        for (int k = 0; k < kMaxParts; ++k)
            if (k < ks) store4_coherent(rs, (uint32_t)k * kTileBytes + (uint32_t)f * 16, zero);
        store_frag(f, sum);
    }
    // every part has seen the full count once all of them have counted out
    if constexpr (kSelfReset) {
        if (depart_last(split_counter, 2u * (uint32_t)ks, s_flag) && threadIdx.x == 0)
            __hip_atomic_store(split_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return 1;
}

// The MFMA shrink items of a launch: num_units shrink units (a 16-row tile,
// one of the long segments it meets and a group of V columns; unit u =
// (2 t + piece) kGroups + group), ks parts each. With one part,
// units are numbered so that each XCD takes a contiguous run of them
// (consecutive tiles belong to the same segments and read the same adapter,
// which then stays in one L2); the run is launched rounded up to a multiple
// of 8. With several parts, the parts of a unit have consecutive ids (they
// wait for one another) and part kp of every unit runs on XCD kp. Returns
// false for padding ids.
__device__ __forceinline__ bool mfma_shrink_item(int item, int first, int num_units, int ks, int &u, int &kp) {
    if (ks == 1) {
        u = xcd_local_item(item, first, num_units);
        kp = 0;
        return u >= 0;
    }
    u = (item - first) / ks;
    kp = (item - first) % ks;
    return u < num_units;
}

// Vector shrink items: segment s, rank group g (of `groups`), numbered so
// that all groups of one segment get ids of the same residue mod 8, i.e.
// run on one XCD (workgroups are dealt to the XCDs round-robin by id) and
// fetch the segment's X rows into one L2 instead of several. Needs
// round_up_xcds(N) * groups items; returns false for the padding.
__device__ __forceinline__ bool vector_shrink_item(int b, int num_segments, int groups, int &s, int &g) {
    const int chunk = b / (kXcds * groups);
    g = (b / kXcds) % groups;
    s = chunk * kXcds + b % kXcds;
    return s < num_segments;
}

// Adapter addresses for an MFMA item: with at most kSpecTable adapters the
// table is read once per wave, together with the segment metadata, instead
// of entry by entry once the pieces are known.
struct MfmaAdapters {
    AdapterTable<true> tab;
    const uint64_t *ptrs;
    int num_adapters;

    __device__ __forceinline__ MfmaAdapters(const uint64_t *p, int n) : ptrs(p), num_adapters(n) {
        tab.load(p, n, threadIdx.x & (kWave - 1));
    }
    // k: a valid adapter id, uniform across the workgroup (read from LDS, so
    // made explicitly uniform: the table lookup selects a lane by it)
    __device__ __forceinline__ const bf16_t *operator()(int k) const {
        k = __builtin_amdgcn_readfirstlane(k);
        return reinterpret_cast<const bf16_t *>(num_adapters <= kSpecTable ? tab.address(ptrs, k) : ptrs[k]);
    }
};

// Items [0, round_up_xcds(N) * R / 4): vector path, one per (segment, group of 4 rank rows),
// skipping segments the MFMA path owns. Items after that: MFMA shrink items,
// one per (16-row tile, part of d_in) (bf16 only).
template <typename T, int R, bool kGather, bool kSmall>
__global__ __launch_bounds__(kBlock) void shrink_kernel(
    float *__restrict__ V, const T *__restrict__ X, const uint64_t *__restrict__ A_ptrs,
    int num_adapters, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ seg_adapter, int num_segments, int M, int d_in, int num_units, int ks,
    uint32_t *counters, float *partials, RowMap<kGather> rm, WaitCtl wc) {
    constexpr int groups = R / kWavesPerBlock;
    const int gemv_items = round_up_xcds(num_segments) * groups;
    if (num_adapters <= 0) return;  // no segment can name a valid adapter
    if ((int)blockIdx.x < gemv_items) {
        int s, grp;
        if (!vector_shrink_item(blockIdx.x, num_segments, groups, s, grp)) return;
        const int j = grp * kWavesPerBlock + (int)threadIdx.x / kWave;
        const int lane = threadIdx.x & (kWave - 1);
        __shared__ ShrinkSplitSmem split_sm;
        if (num_adapters <= kSpecTable)
            shrink_vector_item<T, R, false, true>(V, X, A_ptrs, num_adapters, seg_start, seg_adapter,
                                                  s, j, M, d_in, lane, rm, wc, split_sm);
        else
            shrink_vector_item<T, R, false, false>(V, X, A_ptrs, num_adapters, seg_start, seg_adapter,
                                                   s, j, M, d_in, lane, rm, wc, split_sm);
        return;
    }
    if constexpr (Elem<T>::kMfma) {
        // one tile kind per kernel: the other's registers and LDS are not paid for
        __shared__ typename std::conditional<kSmall, ShrinkSmem<R>, Shrink64Smem<R>>::type sm;
        __shared__ PieceList pl;
        __shared__ int s_flag;
        int u, kp;
        if (!mfma_shrink_item((int)blockIdx.x, gemv_items, num_units, ks, u, kp)) return;
        const uint32_t st = read_status(wc);
        const MfmaAdapters ak_of(A_ptrs, num_adapters);
        const bf16_t *Xb = reinterpret_cast<const bf16_t *>(X);
        uint32_t *const split = ks > 1 ? counters + (size_t)u * kCounterStride : nullptr;
        if constexpr (kSmall) {
            constexpr int CG = ShrinkSmem<R>::kGroups;
            const int cg = u % CG, pi = (u / CG) % kShrinkPieces, t = u / (CG * kShrinkPieces);
            const int t0 = t * kShrinkRows;
            gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M, t0,
                                 min(t0 + kShrinkRows, M));
            if (pi >= pl.n || st != 0) return;
            shrink_mfma_item<R, false, true>(V, Xb, ak_of, pl.p[pi], d_in, t, cg, u, kp, ks, split, partials,
                                             sm, &s_flag, rm, wc);
        } else {
            const int t0 = u * kShrinkTileRows;
            gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M, t0,
                                 min(t0 + kShrinkTileRows, M));
            if (pl.n == 0 || st != 0) return;
            shrink_mfma_item64<R, false, true>(V, Xb, ak_of, pl, d_in, u, kp, ks, split, partials, sm, &s_flag,
                                               rm, wc);
        }
    }
}

// ----------------------------------------------------------------------------
// Expand: up to RB rows of one segment, VEC columns per lane.
// ----------------------------------------------------------------------------
template <typename T, int R, int RB, bool kFlagged, bool kBPre, typename BkFn, typename Ready, typename Commit,
          typename RM>
__device__ __forceinline__ void expand_rows(T *Y, const float *V, BkFn bk_fn, int d_out, int row0,
                                            int nrows, int n0, bool active, float scale, Ready ready,
                                            Commit commit, RM rm, const WaitCtl &wc, const uint4 *bpre) {
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int JC = R < 16 ? R : 16;  // rank rows of B held in registers at a time
    // Loads are unconditional (see shrink_wave): an inactive lane reads
    // column 0, rows past the block repeat the last row; neither is stored.
    const int nc = active ? n0 : 0;
    int rowc[RB];   // segment rows (V)
    int yrow[RB];   // their rows of Y
    bool yok[RB];   // yrow may be stored
    uint4 yv[RB];
    float acc[RB][VEC];
#pragma unroll
    for (int m = 0; m < RB; ++m) {
        rowc[m] = row0 + min(m, nrows - 1);
        yrow[m] = rm(rowc[m], yok[m]);
        yv[m] = ld16(Y + (size_t)yrow[m] * d_out + nc);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[m][e] = 0.f;
    }

    const T *Bk = kBPre ? nullptr : bk_fn();  // after the Y loads: their address is known first
#pragma unroll 1
    for (int jc = 0; jc < R; jc += JC) {
        uint4 b[JC];
#pragma unroll
        for (int jj = 0; jj < JC; ++jj)
            b[jj] = kBPre ? bpre[jc + jj] : ld16_stream(Bk + (size_t)(jc + jj) * d_out + nc);
        if (!ready()) return;  // uniform: V may be read from here on
        float vl = 0.f;  // flagged V: this lane's value of the block
        if constexpr (kFlagged) {
            if (!poll_v_block<RB, JC>(V, row0, nrows, R, jc, vl, wc)) return;  // wave-uniform
        }
#pragma unroll
        for (int m = 0; m < RB; ++m) {
            float v[JC];
            if constexpr (kFlagged) {
#pragma unroll
                for (int jj = 0; jj < JC; ++jj)
                    v[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vl), m * JC + jj));
            } else {
                // uniform across the workgroup: 16-byte scalar loads
                const float4 *vp = reinterpret_cast<const float4 *>(V + (size_t)rowc[m] * R + jc);
#pragma unroll
                for (int q = 0; q < JC / 4; ++q) {
                    const float4 t = vp[q];
                    v[4 * q] = t.x;
                    v[4 * q + 1] = t.y;
                    v[4 * q + 2] = t.z;
                    v[4 * q + 3] = t.w;
                }
            }
#pragma unroll
            for (int jj = 0; jj < JC; ++jj) {
                float bf[VEC];
                widen<T>(b[jj], bf);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[m][e] = fmaf(v[jj], bf[e], acc[m][e]);
            }
        }
    }
    if (!active || !commit()) return;
#pragma unroll
    for (int m = 0; m < RB; ++m) {
        if (m < nrows && yok[m]) {
            float y[VEC];
            widen<T>(yv[m], y);
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = y[e] + scale * acc[m][e];
            // (contiguous: the same row, row0 + m, in the form the compiler had before)
            st16(Y + (size_t)(RM::kIndexed ? yrow[m] : row0 + m) * d_out + n0, narrow<T>(y));
        }
    }
}

// `bk_fn()` returns the address of the segment's B_k. `ready()` is called
// (uniformly, possibly more than once) after B and Y have been requested and
// before V is read; the rows are left untouched if it returns false, or if
// `commit()`, called (uniformly) once V is read and before Y is stored,
// does. Rows
// are taken kMaxRB (4 or 8) at a time: 8 reads B_k half as often, 4 needs
// about 80 fewer registers per lane.
template <typename T, int R, bool kFlagged, int kMaxRB, typename BkFn, typename Ready, typename Commit,
          typename RM>
__device__ __forceinline__ void expand_segment(T *Y, const float *V, BkFn bk_fn, int d_out, int lo,
                                               int hi, int n0, bool active, float scale, Ready ready,
                                               Commit commit, RM rm, const WaitCtl &wc) {
    static_assert(kMaxRB == 4 || kMaxRB == 8, "row blocks of 4 or 8");
    // With R <= 16 the whole column slice of B_k fits in registers: it is
    // requested once for the segment, and every row block reuses it.
    constexpr bool kBPre = R <= 16;
    uint4 bpre[kBPre ? R : 1];
    if constexpr (kBPre) {
        const T *Bk = bk_fn();
        const int nc = active ? n0 : 0;
#pragma unroll
        for (int jj = 0; jj < R; ++jj) bpre[jj] = ld16_stream(Bk + (size_t)jj * d_out + nc);
    }
    for (int row0 = lo; row0 < hi; row0 += kMaxRB) {
        const int nrows = min(kMaxRB, hi - row0);
        if (nrows == 1)
            expand_rows<T, R, 1, kFlagged, kBPre>(Y, V, bk_fn, d_out, row0, nrows, n0, active, scale, ready,
                                                  commit, rm, wc, bpre);
        else if (nrows <= 2)
            expand_rows<T, R, 2, kFlagged, kBPre>(Y, V, bk_fn, d_out, row0, nrows, n0, active, scale, ready,
                                                  commit, rm, wc, bpre);
        else if (kMaxRB == 4 || nrows <= 4)
            expand_rows<T, R, 4, kFlagged, kBPre>(Y, V, bk_fn, d_out, row0, nrows, n0, active, scale, ready,
                                                  commit, rm, wc, bpre);
        else if constexpr (kMaxRB == 8)
            expand_rows<T, R, 8, kFlagged, kBPre>(Y, V, bk_fn, d_out, row0, nrows, n0, active, scale, ready,
                                                  commit, rm, wc, bpre);
    }
}

// One vector-path expand item: columns n0 .. n0 + VEC - 1 (per thread) of
// segment s; `ready` as for expand_segment. Returns false if the segment is
// empty, names no valid adapter or belongs to the MFMA path. In the fused
// launch (kFlagged) a non-zero workspace status as the launch began leaves
// its rows untouched (and returns false). lo, hi receive the segment's
// rows.
template <typename T, int R, bool kFlagged, int kMaxRB, bool kSpec, typename ReadyFn, typename RM>
__device__ __forceinline__ bool expand_vector_item(T *Y, const float *V, const uint64_t *B_ptrs,
                                                   int num_adapters, const int32_t *seg_start,
                                                   const int32_t *seg_adapter, int s, int n0, int M,
                                                   int d_out, float scale, int &lo, int &hi,
                                                   ReadyFn ready, RM rm, const WaitCtl &wc) {
    AdapterTable<kSpec> tab;
    tab.load(B_ptrs, num_adapters, threadIdx.x & (kWave - 1));
    const int k = seg_adapter[s];
    segment_rows(seg_start, s, M, lo, hi);
    if (!vector_segment<T>(lo, hi, k, num_adapters)) return false;
    auto bk = [&]() { return reinterpret_cast<const T *>(tab.address(B_ptrs, k)); };
    if constexpr (kFlagged) {
        // Requested after the metadata (loads complete in order, so waiting
        // for the metadata does not wait for it too) and looked at only
        // before Y is stored, so that V is polled without waiting for it.
        // On a failed workspace the polls end early (see give_up).
        const uint32_t st = read_status(wc);
        expand_segment<T, R, kFlagged, kMaxRB>(Y, V, bk, d_out, lo, hi, n0, n0 < d_out, scale, ready,
                                               [st]() { return st == 0; }, rm, wc);
        return st == 0;
    } else {
        expand_segment<T, R, kFlagged, kMaxRB>(Y, V, bk, d_out, lo, hi, n0, n0 < d_out, scale, ready,
                                               []() { return true; }, rm, wc);
        return true;
    }
}

// Items [0, N * ntiles_g): vector path, one per (segment, tile of
// kBlock * VEC columns; each wave takes kWave * VEC of them), skipping
// segments the MFMA path owns. Items after that: MFMA tiles of kTileRows
// batch rows by kExpandTileCols columns (bf16 only). kMaxRB: rows per block
// of the vector path (see expand_segment).
template <typename T, int R, int kMaxRB, bool kGather>
__global__ __launch_bounds__(kBlock) void expand_kernel(
    T *__restrict__ Y, const float *__restrict__ V, const uint64_t *__restrict__ B_ptrs,
    int num_adapters, const int32_t *__restrict__ seg_start,
    const int32_t *__restrict__ seg_adapter, int num_segments, int M, int d_out, int ntiles_g,
    int ntiles_m, float scale, RowMap<kGather> rm) {
    constexpr int VEC = Elem<T>::kPerVec;
    const int gemv_items = num_segments * ntiles_g;
    if (num_adapters <= 0) return;  // no segment can name a valid adapter
    if ((int)blockIdx.x < gemv_items) {
        const int s = blockIdx.x / ntiles_g;
        const int tile = blockIdx.x % ntiles_g;
        const int n0 = (tile * kBlock + (int)threadIdx.x) * VEC;
        int lo, hi;
        // B_k's address is loaded once the id is known: reading the table
        // early measured slower here, where Y is requested alongside B
        expand_vector_item<T, R, false, kMaxRB, false>(Y, V, B_ptrs, num_adapters, seg_start, seg_adapter,
                                                       s, n0, M, d_out, scale, lo, hi, []() { return true; }, rm,
                                                       WaitCtl{nullptr, 0});
        return;
    }
    if constexpr (Elem<T>::kMfma) {
        __shared__ ExpandSmem<R> sm;
        __shared__ PieceList pl;
        const int e = xcd_local_item(gemv_items, ((M + kTileRows - 1) / kTileRows) * ntiles_m);
        if (e < 0) return;
        const int t0 = (e / ntiles_m) * kTileRows;
        const int t1 = min(t0 + kTileRows, M);
        const int n0 = (e % ntiles_m) * kExpandTileCols * expand_halves(false);
        const MfmaAdapters bk_of(B_ptrs, num_adapters);
        auto load_v4 = [&](size_t idx) { return *reinterpret_cast<const float4 *>(V + idx); };
        auto ready = []() { return true; };
        if constexpr (kMaxRB == 4) {  // a batch of long segments: most tiles have pieces
            const SegPrefetch pre = prefetch_segments(seg_start, seg_adapter, num_segments);
            expand_tile_mfma<R, expand_halves(false), true, true>(
                reinterpret_cast<bf16_t *>(Y), M, d_out, t0, n0, scale, sm, pl,
                [&]() { gather_pieces<true>(pl, pre, seg_start, seg_adapter, num_segments, num_adapters, M, t0, t1); },
                bk_of, load_v4, ready, rm);
        } else {
            expand_tile_mfma<R, expand_halves(false), true, false>(
                reinterpret_cast<bf16_t *>(Y), M, d_out, t0, n0, scale, sm, pl,
                [&]() {
                    gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M,
                                         t0, t1);
                },
                bk_of, load_v4, ready, rm);
        }
    }
}

// ----------------------------------------------------------------------------
// Fused: every shrink item (vector, then MFMA tiles) has a lower workgroup id
// than every expand item (MFMA tiles, then vector).
// ----------------------------------------------------------------------------

// Row blocks of 4 in the fused kernel's vector expand keep its register
// count low enough for two workgroups per CU (r <= 32), so that expand
// workgroups are resident, with their B and Y requested, while the shrink
// workgroups still run.
constexpr int kFusedRB = 4;

// One work item of the fused launch: `item` is its id inside the launch's
// item layout (the workgroup id for a launch of one projection, the offset
// inside the projection's region for a layer-batched launch; congruent to
// the workgroup id modulo 8 either way, so the XCD placement is the same).
template <typename T, int R, bool kGather, bool kSmall>
__device__ __forceinline__ void fused_item(
    T *__restrict__ Y, const T *__restrict__ X, const uint64_t *__restrict__ A_ptrs,
    const uint64_t *__restrict__ B_ptrs, int num_adapters,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_adapter,
    int num_segments, int M, int d_in, int d_out, int ntiles_g, int ntiles_m, int num_tiles,
    int num_units, int ks, float scale, int long_batch, uint32_t *tile_counters,
    uint32_t *split_counters, float *Vws, float *Vpairs, float *partials, RowMap<kGather> rm, const WaitCtl &wc,
    const int item) {
    // The vector path hands V over as flagged pairs (Vpairs), one copy per
    // expand column tile, so each expand workgroup clears its own copy with
    // no counter. Each 64-row expand tile owns one cache line of counters:
    // word 0 counts the shrink parts whose V entries for its rows are stored
    // (of the shrink units of its four 16-row tiles, or of the 64-row tile),
    // polled by the expand workgroups until every part of every unit has
    // counted in; word 1 counts expand departures. A split unit's parts
    // synchronise on a line of their own (split_counters); the last expand
    // workgroup of a 64-row tile resets all of these.
    uint32_t *const tile_arrive = tile_counters;
    uint32_t *const tile_depart = tile_counters + 1;
    constexpr int VEC = Elem<T>::kPerVec;
    constexpr int groups = R / kWavesPerBlock;
    __shared__ int s_flag;
    const int tid = threadIdx.x;
    // Item regions, in dispatch order: producers first (vector shrink, MFMA
    // shrink), then consumers (MFMA expand, vector expand). The MFMA expand
    // tiles come before the vector expand items: they have more to do once
    // V is there, and the vector items, which mostly wait for their
    // segment's shrink, can take the last slots.
    const int a0 = round_up_xcds(num_segments) * groups;   // vector shrink items
    const int a1 = a0 + mfma_shrink_items(num_units, ks);  // MFMA shrink items (unit x part)
    const int aM = a1 + round_up_xcds(num_tiles * ntiles_m);  // MFMA expand tiles
    const int a2 = aM + num_segments * ntiles_g;            // vector expand items

    if (num_adapters <= 0) return;  // no segment can name a valid adapter
    if (item < a0) {
        int s, grp;
        if (!vector_shrink_item(item, num_segments, groups, s, grp)) return;
        const int j = grp * kWavesPerBlock + tid / kWave;
        __shared__ ShrinkSplitSmem split_sm;
        if (num_adapters <= kSpecTable)
            shrink_vector_item<T, R, true, true>(Vpairs, X, A_ptrs, num_adapters, seg_start, seg_adapter,
                                                 s, j, M, d_in, tid & (kWave - 1), rm, wc, split_sm, ntiles_g);
        else
            shrink_vector_item<T, R, true, false>(Vpairs, X, A_ptrs, num_adapters, seg_start, seg_adapter,
                                                  s, j, M, d_in, tid & (kWave - 1), rm, wc, split_sm, ntiles_g);
        return;
    }
    if (item >= aM && item < a2) {
        const int e = item - aM;
        const int s = e / ntiles_g;
        const int tile = e % ntiles_g;
        const int n0 = (tile * kBlock + tid) * VEC;
        float *const Vcopy = Vpairs + (size_t)tile * M * R * 2;  // this column tile's copy (pairs)
        int lo, hi;
        auto ready = []() { return true; };  // the V reads wait for their flags
        // here B is requested before V is waited for, so B_k's address is on
        // the critical path: read the table early when the pool is small
        const bool valid =
            num_adapters <= kSpecTable
                ? expand_vector_item<T, R, true, kFusedRB, true>(Y, Vcopy, B_ptrs, num_adapters, seg_start,
                                                                 seg_adapter, s, n0, M, d_out, scale,
                                                                 lo, hi, ready, rm, wc)
                : expand_vector_item<T, R, true, kFusedRB, false>(Y, Vcopy, B_ptrs, num_adapters, seg_start,
                                                                  seg_adapter, s, n0, M, d_out, scale,
                                                                  lo, hi, ready, rm, wc);
        if (!valid) return;
        // every wave of this workgroup has read its values: clear the copy
        // (no other workgroup reads it)
        __syncthreads();
        zero_pairs(Vcopy, lo, hi, R);
        return;
    }
    if constexpr (Elem<T>::kMfma) {
        // one shrink tile kind per kernel: the other's registers and LDS are not paid for
        __shared__ union {
            typename std::conditional<kSmall, ShrinkSmem<R>, Shrink64Smem<R>>::type shrink;
            ExpandSmem<R> expand;
        } sm;
        __shared__ PieceList pl;
        const bf16_t *Xb = reinterpret_cast<const bf16_t *>(X);
        if (item >= a0 && item < a1) {
            // (shrink unit, part of d_in); each part reports its share of V
            // on the arrival word of the 64-row tile holding these rows
            int u, kp;
            if (!mfma_shrink_item(item, a0, num_units, ks, u, kp)) return;
            const uint32_t st = read_status(wc);
            const MfmaAdapters ak_of(A_ptrs, num_adapters);
            uint32_t *const split = ks > 1 ? split_counters + (size_t)u * kCounterStride : nullptr;
            int done;
            int t64;
            if constexpr (kSmall) {
                constexpr int CG = ShrinkSmem<R>::kGroups;
                const int cg = u % CG, pi = (u / CG) % kShrinkPieces, t = u / (CG * kShrinkPieces);
                const int t0 = t * kShrinkRows;
                gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M,
                                     t0, min(t0 + kShrinkRows, M));
                if (pi >= pl.n || st != 0) return;
                done = shrink_mfma_item<R, true, false>(Vws, Xb, ak_of, pl.p[pi], d_in, t, cg, u, kp, ks, split,
                                                        partials, sm.shrink, &s_flag, rm, wc);
                t64 = t0 / kTileRows;
            } else {
                const int t0 = u * kShrinkTileRows;
                gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M,
                                     t0, min(t0 + kShrinkTileRows, M));
                if (pl.n == 0 || st != 0) return;
                done = shrink_mfma_item64<R, true, false>(Vws, Xb, ak_of, pl, d_in, u, kp, ks, split, partials,
                                                          sm.shrink, &s_flag, rm, wc);
                t64 = u;
            }
            if (done) publish(&tile_arrive[t64 * kCounterStride]);
            return;
        }
        if (item < a1 || item >= aM) return;
        const int e = xcd_local_item(item, a1, num_tiles * ntiles_m);
        if (e < 0) return;
        const int t = e / ntiles_m;
        const int t0 = t * kTileRows;
        const int t1 = min(t0 + kTileRows, M);
        const int n0 = (e % ntiles_m) * kExpandTileCols * expand_halves(!kSmall);
        const uint32_t st = read_status(wc);
        const MfmaAdapters bk_of(B_ptrs, num_adapters);
        // V of these rows is complete once every part of every shrink unit
        // inside them has reported: kGroups units per 16-row tile and long
        // segment meeting it (the shrink tiles find the same long segments);
        // a non-zero status on entry makes the tile a no-op
        int state = -1;  // uniform: -1 not yet waited, else the result of the wait
        auto ready = [&]() {
            if (state < 0) {
                int units = 1;  // 64-row tiles: the tile itself
                if constexpr (kSmall) {
                    units = 0;
                    for (int a = t0; a < t1; a += kShrinkRows) {
                        const int b = min(a + kShrinkRows, t1);
                        for (int q = 0; q < pl.n; ++q) units += pl.p[q].lo < b && pl.p[q].hi > a;
                    }
                    units *= ShrinkSmem<R>::kGroups;
                }
                state = st == 0 &&
                        wait_for(&tile_arrive[t * kCounterStride], (uint32_t)(ks * units), &s_flag, wc);
            }
            return state != 0;
        };
        // V of this tile's rows, read at device scope (written in this launch)
        float *const vt = Vws + (size_t)t0 * R;
        const __amdgpu_buffer_rsrc_t vr = coherent_rsrc(vt, (uint32_t)(kTileRows * R * sizeof(float)));
        auto load_v4 = [&](size_t idx) {
            const f32x4_t v = load4_coherent(vr, (uint32_t)((idx - (size_t)t0 * R) * sizeof(float)));
            return make_float4(v[0], v[1], v[2], v[3]);
        };
        if (long_batch) {  // segments of 16 rows or more on average: most tiles have pieces
            const SegPrefetch pre = prefetch_segments(seg_start, seg_adapter, num_segments);
            expand_tile_mfma<R, expand_halves(!kSmall), false, true>(
                reinterpret_cast<bf16_t *>(Y), M, d_out, t0, n0, scale, sm.expand, pl,
                [&]() { gather_pieces<true>(pl, pre, seg_start, seg_adapter, num_segments, num_adapters, M, t0, t1); },
                bk_of, load_v4, ready, rm);
        } else {
            expand_tile_mfma<R, expand_halves(!kSmall), false, false>(
                reinterpret_cast<bf16_t *>(Y), M, d_out, t0, n0, scale, sm.expand, pl,
                [&]() {
                    gather_pieces<false>(pl, SegPrefetch{}, seg_start, seg_adapter, num_segments, num_adapters, M,
                                         t0, t1);
                },
                bk_of, load_v4, ready, rm);
        }
        if (pl.n == 0) return;
        if (depart_last(&tile_depart[t * kCounterStride], (uint32_t)ntiles_m, &s_flag)) {
            for (int q = 0; q < pl.n; ++q) zero_rows(Vws, pl.p[q].lo, pl.p[q].hi, R);
            reset_pair(&tile_arrive[t * kCounterStride], &tile_depart[t * kCounterStride]);
            // the split counters of its shrink tiles too: their parts all
            // passed their wait before publishing
            const int units_per_tile = kSmall ? ShrinkSmem<R>::kGroups * kShrinkPieces * kTileRows / kShrinkRows : 1;
            if (ks > 1 && tid < units_per_tile) {
                const int u = units_per_tile * t + tid;
                if (u < num_units)
                    __hip_atomic_store(split_counters + (size_t)u * kCounterStride, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <typename T, int R, bool kGather, bool kSmall>
__global__ __launch_bounds__(kBlock) void fused_kernel(
    T *__restrict__ Y, const T *__restrict__ X, const uint64_t *__restrict__ A_ptrs,
    const uint64_t *__restrict__ B_ptrs, int num_adapters,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_adapter,
    int num_segments, int M, int d_in, int d_out, int ntiles_g, int ntiles_m, int num_tiles,
    int num_units, int ks, float scale, int long_batch, uint32_t *tile_counters,
    uint32_t *split_counters, float *Vws, float *Vpairs, float *partials, RowMap<kGather> rm, WaitCtl wc) {
    fused_item<T, R, kGather, kSmall>(Y, X, A_ptrs, B_ptrs, num_adapters, seg_start, seg_adapter, num_segments, M,
                              d_in, d_out, ntiles_g, ntiles_m, num_tiles, num_units, ks, scale, long_batch,
                              tile_counters, split_counters, Vws, Vpairs, partials, rm, wc, (int)blockIdx.x);
}

// Layer-batched fused launch (the launch accounting of the Punica guide's
// "Mathematical Modeling", extended from one layer's A and B launches to all
// of its projections): every projection of one batch in one launch. Each
// projection keeps the item layout of its own fused launch, in a region of
// workgroup ids starting at a multiple of 8; regions follow one another in
// projection order. Inside a region every wait is on lower ids of the same
// region (or on the sibling parts of a split shrink tile), so the argument
// that a fused launch's waits end carries over unchanged.
template <typename T, int R, bool kGather, bool kSmall>
__global__ __launch_bounds__(kBlock) void fused_layer_kernel(
    LayerArgs L, const int32_t *__restrict__ seg_start, const int32_t *__restrict__ seg_adapter,
    int num_segments, int M, float scale, int long_batch, RowMap<kGather> rm) {
    // The descriptors are read in place, in the kernel argument segment (L
    // is the first argument, at offset 0): indexing the by-value copy with a
    // computed index can make the compiler copy the whole argument to the
    // stack.
    using ConstProj = const __attribute__((address_space(4))) LayerProj;
    ConstProj *kargs = (ConstProj *)__builtin_amdgcn_kernarg_segment_ptr();
    const int b = blockIdx.x;
    int p = 0;
    for (int q = 1; q < L.num_projections; ++q) p = b >= kargs[q].base ? q : p;
    p = __builtin_amdgcn_readfirstlane(p);
    // The selected descriptor, field by field, as explicitly uniform values:
    // read through the computed index, some fields would otherwise be kept
    // in vector registers, where the pointers that feed buffer resources
    // (which must be scalar) cannot be.
    LayerProj d;
    {
        ConstProj &src = kargs[p];
        auto up = [](auto *ptr) {
            const uint64_t v = reinterpret_cast<uint64_t>(ptr);
            const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
            const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
            return reinterpret_cast<decltype(ptr)>((hi << 32) | lo);
        };
        auto ui = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
        d.Y = up(src.Y);
        d.X = up(src.X);
        d.A_ptrs = up(src.A_ptrs);
        d.B_ptrs = up(src.B_ptrs);
        d.tile_counters = up(src.tile_counters);
        d.split_counters = up(src.split_counters);
        d.Vws = up(src.Vws);
        d.Vpairs = up(src.Vpairs);
        d.partials = up(src.partials);
        d.num_adapters = ui(src.num_adapters);
        d.d_in = ui(src.d_in);
        d.d_out = ui(src.d_out);
        d.ntiles_g = ui(src.ntiles_g);
        d.ntiles_m = ui(src.ntiles_m);
        d.num_tiles = ui(src.num_tiles);
        d.num_units = ui(src.num_units);
        d.ks = ui(src.ks);
        d.base = ui(src.base);
        d.items = ui(src.items);
    }
    const int item = b - d.base;
    if (item >= d.items) return;  // padding up to the next region
    fused_item<T, R, kGather, kSmall>(reinterpret_cast<T *>(d.Y), reinterpret_cast<const T *>(d.X), d.A_ptrs,
                              d.B_ptrs, d.num_adapters, seg_start, seg_adapter, num_segments, M, d.d_in,
                              d.d_out, d.ntiles_g, d.ntiles_m, d.num_tiles, d.num_units, d.ks, scale,
                              long_batch,
                              d.tile_counters, d.split_counters, d.Vws, d.Vpairs, d.partials, rm, L.wc, item);
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------
static_assert(kTileRows64 == kTileRows && kShrinkRows16 == kShrinkRows,
              "workspace layouts must match the MFMA tiles");
static_assert(kLaunchThreads == kBlock && kExpandCols == kExpandTileCols && kWavesPerBlock == 4 && kXcds == 8,
              "launch sizes counted on the host must match the kernels");

static int mfma_tiles(int dtype, int M) { return dtype == kBF16 ? (M + kTileRows - 1) / kTileRows : 0; }


template <typename T>
static int gemv_col_tiles(int d_out) {
    const int cols = kBlock * Elem<T>::kPerVec;
    return (d_out + cols - 1) / cols;
}

template <typename T, int R, bool kGather, bool kSmall>
static hipError_t launch_shrink_g(const ShrinkArgs &a, hipStream_t st) {
    const ShrinkLayout L = shrink_layout(a.M, a.d_in, a.r, a.dtype);
    const int units = Elem<T>::kMfma ? L.plan.units : 0;
    const int ks = L.plan.ks;
    const unsigned grid = (unsigned)round_up_xcds(a.num_segments) * (R / kWavesPerBlock) +
                          (unsigned)(units ? mfma_shrink_items(units, ks) : 0);
    char *ws = static_cast<char *>(a.workspace);
    hipLaunchKernelGGL((shrink_kernel<T, R, kGather, kSmall>), dim3(grid), dim3(kBlock), 0, st, a.V,
                       reinterpret_cast<const T *>(a.X), a.A_ptrs, a.num_adapters, a.seg_start,
                       a.seg_adapter, a.num_segments, a.M, a.d_in, units, ks,
                       ks > 1 ? reinterpret_cast<uint32_t *>(ws + L.counters) : nullptr,
                       ks > 1 ? reinterpret_cast<float *>(ws + L.partials) : nullptr,
                       RowMap<kGather>{a.rows, a.M},
                       WaitCtl{L.total > 0 ? reinterpret_cast<uint32_t *>(ws) : nullptr, wait_limit()});
    return hipGetLastError();
}

// Kernels are built per shrink tile kind (a bf16 batch of up to
// small_batch_rows(r) rows takes 16-row tiles, a larger one 64-row tiles);
// batches without the MFMA path take the 16-row build.
template <typename T, int R>
static hipError_t launch_shrink_t(const ShrinkArgs &a, hipStream_t st) {
    if constexpr (Elem<T>::kMfma) {
        if (!small_tiles(a.M, R))
            return a.rows ? launch_shrink_g<T, R, true, false>(a, st) : launch_shrink_g<T, R, false, false>(a, st);
    }
    return a.rows ? launch_shrink_g<T, R, true, true>(a, st) : launch_shrink_g<T, R, false, true>(a, st);
}

template <typename T, int R, bool kGather>
static hipError_t launch_expand_g(const ExpandArgs &a, hipStream_t st) {
    const int ntiles_g = gemv_col_tiles<T>(a.d_out);
    const int tiles = Elem<T>::kMfma ? mfma_tiles(a.dtype, a.M) : 0;
    const int ntiles_m = tiles ? ceil_div(a.d_out, kExpandTileCols * expand_halves(false)) : 0;
    const unsigned grid = (unsigned)a.num_segments * ntiles_g + (unsigned)round_up_xcds(tiles * ntiles_m);
    // Batches of short segments (under 16 rows on average) run mostly on the
    // vector path: rows 8 at a time read B_k half as often. Batches of long
    // segments run mostly on the MFMA path, whose occupancy the vector path's
    // registers would otherwise limit: rows 4 at a time.
    const RowMap<kGather> rm{a.rows, a.M};
    if ((int64_t)a.M < 16 * (int64_t)a.num_segments)
        hipLaunchKernelGGL((expand_kernel<T, R, 8, kGather>), dim3(grid), dim3(kBlock), 0, st,
                           reinterpret_cast<T *>(a.Y), a.V, a.B_ptrs, a.num_adapters, a.seg_start,
                           a.seg_adapter, a.num_segments, a.M, a.d_out, ntiles_g, ntiles_m, a.scale, rm);
    else
        hipLaunchKernelGGL((expand_kernel<T, R, 4, kGather>), dim3(grid), dim3(kBlock), 0, st,
                           reinterpret_cast<T *>(a.Y), a.V, a.B_ptrs, a.num_adapters, a.seg_start,
                           a.seg_adapter, a.num_segments, a.M, a.d_out, ntiles_g, ntiles_m, a.scale, rm);
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_expand_t(const ExpandArgs &a, hipStream_t st) {
    return a.rows ? launch_expand_g<T, R, true>(a, st) : launch_expand_g<T, R, false>(a, st);
}

template <typename T, int R, bool kGather, bool kSmall>
static hipError_t launch_fused_g(const FusedArgs &a, hipStream_t st) {
    const FusedLayout L = fused_layout(a.M, a.d_in, a.d_out, a.r, a.dtype);
    const int tiles = Elem<T>::kMfma ? L.tiles : 0;
    const int units = Elem<T>::kMfma ? L.plan.units : 0;
    const int ntiles_g = gemv_col_tiles<T>(a.d_out);
    const int ntiles_m = tiles ? ceil_div(a.d_out, kExpandTileCols * expand_halves(!kSmall)) : 0;
    if (ntiles_g != L.copies) return hipErrorInvalidValue;  // one V copy per vector expand tile
    const unsigned grid = (unsigned)round_up_xcds(a.num_segments) * (R / kWavesPerBlock) +
                          (unsigned)(units ? mfma_shrink_items(units, L.plan.ks) : 0) +
                          (unsigned)a.num_segments * ntiles_g + (unsigned)round_up_xcds(tiles * ntiles_m);
    char *ws = static_cast<char *>(a.workspace);
    uint32_t *tile_c = reinterpret_cast<uint32_t *>(ws + L.tile_counters);
    hipLaunchKernelGGL((fused_kernel<T, R, kGather, kSmall>), dim3(grid), dim3(kBlock), 0, st,
                       reinterpret_cast<T *>(a.Y), reinterpret_cast<const T *>(a.X), a.A_ptrs,
                       a.B_ptrs, a.num_adapters, a.seg_start, a.seg_adapter, a.num_segments, a.M,
                       a.d_in, a.d_out, ntiles_g, ntiles_m, tiles, units, L.plan.ks, a.scale,
                       (int)((int64_t)a.M >= 16 * (int64_t)a.num_segments), tile_c,
                       reinterpret_cast<uint32_t *>(ws + L.split_counters),
                       reinterpret_cast<float *>(ws + L.v), reinterpret_cast<float *>(ws + L.vpairs),
                       reinterpret_cast<float *>(ws + L.partials), RowMap<kGather>{a.rows, a.M},
                       WaitCtl{reinterpret_cast<uint32_t *>(ws), wait_limit()});
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t st) {
    if constexpr (Elem<T>::kMfma) {
        if (!small_tiles(a.M, R))
            return a.rows ? launch_fused_g<T, R, true, false>(a, st) : launch_fused_g<T, R, false, false>(a, st);
    }
    return a.rows ? launch_fused_g<T, R, true, true>(a, st) : launch_fused_g<T, R, false, true>(a, st);
}

template <typename T, int R, bool kGather, bool kSmall>
static hipError_t launch_fused_layer_g(const LayerCall &a, hipStream_t st) {
    LayerArgs L{};
    L.num_projections = a.num_projections;
    char *ws = static_cast<char *>(a.workspace);
    L.wc = WaitCtl{reinterpret_cast<uint32_t *>(ws), wait_limit()};
    size_t ws_off = 0;
    int base = 0;
    for (int q = 0; q < a.num_projections; ++q) {
        const LayerProjIn &in = a.p[q];
        const FusedLayout FL = fused_layout(a.M, in.d_in, in.d_out, a.r, a.dtype);
        LayerProj &d = L.p[q];
        d.Y = in.Y;
        d.X = in.X;
        d.A_ptrs = in.A_ptrs;
        d.B_ptrs = in.B_ptrs;
        d.num_adapters = in.num_adapters;
        d.d_in = in.d_in;
        d.d_out = in.d_out;
        const int tiles = Elem<T>::kMfma ? FL.tiles : 0;
        const int units = Elem<T>::kMfma ? FL.plan.units : 0;
        d.ntiles_g = gemv_col_tiles<T>(in.d_out);
        if (d.ntiles_g != FL.copies) return hipErrorInvalidValue;  // one V copy per vector expand tile
        d.ntiles_m = tiles ? ceil_div(in.d_out, kExpandTileCols * expand_halves(!kSmall)) : 0;
        d.num_tiles = tiles;
        d.num_units = units;
        d.ks = FL.plan.ks;
        char *w = ws + ws_off;
        d.tile_counters = reinterpret_cast<uint32_t *>(w + FL.tile_counters);
        d.split_counters = reinterpret_cast<uint32_t *>(w + FL.split_counters);
        d.Vws = reinterpret_cast<float *>(w + FL.v);
        d.Vpairs = reinterpret_cast<float *>(w + FL.vpairs);
        d.partials = reinterpret_cast<float *>(w + FL.partials);
        d.items = round_up_xcds(a.num_segments) * (R / kWavesPerBlock) +
                  (units ? mfma_shrink_items(units, FL.plan.ks) : 0) + a.num_segments * d.ntiles_g +
                  round_up_xcds(tiles * d.ntiles_m);
        d.base = base;
        base += round_up_xcds(d.items);
        ws_off += align256(FL.total);
    }
    hipLaunchKernelGGL((fused_layer_kernel<T, R, kGather, kSmall>), dim3((unsigned)base), dim3(kBlock), 0, st, L,
                       a.seg_start, a.seg_adapter, a.num_segments, a.M, a.scale,
                       (int)((int64_t)a.M >= 16 * (int64_t)a.num_segments), RowMap<kGather>{a.rows, a.M});
    return hipGetLastError();
}

template <typename T, int R>
static hipError_t launch_fused_layer_t(const LayerCall &a, hipStream_t st) {
    if constexpr (Elem<T>::kMfma) {
        if (!small_tiles(a.M, R))
            return a.rows ? launch_fused_layer_g<T, R, true, false>(a, st)
                          : launch_fused_layer_g<T, R, false, false>(a, st);
    }
    return a.rows ? launch_fused_layer_g<T, R, true, true>(a, st) : launch_fused_layer_g<T, R, false, true>(a, st);
}

// Whether a bf16 batch can hold a segment long enough for the MFMA path:
// with every segment non-empty, the longest has M - N + 1 rows. Batches of
// decode tokens (one or a few rows per segment) cannot, and take kernels
// built without that path. Should empty segments leave a longer one after
// all, the vector path computes it.
static bool long_segments_possible(int M, int num_segments) {
    return (int64_t)M - num_segments + 1 >= kLongRows;
}

#ifdef SGMV_RANK
// One rank's entry points: this file is compiled once per rank (with
// -DSGMV_RANK=8, 16, 32, 64), so the rank's kernels build in parallel with
// the others'.
template <>
hipError_t launch_shrink_rank<SGMV_RANK>(const ShrinkArgs &a, hipStream_t st) {
    if (a.dtype == kF32) return launch_shrink_t<float, SGMV_RANK>(a, st);
    if (!long_segments_possible(a.M, a.num_segments)) return launch_shrink_t<bf16_short_t, SGMV_RANK>(a, st);
    return launch_shrink_t<bf16_t, SGMV_RANK>(a, st);
}

template <>
hipError_t launch_expand_rank<SGMV_RANK>(const ExpandArgs &a, hipStream_t st) {
    if (a.dtype == kF32) return launch_expand_t<float, SGMV_RANK>(a, st);
    if (!long_segments_possible(a.M, a.num_segments)) return launch_expand_t<bf16_short_t, SGMV_RANK>(a, st);
    return launch_expand_t<bf16_t, SGMV_RANK>(a, st);
}

template <>
hipError_t launch_fused_rank<SGMV_RANK>(const FusedArgs &a, hipStream_t st) {
    if (a.dtype == kF32) return launch_fused_t<float, SGMV_RANK>(a, st);
    if (!long_segments_possible(a.M, a.num_segments)) return launch_fused_t<bf16_short_t, SGMV_RANK>(a, st);
    return launch_fused_t<bf16_t, SGMV_RANK>(a, st);
}

template <>
hipError_t launch_fused_layer_rank<SGMV_RANK>(const LayerCall &a, hipStream_t st) {
    if (a.dtype == kF32) return launch_fused_layer_t<float, SGMV_RANK>(a, st);
    if (!long_segments_possible(a.M, a.num_segments))
        return launch_fused_layer_t<bf16_short_t, SGMV_RANK>(a, st);
    return launch_fused_layer_t<bf16_t, SGMV_RANK>(a, st);
}

#else  // the rank dispatch, the helper kernels and the process-wide settings

#define SGMV_RANK_SWITCH(FN, args, st)               \
    switch ((args).r) {                             \
        case 8: return FN<8>((args), (st));         \
        case 16: return FN<16>((args), (st));       \
        case 32: return FN<32>((args), (st));       \
        case 64: return FN<64>((args), (st));       \
        default: return hipErrorInvalidValue;       \
    }

hipError_t launch_shrink(const ShrinkArgs &a, hipStream_t st) { SGMV_RANK_SWITCH(launch_shrink_rank, a, st) }
hipError_t launch_expand(const ExpandArgs &a, hipStream_t st) { SGMV_RANK_SWITCH(launch_expand_rank, a, st) }
hipError_t launch_fused(const FusedArgs &a, hipStream_t st) { SGMV_RANK_SWITCH(launch_fused_rank, a, st) }
hipError_t launch_fused_layer(const LayerCall &a, hipStream_t st) {
    SGMV_RANK_SWITCH(launch_fused_layer_rank, a, st)
}

// ----------------------------------------------------------------------------
// The fused call without a caller-supplied workspace: its workspace is a
// file-scope device array, one per GPU the library runs on (each holds its
// own copy at its own address until the process ends). Host code never uses
// the array's name as an address: it looks the address up once per device
// with hipGetSymbolAddress and passes that pointer on.
// ----------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// One workgroup: if the scratch's status word says an earlier call failed,
// zero all of it (leftovers of that call may lie anywhere in it); otherwise
// every earlier call has left it zero and there is nothing to do. A kernel of
// its own, not a memset, so that the call can be captured in a graph.
__global__ __launch_bounds__(kBlock) void scratch_reset_kernel(uint4 *__restrict__ p, size_t vecs) {
    __shared__ uint32_t s_status;
    if (threadIdx.x == 0)
        s_status = __hip_atomic_load(reinterpret_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_status == 0) return;
    for (size_t i = threadIdx.x; i < vecs; i += kBlock) p[i] = make_uint4(0, 0, 0, 0);
}

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on first use per device).
static hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_fused_noalloc(FusedArgs a, hipStream_t st) {
    void *ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scratch_reset_kernel, dim3(1), dim3(kBlock), 0, st, static_cast<uint4 *>(ws),
                       kScratchBytes / sizeof(uint4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.workspace = ws;
    return launch_fused(a, st);
}

// How many polls a bounded wait makes before it gives up; read at each launch.
static std::atomic<uint32_t> g_wait_limit{kDefaultWaitLimit};

uint32_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
uint32_t set_wait_limit(uint32_t polls) { return g_wait_limit.exchange(polls, std::memory_order_relaxed); }

// Streaming read of `vecs` 16-byte vectors: the plain-kernel HBM ceiling the
// SGMV kernels are measured against. Four loads in flight per lane per
// step; the XOR of everything read goes to sink[block] so no load is dead.
__global__ __launch_bounds__(kBlock) void stream_probe_kernel(const uint4 *__restrict__ src, size_t vecs,
                                                             uint32_t *__restrict__ sink) {
    constexpr int U = 4;
    const size_t stride = (size_t)gridDim.x * kBlock;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    for (; i + (U - 1) * stride < vecs; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld16_stream(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < vecs; i += stride) {
        const uint4 v = ld16_stream(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t part[kWavesPerBlock];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) t ^= part[w];
        sink[blockIdx.x] = t;
    }
}

hipError_t launch_stream_probe(const void *src, size_t vecs, uint32_t *sink, int num_blocks, hipStream_t st) {
    hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)num_blocks), dim3(kBlock), 0, st,
                       static_cast<const uint4 *>(src), vecs, sink);
    return hipGetLastError();
}

// One pool slot's table entries, written by one lane (vector stores).
__global__ __launch_bounds__(kWave) void set_slot_kernel(uint64_t *A_ptrs, uint64_t *B_ptrs, int slot,
                                                        uint64_t a, uint64_t b) {
    if (threadIdx.x == 0) {
        A_ptrs[slot] = a;
        B_ptrs[slot] = b;
    }
}

hipError_t launch_set_slot(uint64_t *A_ptrs, uint64_t *B_ptrs, int slot, uint64_t a, uint64_t b,
                           hipStream_t st) {
    hipLaunchKernelGGL(set_slot_kernel, dim3(1), dim3(kWave), 0, st, A_ptrs, B_ptrs, slot, a, b);
    return hipGetLastError();
}

#endif  // SGMV_RANK

}  // namespace sgmv
