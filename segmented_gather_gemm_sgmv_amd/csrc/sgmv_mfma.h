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
//  * shrink tile: D = X_rows . A_k^T (d_in x r), fp32 accumulation, in one
//    of two tile kinds (see "Two shrink tiles" below): 16-row tiles whose
//    four waves split d_in (batches of up to 768 or 1024 rows), or 64-row tiles with
//    one wave per 16 rows sharing A_k through LDS (larger batches). Both
//    load X and A_k row-contiguously and reach the MFMA layout through LDS;
//    d_in may be split over several workgroups whose partial tiles are
//    summed in a fixed order.
//  * expand piece: D = V_rows (16 x r) . B_k (r x 128 columns). V is fp32 and
//    enters the A operand as two bf16 halves, hi = rne(v) and lo = rne(v - hi),
//    so hi + lo carries 16 significant bits; both halves meet the same B
//    operand. B_k is stored r x d_out (columns contiguous), so it is
//    transposed through LDS on its way in; the result is staged through LDS
//    so that Y is read and written in whole 16-byte vectors per lane. A
//    workgroup takes one or two 128-column halves of a 64-row tile.
#pragma once

#include "sgmv_common.h"

namespace sgmv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kLongRows = 16;           // segments this long or longer take the MFMA path
constexpr int kTileRows = 64;           // batch rows per MFMA tile (4 waves x 16)
constexpr int kExpandTileCols = 128;    // d_out columns per expand tile half
// 128-column halves per MFMA expand workgroup: two in the fused launch of a
// batch of many tiles (prefill), where fewer, longer workgroups wait once
// for the loads of both halves; one elsewhere, where more workgroups in
// flight matter more.
__host__ __device__ constexpr int expand_halves(bool fused_many_tiles) { return fused_many_tiles ? 2 : 1; }
constexpr int kMaxPieces = 8;           // long segments one window of a tile can meet

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroups are dealt to the 8 XCDs of the chip round-robin by id, and each
// XCD has its own L2. Remap a run of `count` MFMA items (the first at
// workgroup id `first_id`) so that each XCD gets a contiguous block of item
// indices: consecutive row tiles belong to the same segments and re-read the
// same adapter, which then stays in one L2. Returns -1 for the padding ids
// (the run is launched rounded up to a multiple of 8).
constexpr int kXcds = 8;
__host__ __device__ constexpr int round_up_xcds(int n) { return (n + kXcds - 1) / kXcds * kXcds; }
// `id`: the workgroup's item id, congruent to its workgroup id modulo 8
// (itself, or its offset inside a launch region that starts at a multiple
// of 8).
__device__ __forceinline__ int xcd_local_item(int id, int first_id, int count) {
    const int j = id - first_id;
    const int per = (count + kXcds - 1) / kXcds;
    const int item = (id % kXcds) * per + j / kXcds;
    return item < count ? item : -1;
}
__device__ __forceinline__ int xcd_local_item(int first_id, int count) {
    return xcd_local_item((int)blockIdx.x, first_id, count);
}

__device__ __forceinline__ int clamp_to(int v, int M) { return v < 0 ? 0 : (v > M ? M : v); }

// Number of offsets p in [0, num_segments] with clamp(seg_start[p]) <= t, by a
// workgroup-wide search that tests kBlockThreads pivots per round (offsets
// are non-decreasing). With kPivot0 the first round's pivot of this thread,
// offset tid * (num_segments / kBlockThreads + 1) clamped to num_segments,
// comes in already loaded (`pivot0`). Every thread returns the same value.
template <bool kPivot0>
__device__ int count_starts_le(const int32_t *seg_start, int num_segments, int M, int t, int pivot0) {
    int base = 0, len = num_segments + 1;
    for (int round = 0; len > 0; ++round) {
        const int stride = (len + kBlockThreads - 1) / kBlockThreads;
        const int off = (int)threadIdx.x * stride;
        const bool pred = off < len && clamp_to(kPivot0 && round == 0 ? pivot0 : seg_start[base + off], M) <= t;
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
    int more, next;
    int starts[kBlockThreads + 1];
    int ids[kBlockThreads];
};

__device__ __forceinline__ void consider_segment(PieceList &pl, int s, int lo, int hi, int k,
                                                 int num_adapters, int t0, int t1) {
    if (hi - lo >= kLongRows && lo < t1 && hi > t0 && k >= 0 && k < num_adapters) {
        const int slot = atomicAdd(&pl.n, 1);
        if (slot < kMaxPieces) pl.p[slot] = Piece{max(lo, t0), min(hi, t1), s, k};
    }
}

// Order LDS accesses across the workgroup without waiting for outstanding
// global loads (a full barrier would also wait for every load in flight).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// This thread's entries of the segment metadata, requested as early as
// possible (N >= 1 segments): the offset that is its first-round pivot in
// count_starts_le, index min(tid * (N / kBlockThreads + 1), N), i.e. index
// min(tid, N) when N < kBlockThreads, and adapter id min(tid, N - 1). Loads
// return in issue order, so metadata requested before a tile's bulk loads
// is not held up behind them.
struct SegPrefetch {
    int start, id;
};

__device__ __forceinline__ SegPrefetch prefetch_segments(const int32_t *seg_start,
                                                         const int32_t *seg_adapter,
                                                         int num_segments) {
    // Kept here the same way as the adapter table loads: otherwise the
    // compiler sinks them to their use, behind the tile's bulk loads.
    // Global (not flat) loads: a flat load would make its consumer wait for
    // the LDS counter too, and with it for every load in flight.
    asm volatile("" : "+s"(seg_start), "+s"(seg_adapter));
    typedef __attribute__((address_space(1))) const int32_t gconst_i32_t;
    const int tid = threadIdx.x;
    const int stride = num_segments / kBlockThreads + 1;
    const SegPrefetch p{((gconst_i32_t *)seg_start)[min(tid * stride, num_segments)],
                        ((gconst_i32_t *)seg_adapter)[min(tid, num_segments - 1)]};
    asm volatile("" ::: "memory");
    return p;
}

// Collect into `pl` the long segments (with a valid adapter) that intersect
// rows [t0, t1) of the batch. With up to kBlockThreads - 1 segments all the
// offsets and ids come in with one load per thread (already in `pre` when
// kPrefetched, and then the workgroup synchronises through LDS only,
// leaving loads in flight). Otherwise the segment holding row t0 is found by
// a k-ary search (its first round's pivots in `pre` when kPrefetched) and
// the offsets are scanned in windows of kWave segments until one starts at
// or past t1. With valid (non-decreasing) offsets at most five long segments
// meet a tile; pieces beyond kMaxPieces (possible only with invalid offsets)
// are dropped. Call with the whole workgroup; pl is visible to all threads
// on return.
template <bool kPrefetched>
__device__ void gather_pieces(PieceList &pl, const SegPrefetch &pre, const int32_t *seg_start,
                              const int32_t *seg_adapter, int num_segments, int num_adapters, int M,
                              int t0, int t1) {
    const int tid = threadIdx.x;
    if (num_segments < kBlockThreads) {
        if (tid == 0) pl.n = 0;
        if (tid <= num_segments) pl.starts[tid] = clamp_to(kPrefetched ? pre.start : seg_start[tid], M);
        if (tid < num_segments) pl.ids[tid] = kPrefetched ? pre.id : seg_adapter[tid];
        if constexpr (kPrefetched)
            lds_barrier();
        else
            __syncthreads();
        if (tid < num_segments) {
            const int lo = pl.starts[tid];
            consider_segment(pl, tid, lo, max(lo, pl.starts[tid + 1]), pl.ids[tid], num_adapters, t0, t1);
        }
        lds_barrier();
        if (tid == 0 && pl.n > kMaxPieces) pl.n = kMaxPieces;
        lds_barrier();
        return;
    }
    const int cnt = count_starts_le<kPrefetched>(seg_start, num_segments, M, t0, pre.start);
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
                if (hi - lo >= kLongRows && lo < t1 && hi > t0)
                    consider_segment(pl, s, lo, hi, seg_adapter[s], num_adapters, t0, t1);
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
// Two shrink tiles. A batch of many tiles (a prefill batch) takes 64-row
// tiles: the A_k chunk of a step is shared by the four waves (each owns 16
// rows) through LDS, so A_k crosses the L1 once per 64 rows, and d_in is
// split between workgroups to fill the chip. A batch of few tiles (a few
// mid-length segments) takes 16-row tiles with the four waves splitting
// d_in: A_k crosses the L1 once per 16 rows, which matters little at r <= 32
// and few tiles, and there is no cross-workgroup combine on the way to V.
// ----------------------------------------------------------------------------
// ----------------------------------------------------------------------------
// 16-row shrink tile (batches of few tiles): V[m, 0:R] = X[m, :] . A_k for
// the rows m of one piece (a long
// segment's rows inside the tile) of the 16-row tile starting at t0, over
// the steps [s_begin, s_end) of d_in (ShrinkSmem<R>::kStepK elements each). The tile size follows the
// segments: a 16-row tile wastes at most 15 rows at a segment's end, where a
// 64-row tile (prefill-sized) would waste up to 63 and leave too few tiles to
// spread a few mid-length segments over the chip.
//
// The four waves split the steps between them (wave w takes the w-th
// contiguous quarter) and each keeps its own 16 x R partial tile; the
// partials meet in LDS once, at the end, and are summed in the fixed order of
// the waves. No wave waits for another inside the loop.
//
// Loads are row-contiguous: in a step, 16 lanes cover the 256 bytes of one
// row (X row or A_k rank row), so each load instruction reads four whole
// row chunks. (Loading straight into the MFMA operand layout would make
// every instruction touch 16 rows, 64 bytes each, 8 KB apart, which streams
// several times slower.) Each wave stages its step in its own LDS buffer,
// chunk c of row rho in slot c ^ (rho % 16), and reads the operands back in
// the MFMA layout: in slice q (elements 32 q .. 32 q + 31 of the step) lane
// (i, g) takes chunk 4 q + g of X row i and of A_k rank row 16 b + i. The
// XOR makes both the writes (16 lanes per row, a permutation of its slots)
// and the reads (16 rows, distinct slots) free of bank conflicts. LDS
// operations of one wave complete in order, so the wave needs no barrier
// between writing its buffer and reading it, nor before rewriting it.
//
// kStages steps are in flight per lane in a ring of registers. Every load is
// unconditional: a chunk past d_in or a step past the wave's range loads a
// clamped address and is staged as zeros (for X and A_k alike, so that a
// non-finite value cannot leak into the sum); rows outside the piece load a
// row of the piece and are never stored.
// ----------------------------------------------------------------------------
constexpr int kShrinkRows = 16;   // rows of an MFMA shrink tile (one MFMA's M)

template <int R>
struct ShrinkSmem {
    static constexpr int kNB = R < 16 ? 1 : R / 16;                 // 16-column MFMA blocks of V
    // Blocks one workgroup computes: at most two (32 columns), so that r = 64
    // takes two workgroups per tile, each reading X and half of A_k: enough
    // work items to fill the chip, and an 80-row step would need more
    // registers and LDS than leave two workgroups per CU.
    static constexpr int kNBW = kNB < 2 ? kNB : 2;
    static constexpr int kGroups = kNB / kNBW;                      // column groups per tile
    static constexpr int kRows = kShrinkRows + 16 * kNBW;           // staged rows: X, then A_k
    static constexpr int kStepK = 128;                              // d_in elements per step
    static constexpr int kCpr = kStepK / 8;                         // 16-byte chunks per row and step
    static constexpr int kRpi = kWave / kCpr;                       // rows per load instruction
    static constexpr int kLoads = kRows / kRpi;                     // row-contiguous loads per lane and step
    static constexpr int kStages = kLoads <= 8 ? 4 : 3;             // steps in flight
    static constexpr int kWaves = kBlockThreads / kWave;
    union {
        uint4 stage[kWaves][kRows * kCpr];      // each wave's staged step
        f32x4_t part[kWaves][kNBW][kWave];      // each wave's partial tile, after the loop
    };
};

template <int NL>
struct ShrinkStage {
    uint4 v[NL];     // rows kRpi l + lane / kCpr (l < NL), chunk lane % kCpr
    uint32_t keep;   // all ones if the chunk lies inside d_in and the step inside the wave's range, else 0
};

// One wave's partial tile over its steps, for the 16 kNBW columns of column
// group cg; acc is in the MFMA D layout (lane (i, g) holds rows 4 g + v,
// v < 4, of column 16 (kNBW cg + b) + i).
template <int R, typename RM>
__device__ __forceinline__ void shrink_wave_mfma(const bf16_t *X, const bf16_t *Ak, int d_in, int t0, int lo,
                                                 int hi, int cg, int s_begin, int s_end, ShrinkSmem<R> &sm,
                                                 f32x4_t (&acc)[ShrinkSmem<R>::kNBW], RM rm) {
    using SM = ShrinkSmem<R>;
    constexpr int NB = SM::kNBW;
    constexpr int NL = SM::kLoads;
    constexpr int S = SM::kStages;
    constexpr int W = SM::kWaves;
    constexpr int CPR = SM::kCpr;
    constexpr int RPI = SM::kRpi;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int per = (s_end - s_begin + W - 1) / W;
    const int first = s_begin + wave * per;
    const int niter = max(0, min(per, s_end - first));  // uniform per wave
    if (niter == 0) return;
    const int last = first + niter - 1;
    // row of load l: RPI l + lane / CPR; X rows first (16), then A_k rank rows
    const int c = lane % CPR;
    const bf16_t *src[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int rho = RPI * l + lane / CPR;
        src[l] = rho < kShrinkRows ? X + (size_t)rm(min(max(t0 + rho, lo), hi - 1)) * d_in
                                   : Ak + (size_t)min(16 * NB * cg + rho - kShrinkRows, R - 1) * d_in;
    }
    uint4 *const buf = sm.stage[wave];

    auto load = [&](ShrinkStage<NL> &st, int it) {
        const int step = first + it;
        const int e = min(step, last) * SM::kStepK + 8 * c;  // steps past the end reload the last step
        const bool ok = step <= last && e < d_in;
        const int ec = ok ? e : d_in - 8;                     // d_in >= 8: always inside the row
        st.keep = ok ? ~0u : 0u;
#pragma unroll
        for (int l = 0; l < NL; ++l) st.v[l] = ld16(src[l] + ec);
    };
    auto consume = [&](const ShrinkStage<NL> &st) {
        // masked word by word: a select between whole vectors would make the
        // compiler pick between their addresses and keep the ring in scratch
        const uint32_t k = st.keep;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int rho = RPI * l + lane / CPR;
            buf[rho * CPR + (c ^ (rho % CPR))] =
                make_uint4(st.v[l].x & k, st.v[l].y & k, st.v[l].z & k, st.v[l].w & k);
        }
        const int i = lane & 15, g = lane >> 4;
#pragma unroll
        for (int q = 0; q < SM::kStepK / 32; ++q) {
            const int ch = 4 * q + g;
            const bf16x8_t xo = as_bf16x8(buf[i * CPR + (ch ^ (i % CPR))]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int rho = kShrinkRows + 16 * b + i;
                acc[b] = mfma_bf16(xo, as_bf16x8(buf[rho * CPR + (ch ^ (rho % CPR))]), acc[b]);
            }
        }
    };

    // The memory counter retires loads in issue order: scheduling barriers
    // keep each step's loads together, so staging the oldest step waits for
    // that step only.
    ShrinkStage<NL> ring[S];
#pragma unroll
    for (int u = 0; u < S - 1; ++u) {
        load(ring[u], u);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int it0 = 0; it0 < niter; it0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            load(ring[(u + S - 1) % S], it0 + u + S - 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(ring[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The whole workgroup: the tile's result for one piece (rows lo .. hi - 1,
// adapter Ak) and column group cg, summed over the waves' partials in wave
// order. On return, thread f < kNBW * 64 holds fragment f = 64 b + lane
// (rows t0 + 4 g + v, column 16 (kNBW cg + b) + i, with g, i from lane) in
// res for the rows of the piece; other rows of res are left as they were.
// Ends with the LDS free again.
template <int R, typename RM>
__device__ __forceinline__ void shrink_tile_mfma(const bf16_t *X, const bf16_t *Ak, int d_in, int t0, int lo,
                                                 int hi, int cg, int s_begin, int s_end, ShrinkSmem<R> &sm,
                                                 f32x4_t &res, RM rm) {
    constexpr int NB = ShrinkSmem<R>::kNBW;
    constexpr int W = ShrinkSmem<R>::kWaves;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    f32x4_t acc[NB];
    shrink_wave_mfma<R>(X, Ak, d_in, t0, lo, hi, cg, s_begin, s_end, sm, acc, rm);
    __syncthreads();  // every wave is done with its staging buffer, which the partials reuse
#pragma unroll
    for (int b = 0; b < NB; ++b) sm.part[wave][b][lane] = acc[b];
    __syncthreads();
    const int f = threadIdx.x;
    if (f < NB * kWave) {
        f32x4_t sum = sm.part[0][f / kWave][f % kWave];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += sm.part[w][f / kWave][f % kWave];
        const int g = (f % kWave) >> 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = t0 + 4 * g + v;
            if (m >= lo && m < hi) res[v] = sum[v];
        }
    }
    __syncthreads();
}

// ----------------------------------------------------------------------------
// 64-row shrink tile (batches of many tiles, such as prefill): V[m, 0:R] =
// X[m, :] . A_k for the rows m of up to two pieces
// (segments, each with its own adapter) of the 64-row tile starting at t0,
// over macro steps [ms_begin, ms_end) of d_in (kMacroK elements each). Wave w
// owns rows t0 + 16 w .. + 15 and all R columns, so the waves share the A_k
// chunk of a macro step (R rows x kMacroK): it is loaded once per workgroup,
// 16 lanes per 256-byte row chunk (whole cache lines), and handed to the
// waves through LDS. X rows go straight into registers: in slice q of a
// macro step, lane (i, g) brings elements 32 q + 8 g .. + 7 of its row, and
// reads the same elements of A_k rows 16 b + i from LDS. kStages macro steps
// are in flight per lane (a ring of registers); LDS holds two A_k chunks per
// piece, the one being read and the one being written.
//
// A tile that meets two segments takes both in one pass over d_in: X is
// loaded once, both adapters' chunks are staged, and each wave multiplies
// its rows by the adapter of every piece those rows touch, into one
// accumulator set per piece. A row keeps the accumulator of its own piece,
// so another adapter's values never reach it.
//
// LDS layout of an A_k chunk: row j occupies 16 slots of 16 bytes; element
// chunk c (elements 8 c .. 8 c + 7 of the macro step) of row j sits in slot
// c ^ (j % 16). The 16 lanes that read one chunk index from 16 different rows
// then hit 16 different slots, i.e. different banks.
// ----------------------------------------------------------------------------
constexpr int kShrinkTileRows = 64;   // rows of a 64-row shrink tile (batches of many tiles)
constexpr int kMacroK = 128;
constexpr int kChunksPerRow = kMacroK * 2 / 16;   // 16-byte chunks per A_k row of a macro step
template <int R>
struct Shrink64Smem {
    static constexpr int kNB = R < 16 ? 1 : R / 16;                   // 16-column MFMA blocks
    static constexpr int kALoads = R * kChunksPerRow < kBlockThreads ? 1 : R * kChunksPerRow / kBlockThreads;
    static constexpr int kStages = R >= 64 ? 2 : (R >= 32 ? 3 : 4);   // macro steps in flight
    // Pieces one pass over d_in can take. At r = 64 a pass takes one: two
    // pieces' A_k chunks would need 64 KB of LDS, leaving room for one
    // workgroup per CU; a tile that meets two segments then reads X twice.
    static constexpr int kPassPieces = R >= 64 ? 1 : 2;
    uint4 a[2][kPassPieces][R * kChunksPerRow];
    uint4 xs[kBlockThreads / 64][16 * kChunksPerRow];  // each wave's X rows of a step, staged
};

template <int R, int NP>
struct Shrink64Stage {
    uint4 a[NP][Shrink64Smem<R>::kALoads];  // this thread's A_k chunks, per piece
    uint4 x[4];                           // this lane's X chunks: rows 4 q + lane / 16, chunk lane % 16
    uint32_t ok;                          // bits 0..3: X chunk inside d_in; bits 4..: A chunk inside d_in
};

// Pieces lo[p] .. hi[p] - 1 (p < NP) are disjoint row ranges inside the tile,
// Ak[p] their adapters; rm maps a segment row to the row of X it reads. On return, res[b][v] of lane (i, g) of wave w holds
// the tile's result for row t0 + 16 w + 4 g + v and column 16 b + i (the MFMA
// D layout) wherever that row lies in a piece; elsewhere res is left as it
// was.
template <int R, int NP, typename RM>
__device__ void shrink_tile64_mfma(const bf16_t *X, const bf16_t *const (&Ak)[NP], int d_in, int t0,
                                 const int (&lo)[NP], const int (&hi)[NP], int ms_begin, int ms_end,
                                 Shrink64Smem<R> &sm, f32x4_t (&res)[Shrink64Smem<R>::kNB], RM rm) {
    constexpr int NB = Shrink64Smem<R>::kNB;
    constexpr int kALoads = Shrink64Smem<R>::kALoads;
    constexpr int S = Shrink64Smem<R>::kStages;
    constexpr int kAChunks = R * kChunksPerRow;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int g = lane >> 4;
    const int i = lane & 15;
    const int row = t0 + 16 * wave + i;
    int rlo = lo[0], rhi = hi[0];
    bool touches[NP];  // uniform per wave: the wave's 16 rows meet piece p
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        rlo = min(rlo, lo[p]);
        rhi = max(rhi, hi[p]);
        touches[p] = t0 + 16 * wave < hi[p] && t0 + 16 * wave + 16 > lo[p];
    }
    // X is loaded row-contiguously: in load q of a step, lane l takes chunk
    // l % 16 (8 elements) of the wave's row 4 q + l / 16, so one instruction
    // reads four whole 256-byte row segments (loads straight into the MFMA
    // layout would touch 16 rows, 64 bytes each). The wave stages the step
    // in its own LDS buffer, chunk c of row rho in slot c ^ rho, and reads it
    // back in the MFMA layout. Rows outside the pieces are never stored; rm
    // gives the token row.
    (void)row;
    const int xc = lane & 15;
    const bf16_t *xrows[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        xrows[q] = X + (size_t)rm(min(max(t0 + 16 * wave + 4 * q + (lane >> 4), rlo), rhi - 1)) * d_in;
    // Every step of the loop is straight-line: a step past ms_end (padding to
    // a multiple of S) or a slice past d_in loads a clamped address and its
    // operands are zeroed, never skipped, so each group of loads stays in
    // flight until its turn.
    const int niter = (ms_end - ms_begin + S - 1) / S * S;

    auto load = [&](Shrink64Stage<R, NP> &st, int it) {
        const int ms = ms_begin + it;
        const bool step_ok = ms < ms_end;
        const int kb = max(0, min(ms, ms_end - 1)) * kMacroK;  // an empty range loads step 0
        st.ok = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = kb + 8 * xc;
            const bool ok = step_ok && k < d_in;
            st.ok |= (uint32_t)ok << q;
            st.x[q] = ld16_stream(xrows[q] + (ok ? k : d_in - 8));
        }
#pragma unroll
        for (int u = 0; u < kALoads; ++u) {
            const int id = min(u * kBlockThreads + tid, kAChunks - 1);  // R = 8: half the threads repeat
            const int k = kb + 8 * (id % kChunksPerRow);
            const bool ok = step_ok && k < d_in;
            st.ok |= (uint32_t)ok << (4 + u);
            const size_t off = (size_t)(id / kChunksPerRow) * d_in + (ok ? k : d_in - 8);
#pragma unroll
            for (int p = 0; p < NP; ++p) st.a[p][u] = ld16(Ak[p] + off);
        }
    };

    f32x4_t acc[NP][NB];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[p][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Consume one stage: its A_k chunks go to LDS buffer `buf`, then every
    // wave multiplies its X slices with the chunk of each piece it touches.
    auto consume = [&](const Shrink64Stage<R, NP> &st, int buf) {
        // this wave's X rows first: LDS operations of a wave complete in
        // order, so its reads below see them without a barrier
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rho = 4 * q + (lane >> 4);
            sm.xs[wave][rho * kChunksPerRow + (xc ^ rho)] = ((st.ok >> q) & 1u) ? st.x[q] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kALoads; ++u) {
            const int id = u * kBlockThreads + tid;
            if (id < kAChunks) {
                const int j = id / kChunksPerRow;
                const int c = id % kChunksPerRow;
                const bool ok = (st.ok >> (4 + u)) & 1u;
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    sm.a[buf][p][j * kChunksPerRow + (c ^ (j & 15))] = ok ? st.a[p][u] : make_uint4(0, 0, 0, 0);
            }
        }
        lds_barrier();
        uint4 xq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xq[q] = sm.xs[wave][i * kChunksPerRow + ((4 * q + g) ^ i)];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (NP > 1 && !touches[p]) continue;  // uniform
            // The A operands of slice q + 1 are requested from LDS before
            // the MFMAs of slice q are issued, so LDS latency overlaps the
            // math instead of preceding every instruction.
            auto lds_slice = [&](uint4 (&av)[NB], int q) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int j = min(16 * b + i, R - 1);  // columns past R are never stored
                    av[b] = sm.a[buf][p][j * kChunksPerRow + ((4 * q + g) ^ (j & 15))];
                }
            };
            uint4 av[2][NB];
            lds_slice(av[0], 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q + 1 < 4) lds_slice(av[(q + 1) & 1], q + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[p][b] = mfma_bf16(as_bf16x8(xq[q]), as_bf16x8(av[q & 1][b]), acc[p][b]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // The memory counter retires loads in issue order: scheduling barriers
    // keep each step's group of loads together, so consuming the oldest
    // group waits for that group only.
    Shrink64Stage<R, NP> ring[S];
#pragma unroll
    for (int u = 0; u < S - 1; ++u) {
        load(ring[u], u);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int it0 = 0; it0 < niter; it0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            load(ring[(u + S - 1) % S], it0 + u + S - 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(ring[u], (it0 + u) & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    lds_barrier();  // the LDS buffers are free for whatever comes next

#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = t0 + 16 * wave + 4 * g + v;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const bool in_piece = m >= lo[p] && m < hi[p];
#pragma unroll
            for (int b = 0; b < NB; ++b) res[b][v] = in_piece ? acc[p][b][v] : res[b][v];
        }
    }
}

// Device-scope (agent) 16-byte loads and stores through a buffer resource:
// the partial tiles of a split shrink are written by one workgroup and read
// by another, possibly on another XCD, so they bypass the non-coherent
// caches. The resource also bounds every access to [base, base + bytes).
constexpr int kCoherentPolicy = 16;  // cache policy bits: device scope
typedef uint32_t u32x4_t_ __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(float *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4_t load4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherentPolicy));
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t_, v), r, byte_off, 0, kCoherentPolicy);
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
    // The delta tile is staged over the B tile once every MFMA has read it,
    // which leaves room for three workgroups per CU.
    union __attribute__((aligned(16))) {
        uint16_t bt[kExpandTileCols * kBtStride];                // B tile, [n][k]
        uint4 bt16[kExpandTileCols * kBtStride / 8];             // the same, 16-byte vectors
        float ys[kTileRows * kYsStride];                         // delta tile, [m][n]
    };
    static_assert(kBtStride % 8 == 0, "B tile rows must be whole 16-byte vectors");
    // Position of the 16-byte chunk c (rank elements 8c .. 8c + 7) in row n:
    // the chunks of a row are permuted by n / 8. A thread transposes eight
    // consecutive columns (rows n = 8 c8 + e) at once, so without the
    // permutation the 16 threads of a wave writing rows 8 c8 + e (same e)
    // would all hit one LDS bank.
    static __device__ __forceinline__ int chunk(int n, int c) { return c ^ ((n >> 3) & (kK / 8 - 1)); }
};

__device__ __forceinline__ uint32_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Expand tile: Y[m, n0:n0+128 NT] += scale * V[m, :] . B_k[:, n0:n0+128 NT]
// for the rows m of every piece (segment with its adapter) of the 64-row
// tile at t0, taken as NT column halves of 128 that share the tile's V,
// pieces and rows. With kEarly the Y tile, and V when kVEarly, are requested
// before the tile's pieces are known, so the segment metadata round trip
// overlaps theirs (`gather()` collects the pieces into pl, from metadata the
// caller requested before anything else). That pays when most tiles have
// pieces; in a batch of short segments most tiles have none, and then the
// early loads would be wasted, so without kEarly they wait for the pieces.
// Pieces are taken one after another: the B_k tiles of all NT halves are
// requested together, then each half in turn is staged, multiplied and
// added into its part of the Y tile held in registers; the tile is stored
// once at the end. A workgroup thus waits once for the loads of NT halves.
//
// `ready()` is called by every thread once the first B tile is on its way
// and before V is read (a consumer of V produced in the same launch waits
// there); if it returns false the tile is left untouched.
// kVEarly: V is final before the launch (a separate shrink), so it is
// requested together with Y.
// load_v4(idx): V[idx .. idx + 3] (idx a multiple of 4).
// rm(p, ok): the row of Y that segment row p updates (never stored if !ok).
template <int R, int NT, bool kVEarly, bool kEarly, typename Gather, typename BkOf, typename LoadV4, typename Ready,
          typename RM>
__device__ __forceinline__ void expand_tile_mfma(bf16_t *Y, int M, int d_out, int t0, int n0, float scale,
                                 ExpandSmem<R> &sm, const PieceList &pl, Gather gather, BkOf bk_of,
                                 LoadV4 load_v4, Ready ready, RM rm) {
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
    const int t1 = min(t0 + kTileRows, M);
    int nh = 0;  // halves inside d_out (uniform)
#pragma unroll
    for (int h = 0; h < NT; ++h) nh += n0 + h * kExpandTileCols < d_out;

    // The Y tile: each thread owns kYPer vectors of 8 per half. Rows past the
    // batch and columns past d_out load a clamped address and are never
    // stored.
    constexpr int kYPer = kTileRows * kColVecs / kBlockThreads;
    uint4 yv[NT][kYPer];
    int yrow[kYPer];    // row of Y behind each vector (the same in every half)
    uint32_t yok = 0;   // bit q: yrow[q] may be stored
    auto fetch_y = [&]() {
#pragma unroll
        for (int q = 0; q < kYPer; ++q) {
            const int idx = tid + q * kBlockThreads;
            bool ok;
            yrow[q] = rm(min(t0 + idx / kColVecs, t1 - 1), ok);
            yok |= (uint32_t)ok << q;
#pragma unroll
            for (int h = 0; h < NT; ++h) {
                const int n = n0 + h * kExpandTileCols + (idx % kColVecs) * 8;
                yv[h][q] = ld16(Y + (size_t)yrow[q] * d_out + (n < d_out ? n : 0));
            }
        }
    };

    // V rows of this wave (A operand): lane (i, g) needs columns
    // ks * 32 + 8 g .. + 7 of row t0 + 16 w + i. Fetched raw first, then split
    // into bf16 hi/lo halves once the values are needed. Rows outside the
    // pieces are never stored; rank columns past R meet zero rows of the
    // staged B tile but are zeroed anyway so a non-finite value cannot leak
    // into a valid row.
    const int vrow = min(t0 + 16 * wave + i, t1 - 1);
    float vraw[KS][8];
    auto fetch_v = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = ks * 32 + 8 * g + 4 * h;
                const float4 v = load_v4((size_t)vrow * R + min(j, R - 4));
                const bool ok = j < R;
                vraw[ks][4 * h + 0] = ok ? v.x : 0.f;
                vraw[ks][4 * h + 1] = ok ? v.y : 0.f;
                vraw[ks][4 * h + 2] = ok ? v.z : 0.f;
                vraw[ks][4 * h + 3] = ok ? v.w : 0.f;
            }
    };
    bf16x8_t ahi[KS], alo[KS];
    auto split_v = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint32_t h[4], l[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float v0 = vraw[ks][2 * e2], v1 = vraw[ks][2 * e2 + 1];
                const uint32_t hb0 = bf16_bits(v0), hb1 = bf16_bits(v1);
                const float r0 = v0 - __uint_as_float(hb0 << 16);
                const float r1 = v1 - __uint_as_float(hb1 << 16);
                h[e2] = hb0 | (hb1 << 16);
                l[e2] = bf16_bits(r0) | (bf16_bits(r1) << 16);
            }
            ahi[ks] = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
            alo[ks] = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
        }
    };
    if constexpr (kEarly) {
        fetch_y();
        if constexpr (kVEarly) fetch_v();
        gather();
    } else {
        gather();
        if (pl.n == 0) return;  // uniform
        fetch_y();
        if constexpr (kVEarly) fetch_v();
    }
    // B tile of one half: thread tid holds, for each of its (rank-row pair,
    // column vector) items, the two rank rows' 16-byte vectors.
    constexpr int kBItems = (R / 2) * kColVecs;
    constexpr int kBPer = (kBItems + kBlockThreads - 1) / kBlockThreads;
    auto load_b = [&](uint4 (&bq)[NT][kBPer][2], int k) {
        const bf16_t *Bk = bk_of(k);
#pragma unroll
        for (int h = 0; h < NT; ++h)
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int idx = min(tid + u * kBlockThreads, kBItems - 1);  // repeats are never staged
                const int jp = idx / kColVecs;
                const int n = n0 + h * kExpandTileCols + (idx % kColVecs) * 8;
                const int nc = n < d_out ? n : 0;  // columns past d_out are never stored
                bq[h][u][0] = ld16(Bk + (size_t)(2 * jp) * d_out + nc);
                bq[h][u][1] = ld16(Bk + (size_t)(2 * jp + 1) * d_out + nc);
            }
    };
    // In a batch of short segments (no kEarly; the pieces are known here and
    // a tile often meets several) the next piece's B tile is requested while
    // this piece is worked on, so a tile waits once for B, not once per
    // piece. The last piece asks for its own tile again (a cache hit): the
    // request stays unconditional, which keeps the compiler from waiting for
    // it where a branch around it would end.
    constexpr bool kAhead = !kEarly && NT == 1;
    uint32_t touched = 0;  // bit q: Y vector q belongs to a piece
    uint4 bq[NT][kBPer][2];
    if constexpr (kAhead) load_b(bq, pl.p[0].k);
    for (int pi = 0; pi < pl.n; ++pi) {
        const Piece pc = pl.p[pi];
        uint4 bn[NT][kBPer][2];
        if constexpr (kAhead)
            load_b(bn, pl.p[min(pi + 1, pl.n - 1)].k);
        else
            load_b(bq, pc.k);
#pragma unroll
        for (int h = 0; h < NT; ++h) {
            if (h >= nh) break;  // uniform
            // B tile -> LDS, transposed: two rank rows per pass, packed as pairs.
#pragma unroll
            for (int u = 0; u < kBPer; ++u) {
                const int idx = tid + u * kBlockThreads;
                if (idx >= kBItems) continue;
                const int jp = idx / kColVecs;
                const int c8 = idx % kColVecs;
                const uint4 r0 = bq[h][u][0], r1 = bq[h][u][1];
                const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
                const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo16 = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
                    const uint32_t hi16 = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xffffu);
                    const int n = c8 * 8 + e;
                    *reinterpret_cast<uint32_t *>(&sm.bt[n * kBt + 8 * ExpandSmem<R>::chunk(n, jp >> 2) +
                                                         2 * (jp & 3)]) = lo16 | (hi16 << 16);
                }
            }
            if constexpr (R < K) {  // zero the padded part of the reduction
                for (int idx = tid; idx < kExpandTileCols * (K - R); idx += kBlockThreads) {
                    const int n = idx / (K - R), k = R + idx % (K - R);
                    sm.bt[n * kBt + 8 * ExpandSmem<R>::chunk(n, k >> 3) + (k & 7)] = 0;
                }
            }
            if (pi == 0 && h == 0) {
                if (!ready()) return;  // uniform
                if constexpr (!kVEarly) fetch_v();
                split_v();
            }
            __syncthreads();  // B tile in LDS

            // All B operands first, then eight independent accumulator chains, so
            // neither LDS nor MFMA latency sits between consecutive instructions.
            constexpr int NBLK = kExpandTileCols / 16;
            uint4 bv[KS][NBLK];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
                    bv[ks][b] = sm.bt16[((16 * b + i) * kBt + 8 * ExpandSmem<R>::chunk(16 * b + i, 4 * ks + g)) / 8];
            f32x4_t acc[NBLK];
#pragma unroll
            for (int b = 0; b < NBLK; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int b = 0; b < NBLK; ++b) acc[b] = mfma_bf16(ahi[ks], as_bf16x8(bv[ks][b]), acc[b]);
#pragma unroll
                for (int b = 0; b < NBLK; ++b) acc[b] = mfma_bf16(alo[ks], as_bf16x8(bv[ks][b]), acc[b]);
            }
            __syncthreads();  // every wave is done with the B tile, whose LDS the delta tile reuses
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) sm.ys[(16 * wave + 4 * g + v) * kYs + 16 * b + i] = acc[b][v];
            __syncthreads();  // delta tile in LDS

#pragma unroll
            for (int q = 0; q < kYPer; ++q) {
                const int idx = tid + q * kBlockThreads;
                const int r = idx / kColVecs;
                const int c8 = idx % kColVecs;
                const int m = t0 + r;
                if (m >= pc.lo && m < pc.hi) {
                    const float4 d0 = *reinterpret_cast<const float4 *>(&sm.ys[r * kYs + c8 * 8]);
                    const float4 d1 = *reinterpret_cast<const float4 *>(&sm.ys[r * kYs + c8 * 8 + 4]);
                    const float d[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                    float y[8];
                    widen<bf16_t>(yv[h][q], y);
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = y[e] + scale * d[e];
                    yv[h][q] = narrow<bf16_t>(y);
                    touched |= 1u << q;
                }
            }
            __syncthreads();  // LDS free for the next half or piece
        }
        if constexpr (kAhead) {
#pragma unroll
            for (int h = 0; h < NT; ++h)
#pragma unroll
                for (int u = 0; u < kBPer; ++u) {
                    bq[h][u][0] = bn[h][u][0];
                    bq[h][u][1] = bn[h][u][1];
                }
        }
    }
#pragma unroll
    for (int h = 0; h < NT; ++h) {
#pragma unroll
        for (int q = 0; q < kYPer; ++q) {
            const int idx = tid + q * kBlockThreads;
            const int n = n0 + h * kExpandTileCols + (idx % kColVecs) * 8;
            const int row = RM::kIndexed ? yrow[q] : t0 + idx / kColVecs;  // contiguous: a touched row is in the tile
            if ((((touched & yok) >> q) & 1u) && n < d_out) st16(Y + (size_t)row * d_out + n, yv[h][q]);
        }
    }
}

}  // namespace sgmv
