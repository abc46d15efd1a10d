// Shared device helpers for the SGMV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgmv {

constexpr int kWave = 64;
constexpr int kBlockThreads = 256;  // threads per workgroup in every kernel (4 waves)

// Storage element types. bf16 is kept as raw 16-bit patterns and widened by a
// shift; fp32 is used as is. bf16_short_t is bf16 storage for batches whose
// segments are all too short for the matrix-core path: kernels built for it
// leave that path out (its code, LDS and registers), and any segment runs on
// the vector path, which is correct for every length.
struct bf16_t {
    uint16_t bits;
};
struct bf16_short_t {
    uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;  // elements per 16-byte vector
    static constexpr bool kMfma = false;  // long segments take the MFMA path
};
template <>
struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;
    static constexpr bool kMfma = true;
};
template <>
struct Elem<bf16_short_t> {
    static constexpr int kPerVec = 8;
    static constexpr bool kMfma = false;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Global-memory (address space 1) views. Adapter pointers come out of a table
// in memory and are generic; casting them here makes the compiler emit global
// rather than flat loads.
typedef __attribute__((address_space(1))) const u32x4_t gconst_vec_t;
typedef __attribute__((address_space(1))) u32x4_t gvec_t;

__device__ __forceinline__ uint4 to_uint4(u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }

// 16-byte loads and stores through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void *p) { return to_uint4(*(gconst_vec_t *)p); }
__device__ __forceinline__ void st16(void *p, uint4 v) {
    *(gvec_t *)p = u32x4_t{v.x, v.y, v.z, v.w};
}

// Streaming load: weights are read once per call, so keep them out of the way
// of data that is reused.
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
    return to_uint4(__builtin_nontemporal_load((gconst_vec_t *)p));
}

// Widen one 16-byte vector to fp32 values.
template <typename T>
__device__ __forceinline__ void widen(uint4 v, float (&out)[Elem<T>::kPerVec]);

template <>
__device__ __forceinline__ void widen<float>(uint4 v, float (&out)[4]) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
}

template <>
__device__ __forceinline__ void widen<bf16_t>(uint4 v, float (&out)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <>
__device__ __forceinline__ void widen<bf16_short_t>(uint4 v, float (&out)[8]) {
    widen<bf16_t>(v, out);
}

// Narrow fp32 values to one 16-byte vector, rounding to nearest-even.
template <typename T>
__device__ __forceinline__ uint4 narrow(const float (&in)[Elem<T>::kPerVec]);

template <>
__device__ __forceinline__ uint4 narrow<float>(const float (&in)[4]) {
    return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                      __float_as_uint(in[3]));
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32: round to nearest-even
    return __builtin_bit_cast(uint32_t, p);
}

template <>
__device__ __forceinline__ uint4 narrow<bf16_t>(const float (&in)[8]) {
    return make_uint4(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                      pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7]));
}

template <>
__device__ __forceinline__ uint4 narrow<bf16_short_t>(const float (&in)[8]) {
    return narrow<bf16_t>(in);
}

// Adapter address lookup for one wave. The address of a segment's adapter
// sits behind two dependent loads (its id, then the pointer table), each a
// full memory round trip before the weights can be requested. When the pool
// holds at most kSpecTable adapters, every lane loads four table entries
// right away, at the same time as the segment metadata, and the uniform id
// then picks its entry out of registers (kSpec = true); larger pools load the
// entry once the id is known (kSpec = false). Callers choose between the two
// with a uniform branch around the whole work item, so that neither copy has
// a load whose register is merged with the other's: the compiler would wait
// for every load in flight where the two sides meet.
constexpr int kSpecTable = 4 * kWave;

template <bool kSpec>
struct AdapterTable;

template <>
struct AdapterTable<true> {
    uint64_t e[4];

    // num_adapters >= 1: every index is clamped into the table.
    __device__ __forceinline__ void load(const uint64_t *ptrs, int num_adapters, int lane) {
        // Keep the loads here. Left alone, the compiler sinks them below the
        // caller's checks on the metadata, i.e. until after it has arrived:
        // the table is read-only, so its loads may move past anything.
        // Hiding where the pointer came from makes them ordinary loads, which
        // the empty barrier then holds in place.
        asm volatile("" : "+s"(ptrs));
        typedef __attribute__((address_space(1))) const uint64_t gconst_u64_t;
        gconst_u64_t *g = (gconst_u64_t *)ptrs;
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = g[min(lane + q * kWave, num_adapters - 1)];
        asm volatile("" ::: "memory");
    }

    // Address of adapter k (0 <= k < num_adapters <= kSpecTable; k uniform).
    __device__ __forceinline__ uint64_t address(const uint64_t *, int k) const {
        const int q = k / kWave;
        const uint64_t v = q == 0 ? e[0] : (q == 1 ? e[1] : (q == 2 ? e[2] : e[3]));
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, k % kWave);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), k % kWave);
        return ((uint64_t)hi << 32) | lo;
    }
};

template <>
struct AdapterTable<false> {
    __device__ __forceinline__ void load(const uint64_t *, int, int) {}
    __device__ __forceinline__ uint64_t address(const uint64_t *ptrs, int k) const { return ptrs[k]; }
};

// Token row of segment-ordered row p. The contiguous calls take the batch in
// segment order (p itself); the gathered calls take it in token order
// through an index, rows[p]. An index outside [0, M) is read as row 0 and
// reported with ok = false: its Y row is never stored.
template <bool kGather>
struct RowMap {
    static constexpr bool kIndexed = kGather;
    const int32_t *rows;
    int M;
    __device__ __forceinline__ int operator()(int p, bool &ok) const {
        if constexpr (kGather) {
            const int q = rows[p];
            ok = (unsigned)q < (unsigned)M;
            return ok ? q : 0;
        } else {
            ok = true;
            return p;
        }
    }
    __device__ __forceinline__ int operator()(int p) const {
        bool ok;
        return (*this)(p, ok);
    }
};

// Segment bounds clamped into [0, M]; an inverted pair is an empty segment.
// Returns whether the offsets as given decrease here (seg_start[s] >
// seg_start[s + 1]): offsets that are not non-decreasing always do so at
// some segment, and only then can two segments share rows.
__device__ __forceinline__ bool segment_rows(const int32_t *seg_start, int s, int M, int &lo,
                                             int &hi) {
    const int a0 = seg_start[s];
    const int b0 = seg_start[s + 1];
    const int a = a0 < 0 ? 0 : (a0 > M ? M : a0);
    const int b = b0 < 0 ? 0 : (b0 > M ? M : b0);
    lo = a;
    hi = b < a ? a : b;
    return a0 > b0;
}

// Sum of NV values per lane across the 64 lanes of a wave, by recursive
// halving: at each step a lane keeps half of its values and adds the
// partner's copy of that half, so the shuffles shrink from NV to NV/2 to
// ... 1, then plain butterflies finish the lane bits that remain. On return
// vals[0] holds the wave-wide total of value index (lane >> (6 - log2 NV)).
// Written as template recursion so every array index is a constant.
template <int COUNT, int OFFSET>
struct WaveHalving {
    static __device__ __forceinline__ void run(float *vals, int lane) {
        constexpr int half = COUNT / 2;
        const bool upper = (lane & OFFSET) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? vals[i] : vals[i + half];
            const float keep = upper ? vals[i + half] : vals[i];
            vals[i] = keep + __shfl_xor(send, OFFSET, kWave);
        }
        WaveHalving<half, OFFSET / 2>::run(vals, lane);
    }
};

template <int OFFSET>
struct WaveHalving<1, OFFSET> {
    static __device__ __forceinline__ void run(float *vals, int) {
#pragma unroll
        for (int o = OFFSET; o >= 1; o >>= 1) vals[0] += __shfl_xor(vals[0], o, kWave);
    }
};

template <int NV>
__device__ __forceinline__ void wave_reduce_transpose(float (&vals)[NV], int lane) {
    static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
    WaveHalving<NV, 32>::run(vals, lane);
}

template <int NV>
__host__ __device__ constexpr int log2_pow2() {
    return NV <= 1 ? 0 : 1 + log2_pow2<NV / 2>();
}

}  // namespace sgmv
