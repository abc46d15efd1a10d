/*
 * SGMV oracle: plain, slow CPU reference of the segmented LoRA delta.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the HIP
 * library: it has its own bf16 widening and rounding, its own indexing and its
 * own loops.
 *
 * What it computes (Punica guide, aifetchly blog, section "The Heterogeneous
 * Batching Bottleneck", equation for y_i, and section "The SGMV Mathematical
 * Formulation", equation for Y[s_i:s_{i+1}, :]):
 *
 *   for every segment s and every row m with seg_start[s] <= m < seg_start[s+1],
 *   with k = seg_adapter[s]:
 *       V[m, j] = sum_{i < d_in} X[m, i] * A_k(i, j)                (shrink)
 *       Y[m, n] = Y_in[m, n] + (alpha / r) * sum_{j < r} V[m, j] * B_k(j, n)
 *                                                                     (expand)
 *
 * Storage of one pool slot (the pages' adapter pointer array points at one
 * contiguous block per adapter): A_k is held as r rows of d_in elements, so
 * A_k(i, j) sits at element j * d_in + i; B_k is held as r rows of d_out
 * elements, so B_k(j, n) sits at element j * d_out + n. Slots are packed
 * back to back in a pool array: slot k starts at element k * r * d_in (A) or
 * k * r * d_out (B).
 *
 * Arithmetic: every input is widened exactly to double and every sum runs in
 * double, in ascending index order, one product at a time. Rows are
 * independent, so the optional OpenMP loop over segments gives bit-identical
 * results for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* bf16 is the upper half of an IEEE binary32 word: widening is exact. */
static double widen(const void *base, int32_t dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Clamp a segment bound into [0, M]. */
static int64_t clamp_row(int64_t v, int64_t M)
{
    return v < 0 ? 0 : (v > M ? M : v);
}

/*
 * Shrink: V[m, j] for every row m of every segment (double, row-major
 * M x r). Rows that lie in no segment are left untouched.
 * Returns 0, or -1 when an adapter id lies outside [0, num_adapters).
 */
int oracle_shrink(double *V, const void *X, const void *A_pool,
                  const int32_t *seg_start, const int32_t *seg_adapter,
                  int32_t num_segments, int32_t num_adapters, int32_t M,
                  int32_t d_in, int32_t r, int32_t dtype)
{
    for (int32_t s = 0; s < num_segments; ++s)
        if (seg_adapter[s] < 0 || seg_adapter[s] >= num_adapters)
            return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t s = 0; s < num_segments; ++s) {
        int64_t k = seg_adapter[s];
        int64_t lo = clamp_row(seg_start[s], M);
        int64_t hi = clamp_row(seg_start[s + 1], M);
        int64_t a_base = k * (int64_t)r * d_in;
        for (int64_t m = lo; m < hi; ++m) {
            for (int64_t j = 0; j < r; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d_in; ++i) {
                    double x = widen(X, dtype, m * d_in + i);
                    double a = widen(A_pool, dtype, a_base + j * d_in + i);
                    acc += x * a;
                }
                V[m * r + j] = acc;
            }
        }
    }
    return 0;
}

/*
 * Expand: Y[m, n] += (alpha / r) * sum_j V[m, j] * B_k(j, n), Y in double,
 * row-major M x d_out, updated in place (it holds Y_in on entry).
 */
int oracle_expand(double *Y, const double *V, const void *B_pool,
                  const int32_t *seg_start, const int32_t *seg_adapter,
                  int32_t num_segments, int32_t num_adapters, int32_t M,
                  int32_t r, int32_t d_out, double alpha, int32_t dtype)
{
    for (int32_t s = 0; s < num_segments; ++s)
        if (seg_adapter[s] < 0 || seg_adapter[s] >= num_adapters)
            return -1;
    double scale = alpha / (double)r;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t s = 0; s < num_segments; ++s) {
        int64_t k = seg_adapter[s];
        int64_t lo = clamp_row(seg_start[s], M);
        int64_t hi = clamp_row(seg_start[s + 1], M);
        int64_t b_base = k * (int64_t)r * d_out;
        for (int64_t m = lo; m < hi; ++m) {
            for (int64_t n = 0; n < d_out; ++n) {
                double acc = 0.0;
                for (int64_t j = 0; j < r; ++j)
                    acc += V[m * r + j] * widen(B_pool, dtype, b_base + j * d_out + n);
                Y[m * d_out + n] += scale * acc;
            }
        }
    }
    return 0;
}

/* Widen n stored elements (fp32 or bf16 bits) to double. */
void oracle_widen(double *out, const void *in, int64_t n, int32_t dtype)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = widen(in, dtype, i);
}

/*
 * Round doubles to bf16 bit patterns, to nearest with ties to even, directly
 * from the double value (one rounding). bf16 keeps 8 significant bits and the
 * binary32 exponent range: normal numbers from 2^-126, subnormals on the
 * fixed grid 2^-133, largest finite (2 - 2^-7) * 2^127.
 */
void oracle_round_bf16(uint16_t *out, const double *in, int64_t n)
{
    const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    for (int64_t i = 0; i < n; ++i) {
        double x = in[i];
        double q;
        if (isnan(x)) {
            out[i] = 0x7FC0;
            continue;
        }
        if (isinf(x)) {
            q = x;
        } else if (fabs(x) < ldexp(1.0, -126)) {
            q = ldexp(nearbyint(ldexp(x, 133)), -133);
        } else {
            int e;
            double f = frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1 */
            q = ldexp(nearbyint(ldexp(f, 8)), e - 8);
            if (fabs(q) > max_finite)
                q = copysign(INFINITY, x);
        }
        float qf = (float)q; /* exact: q is a bf16 value */
        uint32_t bits;
        memcpy(&bits, &qf, sizeof bits);
        out[i] = (uint16_t)(bits >> 16);
    }
}

/* Round doubles to binary32 (C's conversion rounds to nearest, ties to even). */
void oracle_round_f32(float *out, const double *in, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)in[i];
}
