// Host-side sanitizer driver: exercises the oracle (oracle/sgmv_oracle.c)
// and the library's host-only entry points (sgmv_host.cpp) built with
// AddressSanitizer and UndefinedBehaviorSanitizer, on every buffer sized
// exactly (so any read or write past an end is reported), with valid and
// invalid metadata and extreme sizes. Results are also checked: the oracle
// against a brute-force loop on the valid cases, the helpers against their
// documented contracts. Exit status 0 when every check passes.
//
// Test infrastructure only: built and run by tests/test_host_sanitizers.py.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "sgmv.h"

extern "C" {
int oracle_shrink(double *V, const void *X, const void *A_pool, const int32_t *seg_start,
                  const int32_t *seg_adapter, int32_t num_segments, int32_t num_adapters, int32_t M,
                  int32_t d_in, int32_t r, int32_t dtype);
int oracle_expand(double *Y, const double *V, const void *B_pool, const int32_t *seg_start,
                  const int32_t *seg_adapter, int32_t num_segments, int32_t num_adapters, int32_t M,
                  int32_t r, int32_t d_out, double alpha, int32_t dtype);
void oracle_widen(double *out, const void *in, int64_t n, int32_t dtype);
void oracle_round_bf16(uint16_t *out, const double *in, int64_t n);
void oracle_round_f32(float *out, const double *in, int64_t n);
}

static int failures = 0;
#define CHECK(cond, ...)                                    \
    do {                                                    \
        if (!(cond)) {                                      \
            ++failures;                                     \
            fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                   \
            fprintf(stderr, "\n");                          \
        }                                                   \
    } while (0)

// splitmix64
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    int uniform(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }  // [lo, hi]
};

// Exactly sized heap buffers: ASan sees one byte past the end.
template <typename T>
static T *alloc(size_t n) {
    return static_cast<T *>(malloc(std::max<size_t>(n, 1) * sizeof(T)));
}

static double value_of(const void *base, int dtype, int64_t i) {
    if (dtype == 0) return ((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

static void fill(void *base, int dtype, int64_t n, Rng &g) {
    for (int64_t i = 0; i < n; ++i) {
        const float v = (float)((int)(g.next() % 9) - 4) * 0.25f;  // small exact values
        if (dtype == 0) {
            ((float *)base)[i] = v;
        } else {
            uint32_t bits;
            memcpy(&bits, &v, 4);
            ((uint16_t *)base)[i] = (uint16_t)(bits >> 16);
        }
    }
}

static void oracle_cases() {
    Rng g{1};
    for (int c = 0; c < 400; ++c) {
        const int dtype = g.uniform(0, 1);
        const int esz = dtype == 0 ? 4 : 2;
        const int M = g.uniform(0, 40), N = g.uniform(0, 8), P = g.uniform(1, 5);
        const int r = 8 << g.uniform(0, 3), d_in = 8 * g.uniform(1, 9), d_out = 8 * g.uniform(1, 9);
        const bool bad_ids = g.uniform(0, 9) == 0;
        int32_t *ss = alloc<int32_t>(N + 1), *sa = alloc<int32_t>(N);
        // offsets: mostly valid, sometimes outside [0, M] or decreasing (clamped)
        for (int s = 0; s <= N; ++s) ss[s] = g.uniform(-3, M + 3);
        const bool sorted = g.uniform(0, 1) == 1;  // unsorted offsets may overlap: then only run them
        if (sorted) std::sort(ss, ss + N + 1);
        for (int s = 0; s < N; ++s) sa[s] = bad_ids ? g.uniform(-2, P + 1) : g.uniform(0, P - 1);
        bool ids_ok = true;
        for (int s = 0; s < N; ++s) ids_ok = ids_ok && sa[s] >= 0 && sa[s] < P;
        void *X = malloc((size_t)std::max(1, M * d_in) * esz);
        void *A = malloc((size_t)P * r * d_in * esz);
        void *B = malloc((size_t)P * r * d_out * esz);
        fill(X, dtype, (int64_t)M * d_in, g);
        fill(A, dtype, (int64_t)P * r * d_in, g);
        fill(B, dtype, (int64_t)P * r * d_out, g);
        double *V = alloc<double>((size_t)M * r), *Y = alloc<double>((size_t)M * d_out);
        for (int64_t i = 0; i < (int64_t)M * r; ++i) V[i] = 0.0;
        for (int64_t i = 0; i < (int64_t)M * d_out; ++i) Y[i] = 0.5 * (double)(i % 7);
        const int rs = oracle_shrink(V, X, A, ss, sa, N, P, M, d_in, r, dtype);
        const int re = oracle_expand(Y, V, B, ss, sa, N, P, M, r, d_out, 2.0 * r, dtype);
        CHECK((rs == 0) == ids_ok && (re == 0) == ids_ok, "case %d: return codes %d %d, ids ok %d", c, rs, re,
              (int)ids_ok);
        if (ids_ok && sorted) {  // brute force: every row of every (clamped) segment
            std::vector<double> Vb((size_t)M * r, 0.0), Yb((size_t)M * d_out);
            for (int64_t i = 0; i < (int64_t)M * d_out; ++i) Yb[i] = 0.5 * (double)(i % 7);
            for (int s = 0; s < N; ++s) {
                const int lo = std::min(std::max(ss[s], 0), M), hi = std::min(std::max(ss[s + 1], 0), M);
                for (int m = lo; m < hi; ++m) {
                    for (int j = 0; j < r; ++j) {
                        double acc = 0;
                        for (int i = 0; i < d_in; ++i)
                            acc += value_of(X, dtype, (int64_t)m * d_in + i) *
                                   value_of(A, dtype, ((int64_t)sa[s] * r + j) * d_in + i);
                        Vb[(size_t)m * r + j] = acc;
                    }
                    for (int n = 0; n < d_out; ++n) {
                        double acc = 0;
                        for (int j = 0; j < r; ++j)
                            acc += Vb[(size_t)m * r + j] * value_of(B, dtype, ((int64_t)sa[s] * r + j) * d_out + n);
                        Yb[(size_t)m * d_out + n] += 2.0 * acc;
                    }
                }
            }
            for (int64_t i = 0; i < (int64_t)M * r; ++i) CHECK(V[i] == Vb[i], "case %d: V[%ld]", c, (long)i);
            for (int64_t i = 0; i < (int64_t)M * d_out; ++i) CHECK(Y[i] == Yb[i], "case %d: Y[%ld]", c, (long)i);
        }
        free(X), free(A), free(B), free(V), free(Y), free(ss), free(sa);
    }
}

static void rounding_cases() {
    const double inf = std::numeric_limits<double>::infinity();
    std::vector<double> specials = {0.0, -0.0, 1.0, -1.0, inf, -inf, NAN, ldexp(1.0, -149), ldexp(1.0, -150),
                                    ldexp(1.0, -133), ldexp(1.0, -134), ldexp(1.0, 127) * 1.9999999,
                                    ldexp(2.0, 127), 1e300, -1e300, 1e-300, ldexp(1.0, -126),
                                    1.0 + ldexp(1.0, -24), 1.0 + ldexp(1.0, -8)};
    Rng g{2};
    for (int i = 0; i < 20000; ++i) {
        uint64_t b = g.next();
        double d;
        memcpy(&d, &b, 8);
        specials.push_back(d);
    }
    const int64_t n = (int64_t)specials.size();
    double *in = alloc<double>(n);
    std::copy(specials.begin(), specials.end(), in);
    uint16_t *hb = alloc<uint16_t>(n);
    float *hf = alloc<float>(n);
    oracle_round_bf16(hb, in, n);
    oracle_round_f32(hf, in, n);
    for (int64_t i = 0; i < n; ++i) {
        if (isnan(in[i])) {
            CHECK(isnan(hf[i]) && (hb[i] & 0x7F80) == 0x7F80 && (hb[i] & 0x7F), "NaN stays NaN");
            continue;
        }
        // both roundings are monotone and keep the sign
        CHECK(!(in[i] > 0) || (hf[i] >= 0 && !(hb[i] & 0x8000)), "sign of %g", in[i]);
    }
    // widening: every bf16 pattern and random fp32 patterns
    uint16_t *all = alloc<uint16_t>(65536);
    for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
    double *w = alloc<double>(65536);
    oracle_widen(w, all, 65536, 1);
    uint16_t *back = alloc<uint16_t>(65536);
    oracle_round_bf16(back, w, 65536);
    for (int i = 0; i < 65536; ++i) {
        const bool nan = (i & 0x7F80) == 0x7F80 && (i & 0x7F);
        CHECK(nan ? isnan(w[i]) : back[i] == all[i], "bf16 pattern %04x does not round-trip", i);
    }
    float *f = alloc<float>(4096);
    for (int i = 0; i < 4096; ++i) {
        uint32_t b = (uint32_t)g.next();
        memcpy(&f[i], &b, 4);
    }
    double *wf = alloc<double>(4096);
    oracle_widen(wf, f, 4096, 0);
    float *fb = alloc<float>(4096);
    oracle_round_f32(fb, wf, 4096);
    for (int i = 0; i < 4096; ++i) CHECK(isnan(f[i]) ? isnan(fb[i]) : fb[i] == f[i], "fp32 round trip %d", i);
    free(in), free(hb), free(hf), free(all), free(w), free(back), free(f), free(wf), free(fb);
}

static void build_segments_cases() {
    Rng g{3};
    for (int c = 0; c < 500; ++c) {
        const int M = g.uniform(0, 300), P = g.uniform(1, 50);
        int32_t *ids = alloc<int32_t>(M), *perm = alloc<int32_t>(M), *ss = alloc<int32_t>(M + 1),
                *sa = alloc<int32_t>(M);
        for (int i = 0; i < M; ++i) ids[i] = g.uniform(0, P - 1);
        int32_t n = -1;
        CHECK(sgmv_build_segments(ids, M, perm, ss, sa, &n) == SGMV_OK, "build_segments case %d", c);
        CHECK(n >= (M > 0) && n <= M, "segment count %d for M %d", n, M);
        std::vector<int> seen(M, 0);
        for (int p = 0; p < M; ++p) {
            CHECK(perm[p] >= 0 && perm[p] < M, "perm entry");
            if (perm[p] >= 0 && perm[p] < M) seen[perm[p]]++;
            if (p > 0) CHECK(ids[perm[p - 1]] < ids[perm[p]] || (ids[perm[p - 1]] == ids[perm[p]] && perm[p - 1] < perm[p]),
                             "stable sort by adapter");
        }
        for (int i = 0; i < M; ++i) CHECK(seen[i] == 1, "perm is a permutation");
        CHECK(ss[0] == 0 && ss[n] == M, "offsets span the batch");
        for (int s = 0; s < n; ++s) {
            CHECK(ss[s] < ss[s + 1], "segments are non-empty");
            if (s > 0) CHECK(sa[s - 1] < sa[s], "one segment per adapter, ascending");
            for (int p = ss[s]; p < ss[s + 1]; ++p) CHECK(ids[perm[p]] == sa[s], "row in its adapter's segment");
        }
        CHECK(sgmv_check_segments(ss, sa, n, M, P) == SGMV_OK, "built segments pass the check");
        if (M > 0) {
            ids[g.uniform(0, M - 1)] = -1 - g.uniform(0, 5);
            CHECK(sgmv_build_segments(ids, M, perm, ss, sa, &n) == SGMV_ERR_ADAPTER, "negative id refused");
        }
        free(ids), free(perm), free(ss), free(sa);
    }
    int32_t n, one = 0, perm, ss[2], sa;
    CHECK(sgmv_build_segments(nullptr, 1, &perm, ss, &sa, &n) == SGMV_ERR_NULL, "null ids");
    CHECK(sgmv_build_segments(&one, 1, &perm, ss, &sa, nullptr) == SGMV_ERR_NULL, "null count");
    CHECK(sgmv_build_segments(&one, -1, &perm, ss, &sa, &n) == SGMV_ERR_SHAPE, "negative M");
    CHECK(sgmv_build_segments(nullptr, 0, nullptr, ss, nullptr, &n) == SGMV_OK && n == 0 && ss[0] == 0,
          "empty batch");
}

static void check_segments_cases() {
    Rng g{4};
    for (int c = 0; c < 500; ++c) {
        const int N = g.uniform(0, 20), P = g.uniform(1, 10);
        int32_t *ss = alloc<int32_t>(N + 1), *sa = alloc<int32_t>(N);
        ss[0] = 0;
        for (int s = 0; s < N; ++s) {
            ss[s + 1] = ss[s] + g.uniform(0, 5);
            sa[s] = g.uniform(0, P - 1);
        }
        const int M = ss[N];
        CHECK(sgmv_check_segments(ss, sa, N, M, P) == SGMV_OK, "valid metadata accepted");
        CHECK(sgmv_check_segments(ss, sa, N, M + 1, P) == SGMV_ERR_SHAPE, "last offset must be M");
        if (N > 0) {
            const int s = g.uniform(0, N - 1);
            const int32_t keep = sa[s];
            sa[s] = g.uniform(0, 1) ? -1 : P;
            CHECK(sgmv_check_segments(ss, sa, N, M, P) == SGMV_ERR_ADAPTER, "bad id refused");
            sa[s] = keep;
        }
        if (N > 1 && ss[1] > 0) {
            const int32_t keep = ss[1];
            ss[1] = ss[2] + 1;
            if (ss[1] <= M && ss[2] < ss[1]) CHECK(sgmv_check_segments(ss, sa, N, M, P) != SGMV_OK, "decreasing");
            ss[1] = keep;
        }
        free(ss), free(sa);
    }
    CHECK(sgmv_check_segments(nullptr, nullptr, 0, 0, 1) == SGMV_ERR_NULL, "null offsets");
    CHECK(sgmv_check_segments(nullptr, nullptr, -1, 0, 1) == SGMV_ERR_SHAPE, "negative count");
}

static void pool_pointer_cases() {
    Rng g{5};
    alignas(16) static char base[64];
    for (int c = 0; c < 200; ++c) {
        const int P = g.uniform(0, 3000);
        const int64_t slot = 16 * (int64_t)g.uniform(0, 1 << 20);
        uint64_t *t = alloc<uint64_t>(P);
        CHECK(sgmv_pool_pointers(t, base, P, slot) == SGMV_OK, "pool pointers");
        for (int k = 0; k < P; ++k) CHECK(t[k] == (uint64_t)(uintptr_t)base + (uint64_t)k * slot, "slot address");
        free(t);
    }
    uint64_t t[4];
    CHECK(sgmv_pool_pointers(t, base + 8, 4, 64) == SGMV_ERR_ALIGN, "misaligned base");
    CHECK(sgmv_pool_pointers(t, base, 4, 24) == SGMV_ERR_ALIGN, "misaligned slot");
    CHECK(sgmv_pool_pointers(nullptr, base, 4, 64) == SGMV_ERR_NULL, "null table");
    CHECK(sgmv_pool_pointers(t, base, -1, 64) == SGMV_ERR_SHAPE, "negative count");
    CHECK(sgmv_pool_pointers(t, base, 4, (int64_t)1 << 40) == SGMV_OK, "large slots");
}

static void size_cases() {
    const int32_t Ms[] = {0, 1, 15, 16, 17, 63, 64, 65, 2047, 2048, 2049, 1 << 16, 1 << 20, (1 << 24) + 1,
                          std::numeric_limits<int32_t>::max() - 1, std::numeric_limits<int32_t>::max(), -1};
    const int32_t Ns[] = {0, 1, 7, 64, 512, 1 << 20, std::numeric_limits<int32_t>::max(), -5};
    const int32_t Ds[] = {8, 24, 4096, 28672, 1 << 20, std::numeric_limits<int32_t>::max() - 7, 0, 12, -8};
    const int32_t Rs[] = {8, 16, 32, 64, 12};
    for (int32_t M : Ms)
        for (int32_t N : Ns)
            for (int32_t di : Ds)
                for (int32_t dout : Ds)
                    for (int32_t r : Rs)
                        for (int32_t dt = -1; dt <= 2; ++dt) {
                            const size_t b = sgmv_workspace_bytes(N, M, di, dout, r, dt);
                            const bool valid = M >= 0 && N >= 0 && di > 0 && di % 8 == 0 && dout > 0 &&
                                               dout % 8 == 0 && (r == 8 || r == 16 || r == 32 || r == 64) &&
                                               (dt == 0 || dt == 1);
                            CHECK(valid || b == 0, "invalid sizes ask for no workspace");
                            CHECK(b % 256 == 0, "workspace sizes are whole lines");
                            sgmv_projection p[SGMV_MAX_PROJECTIONS + 1];
                            for (int q = 0; q <= SGMV_MAX_PROJECTIONS; ++q)
                                p[q] = sgmv_projection{nullptr, nullptr, nullptr, nullptr, 4, di, dout};
                            const size_t l1 = sgmv_layer_workspace_bytes(p, 1, N, M, r, dt);
                            CHECK(l1 <= b, "one projection's layer workspace fits its single calls' workspace");
                            (void)sgmv_layer_workspace_bytes(p, SGMV_MAX_PROJECTIONS, N, M, r, dt);
                            CHECK(sgmv_layer_workspace_bytes(p, SGMV_MAX_PROJECTIONS + 1, N, M, r, dt) == 0,
                                  "too many projections");
                        }
    for (int s = -20; s <= 5; ++s) CHECK(sgmv_status_string(s) != nullptr, "status string");
    CHECK(sgmv_version() > 0, "version");
}

int main() {
    oracle_cases();
    rounding_cases();
    build_segments_cases();
    check_segments_cases();
    pool_pointer_cases();
    size_cases();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host sanitizer driver: all checks passed\n");
    return 0;
}
