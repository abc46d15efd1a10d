/*
 * sgmv.h — C ABI of the MI355X (gfx950) SGMV library.
 *
 * SGMV (segmented gather matrix-vector multiplication) applies many LoRA
 * adapters to one batch in one pass. The batch's rows are grouped into
 * contiguous segments; segment s covers rows seg_start[s] .. seg_start[s+1]-1
 * and uses adapter k = seg_adapter[s] from a pool reached through a table of
 * pointers. For every row m of segment s:
 *
 *     V[m, :] = X[m, :] . A_k                         (shrink, d_in -> r)
 *     Y[m, :] = Y[m, :] + (alpha / r) * V[m, :] . B_k  (expand, r -> d_out)
 *
 * Sources (Punica guide, aifetchly blog): the per-row LoRA equation for y_i
 * in section "The Heterogeneous Batching Bottleneck" (delta added to the base
 * output, scaled by alpha / r, A_k of logical shape d_in x r, B_k of logical
 * shape r x d_out); the segment offsets S = {s_0 .. s_N} and the pointer
 * array of section "The SGMV Mathematical Formulation"; the single kernel
 * that takes X and the pointers to A and B (figure "Punica: SGMV"); the two
 * launches per layer, one for all A and one for all B (section "Mathematical
 * Modeling", equation 2).
 *
 * Conventions shared by every call
 * --------------------------------
 * dtype        SGMV_F32 or SGMV_BF16. X, Y and every adapter share it. V is
 *              always fp32. Arithmetic accumulates in fp32; Y is rounded once,
 *              to nearest-even, when stored.
 * precision    bf16 segments of 16 rows or more expand on matrix cores, where
 *              each fp32 V value enters as the sum of two bf16 values,
 *              hi = rne(v) and lo = rne(v - hi): 16 significant bits, a
 *              relative error of at most 2^-16 per value (exact for integer
 *              V with |V| < 2^16). The expand error of such a row is then at
 *              most (alpha / r) * 2^-16 * sum_j |V[m, j]| |B_k(j, n)| beyond
 *              fp32 accumulation and the final rounding. Every other product
 *              takes its operands exactly.
 * X            device, row-major M x d_in, contiguous, 16-byte aligned.
 * Y            device, row-major M x d_out, contiguous, 16-byte aligned;
 *              read and written (the delta is added to what Y holds).
 * V            device, row-major M x r fp32, contiguous, 16-byte aligned.
 * A_ptrs       device array of num_adapters 64-bit device addresses. Entry k
 *              points to A_k stored as r rows of d_in elements: logical
 *              element (i, j) of A_k sits at j * d_in + i. 16-byte aligned.
 * B_ptrs       device array of num_adapters addresses. Entry k points to B_k
 *              stored as r rows of d_out elements: (j, n) at j * d_out + n.
 * seg_start    device int32[num_segments + 1], non-decreasing, with
 *              seg_start[0] = 0 and seg_start[num_segments] = M.
 * seg_adapter  device int32[num_segments], each in [0, num_adapters).
 * r            8, 16, 32 or 64.
 * d_in, d_out  positive multiples of 8.
 * stream       a hipStream_t (NULL = the default stream). Every call is
 *              asynchronous and stream-ordered: it only enqueues kernels, makes
 *              no host<->device copy and no synchronisation.
 *
 * Ownership: the caller owns every buffer and must keep it alive until the
 * stream work completes. The library allocates no memory and keeps no pointer
 * after a call returns.
 *
 * Errors: every call returns SGMV_OK (0) or a negative status; no call
 * aborts. Arguments are checked on the host before anything is enqueued; on
 * error nothing is enqueued. M == 0 or num_segments == 0 is a successful
 * no-op. Device-resident metadata cannot be checked without a
 * synchronisation, so the kernels defend themselves instead: segment bounds
 * are clamped into [0, M] (a decreasing pair is an empty segment) and a
 * segment whose adapter id lies outside [0, num_adapters) is skipped (its rows
 * are left as they were). Nothing outside the documented buffers is read or
 * written for any metadata values, and every kernel ends.
 *
 * Failures seen on the device (calls with a workspace): offsets that
 * decrease somewhere let two segments share rows; the values of such rows
 * are then unspecified, and the call sets SGMV_WS_BAD_OFFSETS in the
 * workspace's status word. Workgroups that wait for one another do so for a
 * bounded number of polls (sgmv_set_wait_limit); a wait that gives up leaves
 * its rows unchanged and sets SGMV_WS_WAIT_TIMEOUT. Either bit means the
 * workspace may hold leftovers: every later call on it does nothing (its
 * outputs are left as they were) until the caller zero-fills the workspace
 * again. sgmv_workspace_status reads the word.
 */
#ifndef SGMV_H
#define SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sgmv_dtype { SGMV_F32 = 0, SGMV_BF16 = 1 };

enum sgmv_status {
    SGMV_OK = 0,
    SGMV_ERR_NULL = -1,      /* a required pointer is NULL */
    SGMV_ERR_SHAPE = -2,     /* negative size, d not a multiple of 8, or too large */
    SGMV_ERR_RANK = -3,      /* r not in {8, 16, 32, 64} */
    SGMV_ERR_DTYPE = -4,     /* dtype not SGMV_F32 / SGMV_BF16 */
    SGMV_ERR_ALIGN = -5,     /* X, Y or V not 16-byte aligned */
    SGMV_ERR_WORKSPACE = -6, /* workspace missing or smaller than sgmv_workspace_bytes */
    SGMV_ERR_HIP = -7,       /* the HIP runtime reported an error at launch */
    SGMV_ERR_ADAPTER = -8,   /* host metadata: an adapter id that is negative (or outside the pool) */
    SGMV_ERR_SCRATCH = -9    /* sgmv_fused_noalloc: the batch needs more than SGMV_NOALLOC_SCRATCH_BYTES */
};

/*
 * Shrink (Punica guide, "The SGMV Mathematical Formulation": one launch for
 * every segment; "Mathematical Modeling" eq. 2: the launch for all A).
 * V[m, j] = sum_i X[m, i] * A_k(i, j) for every row m of every segment.
 * V is overwritten for rows that lie in a segment with a valid adapter, and
 * left untouched elsewhere.
 *
 * workspace: as for sgmv_fused (same size query, same zero-filled contract).
 * Long bf16 segments split the reduction over d_in between workgroups and
 * combine the parts there, in a fixed order. May be NULL with
 * workspace_bytes = 0 when sgmv_workspace_bytes(...) is 0.
 */
int sgmv_shrink(float *V, const void *X, const uint64_t *A_ptrs, int32_t num_adapters,
                const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                int32_t M, int32_t d_in, int32_t r, int32_t dtype, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * Expand (same sources; the launch for all B, and the equation for y_i: the
 * delta, scaled by alpha / r, is added to the base output).
 * Y[m, n] += (alpha / r) * sum_j V[m, j] * B_k(j, n). The scale alpha / r is
 * formed once in fp32.
 */
int sgmv_expand(void *Y, const float *V, const uint64_t *B_ptrs, int32_t num_adapters,
                const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                int32_t M, int32_t d_out, int32_t r, float alpha, int32_t dtype, void *stream);

/*
 * Fused shrink + expand in one launch (Punica guide, figure "Punica: SGMV":
 * one kernel call over X and the pointers to A and B).
 * Y[m, :] += (alpha / r) * X[m, :] . A_k . B_k. The intermediate V lives in
 * the workspace and is not returned. Same result as sgmv_shrink followed by
 * sgmv_expand, up to fp32 summation order.
 *
 * workspace: device memory of at least sgmv_workspace_bytes(...) bytes,
 * 256-byte aligned, zero-filled before its first use (for example by
 * hipMemset once after allocating it). Every call leaves the bytes it uses
 * all zero again when its kernel completes, so one workspace serves any later
 * call on the same stream, of any size that fits, without clearing. Calls
 * that overlap in time (different streams) must use different workspaces.
 */
int sgmv_fused(void *Y, const void *X, const uint64_t *A_ptrs, const uint64_t *B_ptrs,
               int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
               int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out, int32_t r,
               float alpha, int32_t dtype, void *workspace, size_t workspace_bytes,
               void *stream);

/*
 * sgmv_fused without a workspace argument and without any allocation: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments (minus the workspace), result and errors as sgmv_fused. The
 * workspace is a static array of SGMV_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU (each GPU the call runs on holds its copy until the
 * process ends); a batch whose fused workspace (sgmv_workspace_bytes) is
 * larger is rejected with SGMV_ERR_SCRATCH and nothing is enqueued. The
 * stream must belong to the current device. Each call first enqueues a
 * one-workgroup kernel that zero-fills the array if an earlier call left a
 * failure status in it (otherwise earlier calls left it zero), then the
 * fused kernel. All calls on one GPU share the array: calls that overlap in
 * time on that GPU (different streams, or different threads) race and must
 * not be made; calls on one stream are ordered and safe. No hipMalloc,
 * hipFree or allocating library routine is called.
 */
#define SGMV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int sgmv_fused_noalloc(void *Y, const void *X, const uint64_t *A_ptrs, const uint64_t *B_ptrs,
                       int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                       int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out, int32_t r,
                       float alpha, int32_t dtype, void *stream);

/*
 * Gathered forms: the batch stays in token order (Punica guide, figure "CUDA
 * Threadblock Tiling": the block of a segment gathers that segment's rows of
 * activations; section "Hardware-Level Optimizations in SGMV": grouping the
 * requests by adapter, which these calls do through an index instead of
 * moving X and Y).
 *
 * rows         device int32[M]: segment row p (p in [0, M), in segment order
 *              exactly as seg_start describes it for the calls above) is
 *              token row rows[p] of X and of Y. Normally the perm that
 *              sgmv_build_segments returns, i.e. a permutation of [0, M).
 * X, Y         token order, M rows each (same layout as above).
 * V            segment order: V row p belongs to token rows[p], as in the
 *              calls above.
 *
 * Each call computes what its contiguous counterpart computes on the batch
 * gathered into segment order, with Y's rows put back at their tokens:
 *     V[p, :]       = X[rows[p], :] . A_k                       (shrink_gather)
 *     Y[rows[p], :] += (alpha / r) * V[p, :] . B_k             (expand_scatter)
 *     Y[rows[p], :] += (alpha / r) * X[rows[p], :] . A_k . B_k  (fused_gather)
 * Arguments, workspace, errors and the device-side defences are those of
 * the contiguous call, plus: rows must not be NULL when M > 0. An entry of
 * rows outside [0, M) makes segment row p absent: no Y row is written for
 * it and V row p is unspecified (X is then read at row 0, never outside X).
 * If two entries name the same token, that token's Y row is unspecified
 * (the writes race); nothing outside the buffers is touched.
 */
int sgmv_shrink_gather(float *V, const void *X, const int32_t *rows, const uint64_t *A_ptrs,
                       int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                       int32_t num_segments, int32_t M, int32_t d_in, int32_t r, int32_t dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

int sgmv_expand_scatter(void *Y, const float *V, const int32_t *rows, const uint64_t *B_ptrs,
                        int32_t num_adapters, const int32_t *seg_start, const int32_t *seg_adapter,
                        int32_t num_segments, int32_t M, int32_t d_out, int32_t r, float alpha,
                        int32_t dtype, void *stream);

int sgmv_fused_gather(void *Y, const void *X, const int32_t *rows, const uint64_t *A_ptrs,
                      const uint64_t *B_ptrs, int32_t num_adapters, const int32_t *seg_start,
                      const int32_t *seg_adapter, int32_t num_segments, int32_t M, int32_t d_in,
                      int32_t d_out, int32_t r, float alpha, int32_t dtype, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Layer-batched fused call: every projection of one batch in one launch
 * (Punica guide, "Mathematical Modeling", equation 2: the execution latency
 * of a layer counts its launches, one per adapter matrix; here one per layer,
 * whatever the number of projections).
 *
 * For every projection q < num_projections, with p = projections[q]:
 *     p.Y[m, :] += (alpha / r) * p.X[m, :] . A_k . B_k
 * where A_k and B_k come from p's own pools (p.A_ptrs, p.B_ptrs, each of
 * p.num_adapters entries) and k is the adapter of m's segment. All
 * projections share the batch: M rows, the segments (seg_start,
 * seg_adapter), r, alpha and dtype; each has its own d_in and d_out, and X
 * and Y of the layouts above (p.X: M x p.d_in, p.Y: M x p.d_out). The
 * result is that of one sgmv_fused call per projection.
 *
 * rows         NULL: X and Y in segment order. Otherwise the token-order
 *              index of the gathered calls above, shared by every projection.
 * projections  host array of num_projections descriptors, read during the
 *              call only (the library keeps no pointer to it).
 * num_projections  0 .. SGMV_MAX_PROJECTIONS (0 is a no-op).
 * workspace    at least sgmv_layer_workspace_bytes(...) bytes, 256-byte
 *              aligned, zero-filled before first use; every call leaves it
 *              zero again (as for sgmv_fused).
 * The Y buffers of different projections must not overlap. Errors and
 * device-side defences as for sgmv_fused, checked for every projection;
 * num_projections outside [0, SGMV_MAX_PROJECTIONS] is SGMV_ERR_SHAPE.
 */
#define SGMV_MAX_PROJECTIONS 8

typedef struct sgmv_projection {
    void *Y;
    const void *X;
    const uint64_t *A_ptrs;
    const uint64_t *B_ptrs;
    int32_t num_adapters;
    int32_t d_in;
    int32_t d_out;
} sgmv_projection;

int sgmv_fused_layer(const sgmv_projection *projections, int32_t num_projections, const int32_t *rows,
                     const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments, int32_t M,
                     int32_t r, float alpha, int32_t dtype, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Workspace bytes sgmv_fused_layer needs (0 on invalid arguments). */
size_t sgmv_layer_workspace_bytes(const sgmv_projection *projections, int32_t num_projections,
                                  int32_t num_segments, int32_t M, int32_t r, int32_t dtype);

/* Bytes of workspace sgmv_shrink and sgmv_fused need for these sizes; one
 * buffer of this size serves both (0 on invalid sizes, or when neither needs
 * any). The gathered forms need the same. */
size_t sgmv_workspace_bytes(int32_t num_segments, int32_t M, int32_t d_in, int32_t d_out,
                            int32_t r, int32_t dtype);

/*
 * Host-side segment metadata (Punica guide, "Hardware-Level Optimizations in
 * SGMV": requests are grouped by adapter so that each adapter's rows are
 * contiguous; "The SGMV Mathematical Formulation": the offsets s_0 .. s_N).
 *
 * token_adapter: host int32[M], the adapter of each token, each >= 0.
 * perm:          host int32[M], out: the stable sort of token indices by
 *                adapter id; row p of the segmented batch is token perm[p].
 * seg_start:     host int32[M + 1], out: the first *num_segments + 1 entries
 *                are the segment offsets (seg_start[0] = 0, last = M).
 * seg_adapter:   host int32[M], out: the first *num_segments entries are the
 *                segments' adapter ids, strictly increasing.
 * num_segments:  host int32, out: the number of distinct adapters.
 * Returns SGMV_ERR_ADAPTER if an id is negative, SGMV_ERR_NULL / _SHAPE on
 * bad arguments. Runs in O(M log M) on the calling thread.
 */
int sgmv_build_segments(const int32_t *token_adapter, int32_t M, int32_t *perm,
                        int32_t *seg_start, int32_t *seg_adapter, int32_t *num_segments);

/*
 * Host-side check of segment metadata before it is copied to the device
 * (the conditions the calls above state for seg_start and seg_adapter; the
 * Punica guide, "The SGMV Mathematical Formulation": offsets s_0 .. s_N
 * that cover the batch, one adapter per segment).
 *
 * seg_start    host int32[num_segments + 1]; seg_adapter host int32[num_segments].
 * Returns SGMV_OK if seg_start[0] == 0, seg_start[num_segments] == M, the
 * offsets never decrease, and every id lies in [0, num_adapters);
 * SGMV_ERR_SHAPE for a bad offset (or negative sizes), SGMV_ERR_ADAPTER for
 * an id outside the pool, SGMV_ERR_NULL for a missing array. Reads only.
 */
int sgmv_check_segments(const int32_t *seg_start, const int32_t *seg_adapter, int32_t num_segments,
                        int32_t M, int32_t num_adapters);

/*
 * Adapter pool pointer table (Punica guide, figure "SGMV Kernel Memory
 * Layout": an array of pointers, each to one adapter's contiguous memory;
 * section "Core Innovation 2": one unified device buffer holds the hot
 * adapters). Fills ptrs_host[k] = base + k * slot_bytes for k < num_adapters,
 * for a pool whose slots are packed back to back. The caller copies the table
 * to the device. Tables for scattered slots may be filled by the caller
 * directly with any 16-byte aligned device addresses.
 */
int sgmv_pool_pointers(uint64_t *ptrs_host, const void *base, int32_t num_adapters,
                       int64_t slot_bytes);

/*
 * Adapter admission (Punica guide, "Core Innovation 2": the hot adapters live
 * in one unified device pool, and a cold one is copied in from host memory
 * on demand, in under 1.5 ms per adapter over the host link).
 *
 * Enqueues on `stream`, in this order: the copy of A_bytes from A_host to
 * the device slot A_slot, the copy of B_bytes from B_host to B_slot, and the
 * update A_ptrs[slot] = A_slot, B_ptrs[slot] = B_slot (a one-workgroup
 * kernel). An SGMV call enqueued after it on the same stream uses the new
 * adapter; one enqueued before it uses the old entries. The caller keeps
 * A_host and B_host unchanged until the copies complete; with pinned host
 * memory (hipHostMalloc) the call returns at once, with pageable memory the
 * runtime may finish the copy before returning.
 *
 * A_slot, B_slot  device memory of A_bytes / B_bytes, 16-byte aligned: A_k
 *                 as r rows of d_in, B_k as r rows of d_out (the layout above).
 * slot            0 <= slot < num_adapters (the table length).
 * Returns SGMV_ERR_NULL, _SHAPE (slot out of range, zero bytes), _ALIGN or
 * _HIP; nothing is enqueued on error.
 */
int sgmv_admit_adapter(void *A_slot, void *B_slot, const void *A_host, const void *B_host,
                       size_t A_bytes, size_t B_bytes, uint64_t *A_ptrs, uint64_t *B_ptrs,
                       int32_t slot, int32_t num_adapters, void *stream);

/*
 * Measurement helper, not part of SGMV: a streaming read of `bytes` bytes at
 * `src` (device, 16-byte aligned, bytes a multiple of 16) by `num_blocks`
 * workgroups of 256 threads, 16-byte loads, each workgroup writing the XOR
 * of the 32-bit words it read to sink[block] (device uint32[num_blocks]).
 * It gives the HBM rate a plain kernel reaches for a given size, the
 * ceiling the SGMV kernels are compared with. Returns SGMV_ERR_NULL,
 * _SHAPE or _ALIGN on bad arguments.
 */
int sgmv_stream_probe(const void *src, size_t bytes, uint32_t *sink, int32_t num_blocks, void *stream);

/*
 * Workspace status (the sticky word at the start of every workspace, see
 * "Failures seen on the device" above): 0 while every call on the workspace
 * succeeded, else the OR of the bits below.
 */
enum sgmv_ws_status {
    SGMV_WS_WAIT_TIMEOUT = 1, /* a bounded wait between workgroups gave up */
    SGMV_WS_BAD_OFFSETS = 2   /* seg_start decreases somewhere */
};

/*
 * Reads the status word of `workspace` (a workspace of sgmv_shrink,
 * sgmv_fused, the gathered calls or sgmv_fused_layer) into *status after
 * every call enqueued before it on `stream` has completed: it synchronises
 * the stream. A non-zero status stays until the caller zero-fills the
 * workspace (all of it: the failed call may have left leftovers anywhere in
 * it). Returns SGMV_ERR_NULL, or SGMV_ERR_HIP if the copy or the
 * synchronisation failed.
 */
int sgmv_workspace_status(const void *workspace, uint32_t *status, void *stream);

/*
 * Sets how many times a workgroup polls for another's result before it gives
 * up (default 32768, several milliseconds at the least); applies to calls
 * launched afterwards (a captured graph keeps the value it was captured
 * with). Process-wide; returns the previous value. 0 makes every wait give
 * up unless its result is there at the first poll: a way to test the failure
 * path from the host.
 */
uint32_t sgmv_set_wait_limit(uint32_t polls);

/* A static, human-readable name for a status code. */
const char *sgmv_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int sgmv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGMV_H */
