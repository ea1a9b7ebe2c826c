/*
 * gated_rmsnorm.h - C ABI of the MI355X (gfx950) SiLU-gated RMSNorm
 * training forward and backward.
 *
 * The operator is the "SiLU-gated RMSNorm" training kernel of flashinfer
 * PR #8701, "perf(cake_rmsnorm_silu_gate_train): L2-prefetching extra-long
 * forward on SM107".  Its PR description names a forward and a backward
 * with an optional FP32 weight gradient and a deterministic variant; its
 * commit 10c6017 message names the inputs x and the gate z (called g here)
 * with rows packed; "How the tables were measured" gives BF16 inputs, the
 * operations fwd, bwd (BF16 or FP32 dw) and the checkpointed step
 * (2 x forward + backward).  Per row i of D values, with a weight w of D
 * values shared by all rows:
 *
 *     r_i  = 1 / sqrt(mean_j(x_ij^2) + eps)
 *     y_ij = x_ij * r_i * w_j * silu(g_ij),    silu(v) = v / (1 + exp(-v))
 *
 * and the backward of L = sum(dy * y) gives dx, dg (per row) and
 * dw_j = sum_i dy_ij * x_ij * r_i * silu(g_ij).  The determinism rule of
 * the same kernel family (flashinfer PR #8878, commit message: weight
 * gradients are accumulated in FP32 in one fixed order so that repeated runs
 * agree bit for bit) is applied to dw here: dw is bit-identical from run to
 * run and does not depend on the launch grid.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Layout: every activation (x, g, dy, y, dx, dg) is a row-major
 *    [rows, D] array.  The plain entry points take packed rows (row stride
 *    = D elements); the _strided ones take a row stride per activation, in
 *    elements: D <= stride <= 2^24 and 16-byte rows (a multiple of 8
 *    elements for BF16/FP16, of 4 for FP32), e.g.
 *    x and g as the two halves of a fused [rows, 2D] projection, which the
 *    commit 10c6017 message of flashinfer PR #8701 distinguishes from rows
 *    held packed.  w is [D].
 *  - dtype: the element type of every activation and of w: GRN_DTYPE_BF16
 *    (the type the pages measure), GRN_DTYPE_F16 or GRN_DTYPE_F32.
 *    Arithmetic is FP32; each BF16/FP16 output is rounded once, to nearest
 *    even (FP16 results beyond its range become infinite).  Any finite
 *    input is in range: a row whose sum of squares exceeds FP32 (entries
 *    beyond about 1.8e19) is summed again over x scaled by 2^-70.  With
 *    eps = 0 (or below about 1e-37), rows whose mean square falls below
 *    FP32's smallest normal number (about 1.2e-38) lose accuracy.
 *  - D: 64, 128 or 256 (the pages measure D = 128).
 *  - rows: 0 <= rows <= GRN_MAX_ROWS.  rows = 0 is allowed: the forward does
 *    nothing, the backward writes dw = 0 (an empty sum).  Activation pointers
 *    may then be NULL.
 *  - Memory: every pointer is device memory of the device that owns
 *    `stream`.  The caller owns every buffer; the library allocates nothing,
 *    keeps no pointer after returning and never synchronizes.  Work is only
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream), so
 *    the calls may be captured into a HIP graph.
 *  - Alignment: activations, w and the workspace must be 16-byte aligned;
 *    dw aligned to its element size.
 *  - Aliasing: no output may overlap any input, another output or the
 *    workspace.  Rows of equal stride that interleave without sharing a
 *    byte (dx and dg as the two halves of one fused buffer) do not overlap;
 *    for unequal strides the check is on address ranges (conservative).
 *    An in-place dx = x would let one workgroup overwrite rows that another
 *    has not read yet; the review of flashinfer PR #8878 ("Follow-up"
 *    findings) reports that race for a sibling kernel.
 *  - eps: finite and >= 0.
 *  - Errors: arguments are checked before anything is enqueued; an invalid
 *    call returns a non-zero grn_status and enqueues nothing.  A failed
 *    launch returns GRN_ERR_HIP.  Nothing is thrown across the ABI.
 *  - Threads: the library's only mutable state is the static scratch of
 *    gated_rmsnorm_bwd_noalloc (see there); every other call is safe to make
 *    concurrently, from any thread and on any stream, if the calls share no
 *    output or workspace.
 *  - Launch shape: the environment variable GATED_RMSNORM_MAX_WG, when set
 *    to a positive integer, caps the number of workgroups per launch (a
 *    tuning and testing knob).  Results do not depend on it.
 *  - Testing knob: GATED_RMSNORM_CKPT_SKIP_FIRST_FWD, when set to anything
 *    but "" or "0", makes gated_rmsnorm_ckpt_step(_strided) skip its first
 *    forward, so that y is written by the recomputed forward alone (which
 *    may run inside the backward's launch).  Every output keeps its value;
 *    only which launch writes y changes.
 */
#ifndef GATED_RMSNORM_H
#define GATED_RMSNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum grn_status {
    GRN_OK = 0,
    GRN_ERR_NULL = 1,      /* a required pointer is NULL                     */
    GRN_ERR_SHAPE = 2,     /* D not 64/128/256, rows outside
                              [0, GRN_MAX_ROWS], or a row stride outside
                              [D, 2^24]                                      */
    GRN_ERR_DTYPE = 3,     /* unknown dtype, or dw_fp32 is not 0 or 1        */
    GRN_ERR_ALIGN = 4,     /* a pointer, or a row stride, is not aligned as
                              required                                       */
    GRN_ERR_ALIAS = 5,     /* an output overlaps an input, output or ws      */
    GRN_ERR_WORKSPACE = 6, /* workspace missing or smaller than required     */
    GRN_ERR_EPS = 7,       /* eps is negative, infinite or NaN               */
    GRN_ERR_HIP = 8,       /* the HIP runtime reported a launch error        */
    GRN_ERR_ARG = 9,       /* a flag argument (deterministic) is not 0 or 1,
                              or (gated_rmsnorm_bwd_noalloc) the stream does
                              not belong to the current device              */
    GRN_ERR_SCRATCH = 10   /* gated_rmsnorm_bwd_noalloc: the call needs more
                              than GRN_NOALLOC_SCRATCH_BYTES of workspace    */
} grn_status;

enum { GRN_DTYPE_BF16 = 0, GRN_DTYPE_F16 = 1, GRN_DTYPE_F32 = 2 };

#define GRN_MAX_ROWS ((int64_t)2147483647)

/* Bytes of device workspace the backward needs for `rows` rows of width D,
 * for any element type: a fixed region of arrival counters, one FP32
 * partial dw of D values per chunk of rows (128 or 256 rows a chunk, see
 * gated_rmsnorm_chunk_rows), and one per group of about sqrt(chunks)
 * chunks.  Returns 0 for rows <= 0 or an unsupported D.
 *
 * Workspace contract: the counter region must be zero before the first
 * backward that uses the workspace (see gated_rmsnorm_workspace_init);
 * every backward returns the counters it used to zero before it completes,
 * so the same workspace then serves any later call of any size.  The rest
 * of the workspace is scratch.  Two calls in flight at the same time must
 * not share a workspace. */
size_t gated_rmsnorm_workspace_bytes(int64_t rows, int32_t D);

/* Rows R in one dw chunk of a backward over `rows` rows of D values of type
 * dtype (the workspace holds one partial per chunk; there are ceil(rows/R)
 * chunks).  A chunk is a fixed set of R rows, made of equal blocks that
 * may lie apart in the tensor (which rows form chunk c depends only on c,
 * rows, D and dtype, never on the launch).  R depends only on the row size
 * in bytes (in this version 256 for 128-byte rows, i.e. D = 64 in BF16 or
 * FP16, and 128 otherwise, whatever `rows`); 0 for rows <= 0 or an
 * unsupported D or dtype. */
int32_t gated_rmsnorm_chunk_rows(int64_t rows, int32_t D, int32_t dtype);

/* Forward: y = x * rsqrt(mean(x^2) + eps) * w * silu(g), row by row.
 * In:  x, g [rows, D]; w [D].   Out: y [rows, D]; all of type dtype.
 * y of a row depends only on that row, w and eps: it is bitwise the same
 * whatever the launch shape. */
grn_status gated_rmsnorm_fwd(const void *x, const void *g, const void *w,
                             void *y, int64_t rows, int32_t D, float eps,
                             int32_t dtype, void *stream);

/* Backward of L = sum(dy * y) (r is recomputed from x; nothing is saved by
 * the forward):
 *   dx = r (dn - n c),  n = x r,  dn = dy w silu(g),  c = mean_j(dn n)
 *   dg = dy w n silu'(g)
 *   dw = sum over rows of dy n silu(g)          (overwritten, not added to)
 * In:  x, g, dy [rows, D] and w [D] of type dtype; workspace of at least
 *      gated_rmsnorm_workspace_bytes(rows, D) bytes whose counter region is
 *      zero (see the workspace contract above; may be NULL when rows = 0).
 * Out: dx, dg [rows, D] of type dtype; dw [D], FP32 if dw_fp32 = 1, else
 *      of type dtype.
 * dw is summed in FP32 in a fixed order that depends only on rows, D and
 * dtype (per chunk of rows, then per group of chunks, then over groups): it
 * is bit-identical from run to run and across launch shapes.  The whole
 * backward is one kernel launch (two dependent kernels never run). */
grn_status gated_rmsnorm_bwd(const void *x, const void *g, const void *w,
                             const void *dy, void *dx, void *dg, void *dw,
                             void *workspace, size_t workspace_bytes,
                             int64_t rows, int32_t D, float eps,
                             int32_t dtype, int32_t dw_fp32, void *stream);

/* The checkpointed training step: forward, forward again (recompute, into
 * the same y), then the backward, enqueued on `stream` (flashinfer PR #8701,
 * "How the tables were measured": 2 x forward + backward).  The backward
 * reads x, g, dy and w, not y, so the recomputed forward may run inside the
 * backward's launch (this version does so for the deterministic dw and
 * tensors below 32 MiB); either way both forwards have completed when the
 * stream reaches the next operation.  Arguments are those of
 * gated_rmsnorm_fwd and gated_rmsnorm_bwd together; y must not overlap any
 * other buffer.  Outputs are bitwise those of gated_rmsnorm_fwd followed by
 * gated_rmsnorm_bwd. */
grn_status gated_rmsnorm_ckpt_step(const void *x, const void *g,
                                   const void *w, const void *dy, void *y,
                                   void *dx, void *dg, void *dw,
                                   void *workspace, size_t workspace_bytes,
                                   int64_t rows, int32_t D, float eps,
                                   int32_t dtype, int32_t dw_fp32,
                                   void *stream);

/* Strided forms.  Same as the plain entry points, with each activation's
 * row stride in elements (see Layout above).  Invalid strides:
 * stride < D or > 2^24 -> GRN_ERR_SHAPE; rows not 16-byte aligned ->
 * GRN_ERR_ALIGN.
 * Results are bitwise those of the plain entry points on packed copies.
 *
 * `deterministic` (backward and checkpointed step): 1 gives the fixed-order
 * dw of the plain entry points.  0 adds each chunk's FP32 partial with FP64
 * atomics into one of a few accumulators (15 for D = 128), and the last
 * chunk rounds their sum once (flashinfer PR #8701 ships such a
 * non-deterministic package beside the deterministic one, PR description):
 * dw then meets the same accuracy but its bits are not guaranteed to repeat
 * from run to run.  dx and dg are the same bits either way, and the same
 * workspace serves both.  Other values -> GRN_ERR_ARG. */
grn_status gated_rmsnorm_fwd_strided(const void *x, int64_t x_stride,
                                     const void *g, int64_t g_stride,
                                     const void *w, void *y, int64_t y_stride,
                                     int64_t rows, int32_t D, float eps,
                                     int32_t dtype, void *stream);

grn_status gated_rmsnorm_bwd_strided(const void *x, int64_t x_stride,
                                     const void *g, int64_t g_stride,
                                     const void *w, const void *dy,
                                     int64_t dy_stride, void *dx,
                                     int64_t dx_stride, void *dg,
                                     int64_t dg_stride, void *dw,
                                     void *workspace, size_t workspace_bytes,
                                     int64_t rows, int32_t D, float eps,
                                     int32_t dtype, int32_t dw_fp32,
                                     int32_t deterministic, void *stream);

grn_status gated_rmsnorm_ckpt_step_strided(
    const void *x, int64_t x_stride, const void *g, int64_t g_stride,
    const void *w, const void *dy, int64_t dy_stride, void *y, int64_t y_stride,
    void *dx, int64_t dx_stride, void *dg, int64_t dg_stride, void *dw,
    void *workspace, size_t workspace_bytes, int64_t rows, int32_t D,
    float eps, int32_t dtype, int32_t dw_fp32, int32_t deterministic,
    void *stream);

/* The backward of gated_rmsnorm_bwd, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the same arguments without the workspace, the
 * same kernels and the same output bits.  Its workspace is a static device
 * array inside the library, GRN_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which
 * each GPU the library runs on holds from the library's loading until the
 * process ends.  A call whose gated_rmsnorm_workspace_bytes-style need
 * (counters and partials for `rows` rows of D values of `dtype`; about
 * 4 bytes per row at D = 128, so up to about 16.7 million such rows) exceeds
 * that size returns GRN_ERR_SCRATCH and enqueues nothing.
 *
 * The stream must belong to the calling thread's current device (else
 * GRN_ERR_ARG).  The first call on a device looks up that device's copy of
 * the array and enqueues a small kernel on `stream` that zeroes its arrival
 * counters; every completed backward leaves them at zero again.  All calls on
 * one GPU share its array, which keeps the last call's contents: two calls
 * whose work overlaps on one GPU (other streams, other threads, graphs
 * replayed concurrently) race and may give a wrong dw; serialize them, or
 * use gated_rmsnorm_bwd with one workspace each.  Allocates nothing: no
 * hipMalloc, hipFree or allocating library routine. */
#define GRN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

grn_status gated_rmsnorm_bwd_noalloc(const void *x, const void *g, const void *w,
                                     const void *dy, void *dx, void *dg, void *dw,
                                     int64_t rows, int32_t D, float eps,
                                     int32_t dtype, int32_t dw_fp32, void *stream);

/* Zero the arrival counters at the front of a workspace (the first
 * gated_rmsnorm_workspace_init_bytes() bytes) by enqueueing a small kernel
 * on `stream`.  A workspace must be zero-filled, by this call or by any
 * other means (e.g. hipMemset), once before its first use by
 * gated_rmsnorm_bwd or gated_rmsnorm_ckpt_step.  Errors: NULL workspace ->
 * GRN_ERR_NULL; fewer bytes than the counters need -> GRN_ERR_WORKSPACE;
 * not 16-byte aligned -> GRN_ERR_ALIGN. */
grn_status gated_rmsnorm_workspace_init(void *workspace, size_t workspace_bytes,
                                        void *stream);

/* Size of the counter region that gated_rmsnorm_workspace_init zeroes. */
size_t gated_rmsnorm_workspace_init_bytes(void);

/* Static description of a status code (never NULL). */
const char *gated_rmsnorm_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* GATED_RMSNORM_H */
