/*
 * tcgemm.h -- C ABI of the MI355X (gfx950) dense GEMM library libtcgemm.so.
 *
 * Operation (tensorcore "GEMM", section "Surface"): in BLAS row-major layout,
 *
 *     C[M,N] = alpha * op(A)[M,K] @ op(B)[K,N] + beta * C[M,N]
 *
 * where op(A) = A stored [M,K] (lda >= K) or, with transpose_a, A stored
 * [K,M] (lda >= M); op(B) = B stored [K,N] (ldb >= N) or, with transpose_b,
 * B stored [N,K] (ldb >= K).  A transposed operand is the same storage read
 * with swapped strides; no transpose pass runs (tensorcore "GEMM", section
 * "Transposes").  The NT form is a linear layer's x @ W^T (Phobos "Matrix
 * products", matmul_t).  Leading dims of 0 mean contiguous.  All sizes and
 * leading dims count ELEMENTS.
 *
 * Types (a_dtype == b_dtype; accum_dtype as listed):
 *     f32  x f32  -> f32            accum f32
 *     f16  x f16  -> f16 or f32     accum f32 (always; tensorcore "GEMM",
 *     bf16 x bf16 -> bf16 or f32     section "The 64x64 tile")
 *     i8   x i8   -> i32            accum i32, exact (tessl "Architecture",
 *                                    section "Integer GEMM"); alpha must be 1,
 *                                    beta 0 and K <= 131071 so no sum can wrap.
 * The accumulator stays in registers for the whole K loop and C is written
 * once (tessl "Architecture", section "Two Accumulation Models"); C is read
 * only when beta != 0 (same page, section "Fused Epilogue").  Float results
 * are rounded to c_dtype round-to-nearest-even.  alpha == 0 gives C = beta*C
 * without reading A or B (BLAS convention).
 *
 * Pointers: A, B, C are device pointers owned by the caller (for example the
 * storage of torch tensors).  The library never allocates, frees or retains
 * them.  C must not overlap A or B; A may alias B.
 *
 * Errors (tessl "Architecture", section "The Kernel Library and the nn
 * Boundary"): every argument is validated, with checked 64-bit arithmetic,
 * before anything is enqueued.  A call that returns an error has launched
 * nothing and tc_dispatch_count() is unchanged; tc_last_error() describes the
 * failure.  The library refuses rather than silently falling back.
 *
 * Streams (tensorcore "GEMM", section "Async, batched, and streams"): the
 * _async calls enqueue on a tc_stream and return; tc_stream_sync waits.  The
 * synchronous calls run on the context's own stream and return after the
 * result is in C.  A tc_context is not thread-safe; use one per host thread.
 */
#ifndef TCGEMM_H
#define TCGEMM_H

#include <stdbool.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TC_F32 = 0,
    TC_F16 = 1,
    TC_BF16 = 2,
    TC_I8 = 3,
    TC_I32 = 4
} tc_dtype_t;

typedef enum {
    TC_OK = 0,
    TC_ERR_INVALID_ARGUMENT = 1, /* null pointer, dim < 1, ld too small, non-finite scalar */
    TC_ERR_UNSUPPORTED = 2,      /* dtype combination or int8 alpha/beta outside the contract */
    TC_ERR_OVERFLOW = 3,         /* an extent, index or integer sum would not fit */
    TC_ERR_ALIASING = 4,         /* C overlaps A or B, or batch outputs overlap */
    TC_ERR_OUT_OF_MEMORY = 5,    /* split-K workspace could not be allocated */
    TC_ERR_DEVICE = 6            /* HIP reported an error (message in tc_last_error) */
} tc_status_t;

/* The GEMM descriptor: fields as listed by tensorcore "GEMM", "Surface". */
typedef struct {
    int32_t M, N, K;
    tc_dtype_t a_dtype, b_dtype, c_dtype, accum_dtype;
    bool transpose_a, transpose_b;
    float alpha, beta;
    int32_t lda, ldb, ldc;        /* elements; 0 = contiguous */
} tc_gemm_desc;

/* Batched same-shape GEMM (tensorcore "GEMM", "Async, batched, and
 * streams"): problem z uses A + z*stride_a, B + z*stride_b, C + z*stride_c
 * (strides in elements).  stride_a or stride_b may be 0 (operand shared by
 * every problem); the C ranges of different problems must not overlap. */
typedef struct {
    tc_gemm_desc base;
    int32_t batch;
    int64_t stride_a, stride_b, stride_c;
} tc_gemm_batched_desc;

/* Fused epilogue (tessl "Architecture", section "Fused Epilogue"):
 *
 *     C = activation(alpha * op(A)@op(B) + beta * C + bias)
 *
 * computed while the accumulator is still in registers, so C is written once
 * and read only when beta != 0 -- no separate bias or activation pass.  bias
 * is per column: problem z adds bias[z*bias_stride + n] to every row's column
 * n (the page's row-stride-0 view of a C-shaped tensor), stored in C's
 * element type (c_dtype).  bias may be NULL (activation only).  Activations:
 *     TC_ACT_NONE       identity
 *     TC_ACT_RELU       max(y, 0)
 *     TC_ACT_GELU_TANH  0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))
 * evaluated in fp32 before the single rounding to c_dtype.
 *
 * Per-column dequantization (same page, section "Integer GEMM",
 * gemm_i8_dequant): with col_scale, column n of the product is multiplied by
 * col_scale[z*scale_stride + n] first,
 *
 *     C = activation(alpha * (op(A)@op(B)) * col_scale + beta * C + bias),
 *
 * and int8 inputs may then write a float C (f32, f16 or bf16; accum_dtype
 * TC_I32; alpha and beta any finite values; K <= 131071): the int32 sums are
 * exact, converted to fp32 (rounded to nearest), scaled, and rounded once to
 * c_dtype.  col_scale also applies to float inputs. */
typedef enum {
    TC_ACT_NONE = 0,
    TC_ACT_RELU = 1,
    TC_ACT_GELU_TANH = 2
} tc_activation_t;

typedef struct {
    const void *bias;             /* device pointer, caller-owned; N values of
                                     c_dtype per problem, or NULL */
    int64_t bias_stride;          /* elements between the bias vectors of
                                     consecutive batch problems; 0 = one vector
                                     shared by all (ignored when batch == 1) */
    tc_activation_t activation;
    const float *col_scale;       /* device pointer, caller-owned; N fp32
                                     per-column scales per problem, or NULL */
    int64_t scale_stride;         /* as bias_stride, for col_scale */
} tc_epilogue;

typedef struct tc_context tc_context;
typedef struct tc_stream tc_stream;

/* What the planner chose for a descriptor (introspection, no GPU needed).
 * A call runs one part, or two when a thin ragged strip of the output is
 * split off the whole tiles (the strip runs after them as a GEMM of its
 * own).  Each part launches, in order: pack_a / pack_b when an operand must
 * first be copied into 16-byte row pitches, the GEMM kernel, and the split-K
 * reduction when K is split. */
typedef struct {
    char kernel[128];             /* the launches: names joined by '+', parts by '|' */
    int32_t tile_m, tile_n, tile_k;   /* tile fields: the first (main) part */
    int32_t threads;
    int32_t tiles_m, tiles_n;
    int32_t splits;               /* split-K factor S (1 = no split) */
    int32_t k_per_split;
    int64_t grid;                 /* workgroups of the GEMM launches, all parts */
    int64_t workspace_bytes;      /* split-K partials plus packed operands, the
                                     larger part (parts run one after the other) */
    int32_t launches;             /* kernels one call enqueues (1 to 8) */
    int32_t band;                 /* tile-order band height */
} tc_plan_info;

/* Context: host-side state only; creating one touches no GPU.  The HIP
 * device current at the first launching call (or tc_stream_create/wrap) is
 * bound to the context from then on.  The context owns an internal stream
 * (created at the first synchronous call) for tc_gemm / tc_gemm_batched. */
tc_status_t tc_context_create(tc_context **out);
void tc_context_destroy(tc_context *ctx);

/* Streams.  tc_stream_create owns a new hipStream_t; tc_stream_wrap borrows
 * an existing one (for example torch's current stream) and never destroys
 * it.  Each tc_stream owns the workspace of the calls enqueued on it
 * (split-K partials and packed operand copies; grown on demand, freed by
 * tc_stream_destroy), so two streams never share scratch memory. */
tc_status_t tc_stream_create(tc_context *ctx, tc_stream **out);
tc_status_t tc_stream_wrap(tc_context *ctx, void *hip_stream, tc_stream **out);
tc_status_t tc_stream_sync(tc_stream *s);
void tc_stream_destroy(tc_stream *s);

/* One GEMM, synchronous: returns when C holds the result. */
tc_status_t tc_gemm(tc_context *ctx, const tc_gemm_desc *d,
                    const void *A, const void *B, void *C);

/* One GEMM enqueued on stream s; returns after enqueue. */
tc_status_t tc_gemm_async(tc_context *ctx, const tc_gemm_desc *d,
                          const void *A, const void *B, void *C, tc_stream *s);

/* batch same-shape GEMMs in one GEMM launch per part, synchronous. */
tc_status_t tc_gemm_batched(tc_context *ctx, const tc_gemm_batched_desc *bd,
                            const void *A, const void *B, void *C);

/* Batched, enqueued on stream s. */
tc_status_t tc_gemm_batched_async(tc_context *ctx, const tc_gemm_batched_desc *bd,
                                  const void *A, const void *B, void *C,
                                  tc_stream *s);

/* Allocation-free form of tc_gemm_batched_async, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  Same descriptor, pointers, result and
 * errors, except:
 *   - the scratch memory some plans use (split-K partial sums, packed copies
 *     of operands whose rows are not whole 16-byte chunks) comes from one
 *     static device array of 32 MiB per GPU, held from the library's load
 *     until the process ends, instead of the stream's workspace; a call whose
 *     plan needs more returns TC_ERR_OUT_OF_MEMORY with nothing enqueued
 *     (tc_gemm_plan's workspace_bytes shows the need for aligned pointers);
 *   - it never allocates or frees memory (no hipMalloc, no hipFree) and never
 *     autotunes (the planner's own plan runs).
 * Every call on one GPU shares that GPU's array and leaves its last contents
 * there; no kernel relies on the array starting at zero.  Calls that overlap
 * in time on one GPU (two streams, or two host threads) race on the array:
 * serialize them.  s may not be NULL. */
tc_status_t tc_gemm_batched_async_noalloc(tc_context *ctx, const tc_gemm_batched_desc *bd,
                                          const void *A, const void *B, void *C,
                                          tc_stream *s);

/* Batched GEMM with the fused epilogue *ep (see tc_epilogue), synchronous.
 * Same descriptor, pointers and errors as tc_gemm_batched, plus:
 * TC_ERR_INVALID_ARGUMENT for a NULL ep, an unknown activation or a negative
 * bias_stride / scale_stride; TC_ERR_UNSUPPORTED for int8 inputs into an
 * int32 C (that result is the exact sum; the page refuses the fused form
 * where there is no float result rather than falling back to separate
 * passes) and for int8 into a float C without col_scale; TC_ERR_ALIASING
 * when the bias or scale vectors overlap C; TC_ERR_INVALID_ARGUMENT when
 * they do not lie inside one device allocation.  An ep with no bias, no
 * scale and TC_ACT_NONE computes exactly what tc_gemm_batched computes. */
tc_status_t tc_gemm_epilogue(tc_context *ctx, const tc_gemm_batched_desc *bd,
                             const tc_epilogue *ep, const void *A, const void *B,
                             void *C);

/* The same, enqueued on stream s. */
tc_status_t tc_gemm_epilogue_async(tc_context *ctx, const tc_gemm_batched_desc *bd,
                                   const tc_epilogue *ep, const void *A,
                                   const void *B, void *C, tc_stream *s);

/* First-call autotuning (the tile-class choice the pages leave to a
 * measured cache; tessl "Architecture", "GEMM Pipeline & Kernel Selection").
 * With it on, the first call of each problem (types, layout, M, N, K, batch,
 * leading dims, strides, beta == 0 or not, fused epilogue or not, 16-byte
 * alignment of A and B) runs every candidate plan -- the planner's own, each
 * tile class the input type has (with and without split-K variants), the
 * thin-output kernel and the small-M route where they apply -- on the call's
 * stream, one warm-up and three timed runs each, into a scratch C with beta
 * = 0 (C itself is not touched), keeps the fastest for the context, and then
 * runs the call.  That first call synchronizes the stream, allocates and
 * frees the scratch C, and adds the candidates' launches to
 * tc_dispatch_count.  Later calls with the same key launch only the chosen
 * plan.  Off by default; the environment variable TCGEMM_AUTOTUNE=1 turns it
 * on for contexts created afterwards.  Returns TC_ERR_INVALID_ARGUMENT for a
 * NULL ctx. */
tc_status_t tc_set_autotune(tc_context *ctx, int enable);

/* Number of problems the context has tuned (0 for NULL). */
int64_t tc_autotune_entries(const tc_context *ctx);

/* Validate and plan without touching the GPU or any pointer.  Fills *info
 * (if non-NULL) with the kernel, tile, grid and split-K choice; returns the
 * status the descriptor alone earns.  ctx may be NULL; when non-NULL the
 * error text goes to tc_last_error(ctx). */
tc_status_t tc_gemm_plan(tc_context *ctx, const tc_gemm_batched_desc *bd,
                         tc_plan_info *info);

/* Name of the kernel instantiation the last successful call launched
 * (the analog of tensorcore's tc_last_backend()). "" before any call. */
const char *tc_last_kernel(const tc_context *ctx);

/* Number of kernels this context has launched so far. */
uint64_t tc_dispatch_count(const tc_context *ctx);

/* Measurement hook.  start_event and end_event are hipEvent_t handles the
 * caller created (for example the handles behind two torch.cuda.Event
 * objects).  The next GEMM call on this context that launches a GEMM kernel
 * records start_event on its stream immediately before its main GEMM kernel
 * (the first part's, when the call runs two parts) and end_event right
 * after it, so hipEventElapsedTime gives that kernel's own duration.  One
 * arming serves one call; two NULLs disarm.  Returns TC_ERR_INVALID_ARGUMENT
 * for a NULL ctx or exactly one NULL event.  A failed hipEventRecord makes
 * that GEMM call return TC_ERR_DEVICE. */
tc_status_t tc_time_next_gemm(tc_context *ctx, void *start_event, void *end_event);

/* Static text for a status code; never NULL. */
const char *tc_status_string(tc_status_t status);

/* Text of the last error on this context ("" if none); NULL ctx gives the
 * last error of tc_gemm_plan calls made without a context. */
const char *tc_last_error(const tc_context *ctx);

/* The workgroup -> output tile order every GEMM launch uses, evaluated on the
 * host: workgroup wg of a launch of n_wg = tiles_m*tiles_n*groups workgroups
 * gets tile (*tm, *tn) of group *g (group = batch element x split slice).
 * Workgroups are first regrouped so that each of the 8 XCDs of the chip runs
 * a contiguous range of logical ids; inside a group tiles follow the
 * column-panel band order of tessl "Architecture", "Column-Panel Grid
 * Swizzling", with band height `band` (band <= 0 selects plain row-major).
 * Returns TC_ERR_INVALID_ARGUMENT for wg outside [0, n_wg). */
tc_status_t tc_tile_of_workgroup(int32_t tiles_m, int32_t tiles_n, int32_t groups,
                                 int32_t band, int64_t wg,
                                 int32_t *tm, int32_t *tn, int32_t *g);

/* Library version string. */
const char *tc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TCGEMM_H */
