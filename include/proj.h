/*
 * proj.h -- C ABI of libproj: the dense projection Y = X . W^T (+ bias)
 *           (-> GELU tanh) on bf16 inputs with fp32 accumulation, for AMD
 *           Instinct MI355X (gfx950).
 *
 * The operation (worklog "How I made Muse's GPU projections 1.32x faster in
 * the Open Kernel Challenge", section "The full equation, now with the
 * letters explained"): for every token row m < M and output feature n < N,
 *     Y[m, n] = sum over k < K of X[m, k] * W[n, k]
 * with W stored one output feature per row, so the product is X times the
 * transpose of W (same page, section "Why the transpose appears").  Inputs
 * are bf16, products are accumulated in fp32 and only the final value is
 * rounded to the output type (same page, section "Inputs, products,
 * accumulators, and outputs are separate choices").  An optional bias is
 * added to the finished sum (same page, section "What makes it linear?",
 * affine maps), and an optional GELU is applied after the bias, written
 * once with the product (page "blackroom" on Devpost, section "How we built
 * it", the GEMM + GELU epilogue row).  GELU is the tanh form
 *     0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))).
 *
 * Layout, all row-major with unit stride on the last axis:
 *   X    bf16 [M, K]   token rows            (element m*K + k)
 *   W    bf16 [N, K]   one row per output    (element n*K + k)
 *   bias bf16 [N]      (only read when the epilogue has a bias)
 *   Y    fp32 or bf16 [M, N]                 (element m*N + n)
 * Pointers are device pointers (hipMalloc'ed or torch CUDA tensors); the
 * caller owns every buffer and keeps it alive until the enqueued work ends.
 * Y must not share memory with X, W or bias (PROJ_ERR_INVALID_ARG).
 * X/W/bias may be any alignment; the fast kernels need X and W 16-byte
 * aligned and K a multiple of 8, and other cases run a slower generic kernel
 * that gives results within the same tolerance.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the legacy
 * default stream).  Once a shape's plan is chosen (the first uncaptured call
 * for a shape measures the candidate plans, synchronising the stream; while
 * it times small shapes it holds a 512 MiB buffer that it reads to flush the
 * caches, then, in its place, copies of the operands for graph timing (at
 * most 512 MiB), all allocated for that tuning call and freed before it
 * returns; see proj_run), proj_run only enqueues work and returns: it never
 * synchronises, allocates or reads device memory on the host, so it may be
 * recorded into a HIP graph (stream capture) -- see "Capture" below.
 *
 * Memory the library owns: per context, the split-K workspace (exactly the
 * caller's bound, given to proj_create) and 1.25 KiB of zero page and sink;
 * per tuning call, the flush buffer and operand copies above; per GPU, the 2 MiB static array
 * of split-K partials that proj_run_noalloc uses (part of the library's code
 * object, held until the process ends).  Nothing else.
 *
 * Errors: every call returns a proj_status; nothing throws across the ABI.
 * Arguments are validated before any HIP call.  HIP failures return
 * PROJ_ERR_HIP and the message is kept in the context (proj_last_error).
 *
 * Environment: PROJ_TUNE=0 takes untimed default plans instead of measuring
 * (see proj_run).  PROJ_PLAN_FILE=<path> keeps measured plans in a text
 * file: every plan a context tunes is appended as one line, keyed by the
 * device (architecture and compute-unit count) and the shape key, and
 * proj_create loads the lines of its device (the last line of a key wins;
 * lines naming a plan this build does not have, or whose split-K partials
 * do not fit the context's workspace, are skipped).  PROJ_LOG=1 prints each
 * plan decision (tuned, default, loaded) to stderr.
 *
 * Threading: a context holds one split-K partial workspace.  Calls that may
 * run at the same time on the GPU (different streams) must use different
 * contexts, or the caller must order them.  Host-side, a context may be used from one
 * thread at a time.
 */
#ifndef PROJ_H
#define PROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct proj_ctx proj_ctx;
typedef struct proj_graph proj_graph;

typedef enum {
    PROJ_OK = 0,
    PROJ_ERR_INVALID_ARG = 1,  /* NULL/negative/inconsistent argument */
    PROJ_ERR_UNSUPPORTED = 2,  /* valid request this library does not do */
    PROJ_ERR_HIP = 3,          /* a HIP runtime call failed */
    PROJ_ERR_NO_MEMORY = 4,    /* workspace or allocation too small/failed */
    PROJ_ERR_NOT_TUNED = 5,    /* tuning requested while the stream captures */
    PROJ_ERR_DESTROYED = 6     /* handle already destroyed */
} proj_status;

typedef enum {
    PROJ_EPI_NONE = 0,           /* Y = X.W^T */
    PROJ_EPI_BIAS = 1,           /* Y = X.W^T + bias */
    PROJ_EPI_GELU_TANH = 2,      /* Y = GELU(X.W^T) */
    PROJ_EPI_BIAS_GELU_TANH = 3  /* Y = GELU(X.W^T + bias) */
} proj_epilogue;

typedef enum {
    PROJ_OUT_F32 = 0,  /* fp32 output, round to nearest even from fp32 */
    PROJ_OUT_BF16 = 1  /* bf16 output, round to nearest even from fp32 */
} proj_out_dtype;

/* Create a context on HIP device `device`.
 *
 * max_workspace_bytes bounds the split-K partial workspace: plans that split
 * K over S workgroups write S fp32 partials of [M][N] (S * M * N * 4 bytes)
 * there before a second kernel sums them (worklog "How I made Muse's GPU
 * projections 1.32x faster in the Open Kernel Challenge", section "The
 * temporary array is a real cost").  The workspace is allocated here, at
 * that size rounded down to 256 bytes; 0 allocates none, and every plan then
 * keeps K whole.  The planner only chooses plans whose partials fit, tuned or
 * default, so proj_run never needs more; proj_run_candidate (and its _hilo /
 * _packed forms) returns PROJ_ERR_NO_MEMORY for a candidate whose partials
 * do not fit, also while the stream captures.  64 MiB covers every split of
 * the weight-streaming shapes up to 64 token rows x 65,536 outputs at S = 4.
 * A 256-byte zero page (masked loads) and a 1 KiB sink are also allocated.
 *
 * Returns PROJ_ERR_INVALID_ARG if ctx is NULL or the device index is out of
 * range, PROJ_ERR_HIP if the device cannot be used (e.g. no GPU),
 * PROJ_ERR_UNSUPPORTED if it is not gfx950, PROJ_ERR_NO_MEMORY if the
 * workspace cannot be allocated. */
proj_status proj_create(proj_ctx **ctx, int device, size_t max_workspace_bytes);

/* Enqueue Y = epilogue(X . W^T [+ bias]) on `stream`.
 *
 * M, N, K >= 0.  M == 0 or N == 0: nothing to do, PROJ_OK.  K == 0: the
 * empty sum is 0, so Y = epilogue(bias or 0).  `epilogue` is a
 * proj_epilogue, `out_dtype` a proj_out_dtype; unknown values give
 * PROJ_ERR_INVALID_ARG, as do NULL X/W/Y (when the sizes need them) and a
 * bias epilogue with bias == NULL.
 *
 * Kernel families: a register-streaming GEMV (M <= 8), an LDS-staged
 * weight-streaming kernel with MFMA (M <= 64, and up to 512 in row blocks),
 * MFMA GEMMs (any M, K a multiple of 32 or 64), and an any-shape kernel;
 * K may be split over workgroups, with a second kernel adding the fp32
 * partials in split order and applying the epilogue (only plans whose
 * partials fit the context's workspace are considered); for fp32 output
 * without GELU a split may instead add its partials straight into Y with
 * fp32 atomics after a fill kernel has zeroed Y (plans named "_atomic").
 * Every plan except those atomic ones gives the same bits on every run of
 * that plan; with an atomic plan the order of the additions, and so the
 * last bits of the result, may change from run to run (the result stays
 * within the accuracy of an fp32 sum).  Different plans add in different
 * orders, so a shape may round differently in another process that tuned
 * another plan (PROJ_PLAN_FILE pins the plans).  Integer-valued sums below
 * 2^24 are exact in every plan.
 *
 * Plan choice (kernel family, tile shape, split count): on the first call
 * for a shape key (M, N, K, epilogue, out dtype, alignment) outside stream
 * capture, every candidate plan is run on the caller's buffers and timed
 * with HIP events; the fastest is cached and used from then on (this first
 * call synchronises `stream` and overwrites Y several times; the last run
 * is the winner's, so Y holds the right result).  Under capture, or with
 * the environment variable PROJ_TUNE=0, an untimed default plan is used and
 * cached as "default" (a later uncaptured proj_tune replaces it).
 *
 * Capture: proj_run never allocates, synchronises or touches the host
 * during capture, and keeps no state between calls on the device (split-K
 * partials are fully rewritten by every call before they are summed), so a
 * captured graph can be replayed any number of times with fresh X.  */
proj_status proj_run(proj_ctx *ctx, const void *X, const void *W, const void *bias,
                     int epilogue, int64_t M, int64_t N, int64_t K, void *Y,
                     int out_dtype, void *stream);

/* proj_run for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, validation and result as proj_run; it runs the
 * plan cached for the shape in ctx (tuned or default), or, when none is
 * cached, the default plan among those whose partials fit the scratch below
 * (not cached, never timed).  It allocates no device memory and never
 * synchronises: a plan that splits K writes its fp32 partials to a static
 * device array of the library, 2 MiB per GPU (held from the first context on
 * that GPU until the process ends), instead of the context's workspace.
 * Returns PROJ_ERR_NO_MEMORY (nothing enqueued) if the plan's partials,
 * S * M * N * 4 bytes, exceed 2 MiB.  Every call on one GPU shares that
 * array, so proj_run_noalloc calls whose kernels may overlap on one GPU
 * (different streams, any contexts) race on it; order them. */
proj_status proj_run_noalloc(proj_ctx *ctx, const void *X, const void *W, const void *bias,
                             int epilogue, int64_t M, int64_t N, int64_t K, void *Y,
                             int out_dtype, void *stream);

/* Measure the candidates for this shape key now and cache the winner, as
 * the first uncaptured proj_run does (also re-tunes a key that holds a
 * default plan).  Returns PROJ_ERR_NOT_TUNED while `stream` is capturing. */
proj_status proj_tune(proj_ctx *ctx, const void *X, const void *W, const void *bias,
                      int epilogue, int64_t M, int64_t N, int64_t K, void *Y,
                      int out_dtype, void *stream);

/* ---- fp32 weights as a bf16 high/low pair (worklog "How I made Muse's GPU
 * projections 1.32x faster in the Open Kernel Challenge", section "Why the
 * high-plus-low router scheme helped"; the router's weights are fp32 in the
 * section "The same calculation shows up in different sizes").
 *
 * Registration: for fp32 W [N][K] (device, row-major), writes Whl, a
 * caller-allocated device array of bf16 [N][2K], row n = [H(n, 0..K-1),
 * L(n, 0..K-1)] with H = bf16(W), L = bf16(W - fp32(H)), both rounded to
 * nearest even.  Enqueued on `stream`; W and Whl stay owned by the caller.
 * N = 0 or K = 0 is a no-op; NULL or misaligned pointers (W to 4, Whl to 2
 * bytes) and negative sizes give PROJ_ERR_INVALID_ARG. */
proj_status proj_prepare_hilo(proj_ctx *ctx, const float *W, int64_t N, int64_t K, void *Whl,
                              void *stream);

/* Y = epilogue(X H^T + X L^T (+ bias)) for X bf16 [M][K] and a registered
 * pair Whl bf16 [N][2K]: one product of depth 2K, fp32 accumulation, whose X
 * columns wrap at K (the high and the low part meet the same X values).
 * Arguments, output and capture rules as proj_run, with K the X row length.
 * The plan is measured per shape as for proj_run, among the kernels that
 * read a wrapped X (the weight-streaming kernel's buffer-resource path when
 * K is a multiple of its stage depth, the persistent GEMM when K is a
 * multiple of 64), with the any-shape kernel as the fallback. */
proj_status proj_run_hilo(proj_ctx *ctx, const void *X, const void *Whl, const void *bias,
                          int epilogue, int64_t M, int64_t N, int64_t K, void *Y,
                          int out_dtype, void *stream);

/* ---- Registered (packed) bf16 weights (worklog "How I made Muse's GPU
 * projections 1.32x faster in the Open Kernel Challenge", section "Weight
 * packing and library descriptors solve related but different problems":
 * the same bf16 values moved to new addresses once, so that each block reads
 * its weights as one contiguous run).
 *
 * Layout for tile height R = 16 * tile16 rows: W [N][K] row-major becomes
 * ceil(N / R) tiles, tile t holding rows t*R .. t*R + R - 1 as K/128
 * consecutive blocks of [R rows][128 columns] (block b holds columns
 * 128b .. 128b + 127); rows past N are zero.  Element (n, k) sits at
 * ((n / R) * K/128 + k / 128) * R * 128 + (n % R) * 128 + k % 128.
 * Values are copied bit for bit.  The streaming kernel then reads a stage of
 * a tile as one contiguous run instead of R row pieces 2K bytes apart.
 * tile16 must be a tile height of the streaming kernel (1, 2, 4 or 7) and K
 * a positive multiple of 128. */

/* Size in bytes of the packed array for (N, K, tile16), or -1 if that
 * packing is not offered. */
int64_t proj_packed_bytes(int64_t N, int64_t K, int tile16);

/* Pack bf16 W [N][K] (device, row-major) into the caller-allocated device
 * array Wp of proj_packed_bytes(N, K, tile16) bytes, enqueued on `stream`.
 * W and Wp stay owned by the caller and must not overlap.  N = 0 or K = 0 is
 * a no-op; invalid sizes, tile heights, NULL or non-16-byte-aligned
 * pointers give PROJ_ERR_INVALID_ARG. */
proj_status proj_pack_weights(proj_ctx *ctx, const void *W, int64_t N, int64_t K, int tile16, void *Wp,
                              void *stream);

/* Y = epilogue(X W^T (+ bias)) with W given packed (Wp, tile16 as packed).
 * Arguments, output and capture rules as proj_run.  The plan is measured
 * per shape among the streaming kernel's variants of that tile height
 * (row blocks and K splits included); PROJ_ERR_UNSUPPORTED where none
 * applies (M above 512, unaligned X or Wp). */
proj_status proj_run_packed(proj_ctx *ctx, const void *X, const void *Wp, int tile16, const void *bias,
                            int epilogue, int64_t M, int64_t N, int64_t K, void *Y, int out_dtype,
                            void *stream);

/* Introspection for packed weights, as for proj_run. */
proj_status proj_get_plan_packed(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int tile16, int epilogue,
                                 int out_dtype, int aligned16, char *buf, size_t buflen);
int proj_num_candidates_packed(int64_t M, int64_t N, int64_t K, int tile16, int epilogue, int out_dtype,
                               int aligned16);
proj_status proj_candidate_name_packed(int64_t M, int64_t N, int64_t K, int tile16, int epilogue,
                                       int out_dtype, int aligned16, int index, char *buf, size_t buflen);
proj_status proj_run_candidate_packed(proj_ctx *ctx, int index, const void *X, const void *Wp, int tile16,
                                      const void *bias, int epilogue, int64_t M, int64_t N, int64_t K,
                                      void *Y, int out_dtype, void *stream);

/* Free the context's device memory and plans (synchronises its device
 * first).  The handle itself stays allocated (a few hundred bytes) as a
 * marker: any later call with it, a second destroy included, returns
 * PROJ_ERR_DESTROYED. */
proj_status proj_destroy(proj_ctx *ctx);

/* Static text for a status code (never NULL). */
const char *proj_status_string(int status);

/* Last error message recorded in ctx ("" if none; never NULL). */
const char *proj_last_error(const proj_ctx *ctx);

/* Introspection: the plan cached for a shape key, as text, e.g.
 * "stream_mt1_nt2_w4_k128_d5_s1 (tuned 24.20us)".  PROJ_ERR_INVALID_ARG if no plan
 * is cached for that key or buf is too small. */
proj_status proj_get_plan(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int epilogue,
                          int out_dtype, int aligned16, char *buf, size_t buflen);

/* Candidate plans for a shape: how many there are, and their names.  Index
 * order is stable for a given library build.  Used by tests to run every
 * kernel variant, and by tools to report the sweep. */
int proj_num_candidates(int64_t M, int64_t N, int64_t K, int epilogue, int out_dtype,
                        int aligned16);
proj_status proj_candidate_name(int64_t M, int64_t N, int64_t K, int epilogue,
                                int out_dtype, int aligned16, int index, char *buf,
                                size_t buflen);

/* Enqueue one specific candidate (index as above), bypassing the plan
 * cache.  Same argument rules as proj_run; PROJ_ERR_INVALID_ARG for an
 * index out of range, PROJ_ERR_NO_MEMORY (nothing enqueued) if its split-K
 * partials need more than the context's workspace (proj_create's bound). */
proj_status proj_run_candidate(proj_ctx *ctx, int index, const void *X, const void *W,
                               const void *bias, int epilogue, int64_t M, int64_t N,
                               int64_t K, void *Y, int out_dtype, void *stream);

/* The same three for a hi/lo pair (proj_run_hilo's shapes; K is the X row
 * length). */
proj_status proj_get_plan_hilo(proj_ctx *ctx, int64_t M, int64_t N, int64_t K, int epilogue,
                               int out_dtype, int aligned16, char *buf, size_t buflen);
int proj_num_candidates_hilo(int64_t M, int64_t N, int64_t K, int epilogue, int out_dtype,
                             int aligned16);
proj_status proj_candidate_name_hilo(int64_t M, int64_t N, int64_t K, int epilogue,
                                     int out_dtype, int aligned16, int index, char *buf,
                                     size_t buflen);
proj_status proj_run_candidate_hilo(proj_ctx *ctx, int index, const void *X, const void *Whl,
                                    const void *bias, int epilogue, int64_t M, int64_t N,
                                    int64_t K, void *Y, int out_dtype, void *stream);

/* Measured read floor (worklog "How I made Muse's GPU projections 1.32x faster
 * in the Open Kernel Challenge", section "A rough way to ask how much room was
 * left": timed plain reads of a weight-sized buffer as the practical floor a
 * weight-streaming projection is compared with).  Enqueues on `stream` one
 * plain streaming read of the `bytes` bytes at device address `buf`
 * (contiguous slabs per workgroup, 16-byte non-temporal loads), so a caller
 * can time it next to proj_run on the same buffers.  Reads only; computes
 * nothing the caller sees.  buf and bytes must be multiples of 16
 * (PROJ_ERR_INVALID_ARG otherwise); bytes = 0 is a no-op. */
proj_status proj_read_probe(proj_ctx *ctx, const void *buf, size_t bytes, void *stream);

/* HIP-graph capture of repeated launches (worklog "How I made Muse's GPU
 * projections 1.32x faster in the Open Kernel Challenge", sections "How I
 * checked whether an idea was actually faster", where the calls ran as
 * graphs, and "Fresh graph replay is a correctness test too": a replay must
 * follow the X it finds, not an answer kept from an earlier run).  Records n_calls proj_run calls, call i using X[i], W[i], bias[i], Y[i]
 * (bias may be NULL, or bias[i] NULL, when the epilogue has none), all with
 * one shape, into a graph on `stream`, and instantiates it.  The plan for
 * the shape is tuned first (outside capture) unless PROJ_TUNE=0.  Replaying
 * the graph re-runs every call on the same buffers, reading whatever X holds
 * at replay time. */
proj_status proj_graph_capture(proj_ctx *ctx, int n_calls, const void *const *X,
                               const void *const *W, const void *const *bias,
                               void *const *Y, int epilogue, int64_t M, int64_t N,
                               int64_t K, int out_dtype, void *stream,
                               proj_graph **graph);

/* Enqueue one replay of the graph on `stream`.  The graph's kernels use its
 * context's workspace: once that context is destroyed, the graph is not
 * replayed and PROJ_ERR_DESTROYED is returned (nothing enqueued).  Destroy a
 * context's graphs before the context; proj_destroy waits for replays
 * already enqueued. */
proj_status proj_graph_launch(proj_graph *graph, void *stream);

/* Free the graph (does not synchronise; the caller waits for replays).  As
 * with contexts, the handle stays allocated as a marker and later calls with
 * it return PROJ_ERR_DESTROYED.  Allowed after its context is destroyed. */
proj_status proj_graph_destroy(proj_graph *graph);

#ifdef __cplusplus
}
#endif

#endif /* PROJ_H */
