/*
 * arrms.h - fused rank-partial sum + residual add + RMSNorm on one AMD Instinct
 * MI355X (gfx950), as a C ABI.
 *
 * The operation is the contract of the page "[TLERaw] Add NVSHMEM allreduce
 * RMSNorm tutorial" (FlagTree PR #1122), section Summary, restated in section
 * Implementation 3 ("Residual + RMSNorm epilogue"):
 *
 *     reduced      = sum over W rank partials of x
 *     residual_out = reduced + residual
 *     norm_out     = RMSNorm(residual_out, weight, eps)
 *
 * on BF16 token rows (section Correctness: BF16, hidden size 2048, world size 4),
 * with token rows mapped to independent workgroups (section Implementation 2,
 * "Row-parallel execution").  The W rank partials are W BF16 buffers already
 * resident in this GPU's memory (for example landed there by peer copies); this
 * library moves no data between GPUs.
 *
 * Arithmetic, per element h of token row t (identical in every variant):
 *   acc  = x_0[t][h] + x_1[t][h] + ... + x_{W-1}[t][h]   binary32, rank order
 *   red  = bf16(acc)                                     round to nearest even
 *   ro   = bf16(red + residual[t][h])                    -> residual_out
 *   inv  = (float)(1 / sqrt(sum_h ro^2 / H + eps))       binary64, rounded once
 *   norm = bf16((ro * inv) * weight[h])                  -> norm_out
 *
 * Layout: every [T][H] tensor is BF16 (16-bit bfloat) row-major with row
 * stride H elements; weight is BF16 [H]; eps is binary32.  All pointers are
 * device pointers on the handle's device unless stated otherwise.
 *
 * Ownership: the caller owns every tensor.  A handle owns only its split-H
 * workspace.  Calls are asynchronous on the caller's stream: no host
 * synchronisation, no internal streams, no allocation after arrms_create.
 *
 * Threading: a handle may have at most one arrms_fused in flight at a time
 * (the split-H variant uses the handle's workspace).  Use one handle per
 * stream for concurrent streams.
 */
#ifndef ARRMS_H
#define ARRMS_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define ARRMS_OK 0
#define ARRMS_ERR_INVALID_ARG 1 /* bad pointer, size, eps, alignment or aliasing */
#define ARRMS_ERR_UNSUPPORTED 2 /* a valid request the selected variant cannot run */
#define ARRMS_ERR_HIP 3         /* a HIP call failed; see arrms_last_hip_error */
#define ARRMS_ERR_OOM 4         /* workspace allocation failed in arrms_create */
#define ARRMS_ERR_SCRATCH 5     /* arrms_fused_noalloc: the call needs more than its static scratch */

/* ---- kernel variants ----------------------------------------------------- */
#define ARRMS_VARIANT_AUTO 0   /* choose per call from the shape (default) */
#define ARRMS_VARIANT_ROW 1    /* one token row per workgroup (or per lane group) */
#define ARRMS_VARIANT_SPLITH 2 /* each row split over several workgroups, two kernels */
#define ARRMS_VARIANT_SCALAR 3 /* 8-, 4- or 2-byte loads: any H, any 2-byte alignment */
/* Plan kinds of arrms_reduce (the rank sum alone). */
#define ARRMS_VARIANT_REDUCE 4        /* 16-byte vector loads, flat over T*H elements */
#define ARRMS_VARIANT_REDUCE_SCALAR 5 /* 8-, 4- or 2-byte loads: pointers at different offsets modulo 16 */

#define ARRMS_MAX_WORLD 16        /* largest W */
#define ARRMS_MAX_HIDDEN 65536    /* largest H */
#define ARRMS_ROW_MAX_HIDDEN 16384 /* largest H of the row variant */
#define ARRMS_NOALLOC_SCRATCH_DOUBLES 131072 /* static split-H scratch of arrms_fused_noalloc (1 MiB per GPU) */

typedef struct arrms_ctx* arrms_handle_t;

/* Launch plan of one call, as chosen by arrms_plan / arrms_query_plan. */
typedef struct {
    int variant;         /* ARRMS_VARIANT_ROW, _SPLITH or _SCALAR (0 when tokens == 0) */
    int grid;            /* workgroups launched per kernel (0: nothing is launched) */
    int block;           /* threads per workgroup */
    int vec_per_thread;  /* 16-byte vectors per lane per input (row, split-H); 0 for scalar */
    int threads_per_row; /* lanes sharing one row (row) or one chunk (split-H) */
    int rows_per_block;  /* token rows per workgroup (row), else 1 */
    int chunks_per_row;  /* split-H chunks per row (split-H), else 1 */
    int kernels;         /* kernel launches per call: 2 for split-H, else 1 (0: none) */
    int blocks;          /* logical workgroups per kernel (grid minus padding of the XCD mapping) */
    int xcd_chunk;       /* K > 0: runs of K consecutive workgroups (rows) kept on one XCD; 0: hardware order */
    int elems_per_load;  /* scalar: BF16 elements per load (4, 2 or 1: 8-, 4- or 2-byte loads); rank sum: 8, 4,
                            2 or 1; else 0 */
    int residual_out_cached; /* 1: residual_out written with write-back stores, 0: with streaming (non-temporal)
                                stores; split-H always 1 (its second kernel reads residual_out back); rank sum 0 */
    int rank_loop;       /* 1: the ranks after x_0 are added one load round at a time (the scalar kernel with more
                            than 8 ranks, or chosen automatically for 6-8 ranks; the rank sum with 6 ranks or more
                            and at least 8 workgroups per CU); 0: every rank's loads are issued together */
    int kernarg_preload; /* 1: the kernel takes its arguments as a flat list whose leading 14 dwords (sizes,
                            residual, first partials) are preloaded into scalar registers at wave launch, so its
                            waves start without fetching them (row, scalar and rank sum with W <= 8, calls of at
                            least 16 MiB, where the longer host launch is hidden); 0: one argument block */
} arrms_plan_t;

/* Optional tuning overrides; 0 (or -1 where stated) keeps the automatic choice.
 * None of them changes any result bit, only speed. */
typedef struct {
    int vec_per_thread;    /* row / split-H: 1, 2, 4 or 8 */
    int threads_per_row;   /* row: 16, 32 or a multiple of 64 up to 1024; scalar: lanes per row when a multiple
                              of 64 (capped at 1024) */
    int splith_block;      /* split-H: threads per workgroup, 64..1024, multiple of 64 */
    int splith_max_tokens; /* automatic variant uses split-H when tokens <= this; -1 automatic */
    int xcd_chunk;         /* -1 automatic; 0 hardware round-robin; K > 0 runs of K blocks per XCD */
    int rows_per_block;    /* row: token rows per workgroup (power of two); 0 automatic */
    int scalar_elems;      /* scalar and rank sum: at most this many BF16 elements per load (1, 2 or 4); 0 automatic */
    int residual_out_store; /* row and scalar: 0 or 1 streaming stores (automatic), 2 write-back stores (faster
                               only when the call's data is cache-resident) */
    int kernarg_preload;   /* 0 automatic; 1 never; 2 whenever the kernel has a flat twin (W <= 8, not split-H,
                              not the rank loop).  Calls captured into a HIP graph pay no host launch per replay:
                              there 2 also speeds up decode-sized calls (T = 1 and 64 replayed 4-6 % faster) */
} arrms_tuning_t;

/*
 * Create a handle bound to HIP device `device`.
 * Source: page 1, section Implementation 4 ("Host-side NVSHMEM lifecycle"),
 * which gives the operator's host side an initialization step, symmetric
 * workspace management and a host-side C ABI.  On one GPU that is: bind the
 * device, read its compute-unit count and allocate the workspace, all once,
 * here, so that arrms_fused never allocates.
 *   max_world  : largest W a call will pass, 1..ARRMS_MAX_WORLD
 *   max_tokens : largest T a call will pass, >= 0
 *   max_hidden : largest H a call will pass, 1..ARRMS_MAX_HIDDEN
 * Reads the device's compute-unit count, allocates the split-H workspace
 * (max_tokens * ceil(max_hidden / 512) doubles, written before it is read in
 * every call, so never cleared), and reads the environment variable
 * ARRMS_FORCE_VARIANT (row | splith | scalar) once.  All one-time work
 * happens here.  Returns ARRMS_OK and *out, or ARRMS_ERR_INVALID_ARG (bad
 * limits, out NULL), ARRMS_ERR_HIP (no such device) or ARRMS_ERR_OOM; *out is
 * NULL on error.
 */
int arrms_create(arrms_handle_t* out, int device, int max_world, int max_tokens, int max_hidden);

/*
 * Enqueue the fused operator on `stream` (0 = the null stream of the handle's device).
 * Source: page 1, section Summary (the three-line contract above) and section
 * Implementation 3 (the residual + RMSNorm epilogue after the reduction); rows
 * map to workgroups as in section Implementation 2 (Row-parallel execution).
 *   partials     : HOST array of `world` device pointers, each BF16 [tokens][hidden];
 *                  read at call time, the caller may free the array on return
 *   world        : W, 1..max_world
 *   tokens       : T, 0..max_tokens (0: returns ARRMS_OK, enqueues nothing)
 *   hidden       : H, 1..max_hidden
 *   residual     : BF16 [tokens][hidden]
 *   weight       : BF16 [hidden]
 *   eps          : finite, >= 0
 *   residual_out : BF16 [tokens][hidden] output; may be exactly `residual` (in place)
 *   norm_out     : BF16 [tokens][hidden] output
 * Pointers must be 2-byte aligned.  Outputs may not overlap each other or any
 * input, except residual_out == residual.  Inputs may overlap each other.
 * Only H a multiple of 8 with every pointer 16-byte aligned can use the vector
 * kernels (the automatic choice still gives some of those calls to the scalar
 * kernel where it measured faster: 6-16 ranks with enough rows, rows whose stride
 * is not a multiple of 128 bytes); anything else uses the scalar kernel.  The
 * scalar kernel gives the same results and loads 4 BF16 elements at a time when
 * H % 4 == 0 and every pointer is 8-byte aligned, 2 when H is even and every
 * pointer 4-byte aligned, else 1.
 * All checks happen before anything is enqueued: an error has no side effect.
 * Returns ARRMS_OK, ARRMS_ERR_INVALID_ARG, ARRMS_ERR_UNSUPPORTED (a forced
 * variant cannot run this shape, or the launch would exceed 2^32 - 1 work-items,
 * e.g. T * H beyond about 2^35 elements) or ARRMS_ERR_HIP (launch failure).
 */
int arrms_fused(arrms_handle_t h, const void* const* partials, int world, int tokens, int hidden,
                const void* residual, const void* weight, float eps, void* residual_out,
                void* norm_out, hipStream_t stream);

/*
 * Free the handle's workspace and the handle.  NULL is accepted (ARRMS_OK).
 * Source: page 1, section Implementation 4 ("Host-side NVSHMEM lifecycle"),
 * its resource-cleanup step.
 * The caller must make sure no call on the handle is still executing
 * (synchronise its stream first).  Using a destroyed handle is undefined.
 */
int arrms_destroy(arrms_handle_t h);

/* Static text for a status code ("unknown status" for others).  Part of the
 * host-side C ABI of page 1, section Implementation 4. */
const char* arrms_status_string(int status);

/* hipError_t of the last failed HIP call on this handle (0 if none; -1 for a NULL handle).
 * A HIP failure the library reports through its status is also cleared from HIP's
 * per-thread last-error state, so it does not resurface in the caller's next check. */
int arrms_last_hip_error(arrms_handle_t h);

/* Force a variant (ARRMS_VARIANT_*) for later calls; AUTO restores per-shape choice.
 * Returns ARRMS_ERR_INVALID_ARG for an unknown variant or NULL handle. */
int arrms_set_variant(arrms_handle_t h, int variant);

/* Set (tuning != NULL) or clear (NULL) tuning overrides; checked like arrms_plan. */
int arrms_set_tuning(arrms_handle_t h, const arrms_tuning_t* tuning);

/*
 * Host-only validation and launch planning, exactly as arrms_fused does it,
 * without touching any device: pointers are compared, never dereferenced.
 *   cu_count  : compute units of the device (256 on MI355X)
 *   variant   : ARRMS_VARIANT_* (AUTO chooses)
 *   tuning    : overrides or NULL
 *   max_*     : the limits a handle was created with
 * Other arguments as for arrms_fused.  Fills *plan and returns the status
 * arrms_fused would return before launching.
 */
int arrms_plan(int cu_count, int variant, const arrms_tuning_t* tuning, int max_world,
               int max_tokens, int max_hidden, const void* const* partials, int world, int tokens,
               int hidden, const void* residual, const void* weight, float eps,
               const void* residual_out, const void* norm_out, arrms_plan_t* plan);

/* arrms_plan with the handle's device, limits, forced variant and tuning. */
int arrms_query_plan(arrms_handle_t h, const void* const* partials, int world, int tokens,
                     int hidden, const void* residual, const void* weight, float eps,
                     const void* residual_out, const void* norm_out, arrms_plan_t* plan);

/*
 * The contract's first line on its own: reduced = BF16(sum over W partials),
 * the rank sum of the page's collective stage (section Implementation 1) on
 * this GPU's share, with the same arithmetic as arrms_fused (binary32 sum in
 * rank order from partials[0], one rounding to BF16).  Together with
 * arrms_fused(world = 1, partials = {reduced}) it forms the page's two-stage
 * (collective, then epilogue) form of the operator, and gives the same bits as
 * one arrms_fused call.
 *   partials : HOST array of `world` device pointers, each BF16 [tokens][hidden]
 *   reduced  : BF16 [tokens][hidden] output; may be exactly one of the partials,
 *              may not otherwise overlap them
 * Limits, 2-byte alignment, asynchrony and error behaviour as for arrms_fused.
 * The sum is flat over the T*H elements, so only the pointers' offsets matter:
 * loads are 16 bytes wide when every pointer has the same offset modulo 16 (the
 * few elements before the first aligned one are summed one by one), else 8, 4 or
 * 2 bytes wide, the widest at which the offsets agree.  Uses no workspace.
 */
int arrms_reduce(arrms_handle_t h, const void* const* partials, int world, int tokens, int hidden,
                 void* reduced, hipStream_t stream);

/* Host-only validation and planning of arrms_reduce (see arrms_plan). */
int arrms_plan_reduce(int cu_count, const arrms_tuning_t* tuning, int max_world, int max_tokens,
                      int max_hidden, const void* const* partials, int world, int tokens, int hidden,
                      const void* reduced, arrms_plan_t* plan);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, hosts that forbid hipMalloc): arrms_fused without a
 * handle and without any allocation, on the CURRENT device (hipGetDevice) and
 * `stream`, which must belong to it.  Arguments, layout, aliasing rules,
 * results and error behaviour are those of arrms_fused with the automatic
 * variant, no tuning and the largest limits (world <= ARRMS_MAX_WORLD,
 * hidden <= ARRMS_MAX_HIDDEN, any tokens >= 0).
 * The split-H workspace is a static device array of
 * ARRMS_NOALLOC_SCRATCH_DOUBLES doubles that each GPU holds from its first call
 * until the process ends; its address is looked up once per device, at that
 * device's first call, which should therefore be made outside graph capture.
 * Devices with an index of 64 or more are not served (ARRMS_ERR_HIP).  A call whose plan is split-H and needs more than that,
 * tokens * chunks_per_row doubles (see arrms_plan with ARRMS_MAX_WORLD, INT_MAX
 * tokens and ARRMS_MAX_HIDDEN as limits), returns ARRMS_ERR_SCRATCH and
 * enqueues nothing; other plans use no scratch.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams or host
 * threads) race when they run split-H.  The array needs no clearing (each call
 * writes every slot it reads).  Returns ARRMS_OK, ARRMS_ERR_INVALID_ARG,
 * ARRMS_ERR_UNSUPPORTED, ARRMS_ERR_SCRATCH or ARRMS_ERR_HIP (no current device,
 * the device set-up or the launch failed).
 */
int arrms_fused_noalloc(const void* const* partials, int world, int tokens, int hidden, const void* residual,
                        const void* weight, float eps, void* residual_out, void* norm_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ARRMS_H */
