/*
 * moe_ffn.h — C ABI of the MI355X (gfx950) MoE expert-FFN layer.
 *
 * The operation (HyperMegaMoE issue page, section 2.1 "forward fusion" and the
 * parameter table of section 3.1 "Python API"): for T tokens x [T, H], each
 * routed to K experts topk_ids [T, K] with gates topk_weights [T, K],
 *
 *     h_s   = x_t · up_proj_weight[e_s]            up_proj_weight   [E, H, 2I]
 *     act_s = silu(h_s[:, 0:I]) ⊙ h_s[:, I:2I]     (SwiGLU; gate half first)
 *     o_s   = act_s · down_proj_weight[e_s]        down_proj_weight [E, I, H]
 *     y_t   = Σ_k topk_weights[t, k] · o_{t·K+k}   y [T, H]
 *
 * where slot s = t·K + k.  The routing (per-expert counts, prefix-sum offsets,
 * the stable permutation of slots into expert-contiguous order and its
 * inverse), the unpermute and the gate-weighted combine all happen inside the
 * call (section 3.1: the call keeps the full MoE semantics).  The backward
 * (section 2.2 "backward fusion") returns dx, d_up_proj_weight,
 * d_down_proj_weight and d_topk_weights; topk_ids has no gradient.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers to dense row-major arrays owned by
 *    the caller.  The library keeps no pointer after a call returns and holds
 *    no per-call state; two calls with distinct buffers are independent.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous on that stream unless stated otherwise; outputs are valid
 *    once the stream has reached the call.
 *  - Every function returns a moe_ffn_status.  Host-detectable errors (NULL
 *    pointers, sizes, dtypes, alignment, workspace size) are returned before
 *    anything is launched; nothing is written then.
 *  - Device pointers must be 16-byte aligned; H and I must be multiples of 8.
 *  - Workspace `ws` is caller-allocated scratch of at least the size the
 *    matching *_workspace_size query returns; its contents need no
 *    initialisation and are meaningless after the call.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility on the host side; the
 * declarations below are its exported interface. */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

/* Element types. x, both weights, y, dy, dx and the weight gradients share
 * one floating-point dtype; topk_weights and d_topk_weights are fp32. */
typedef enum {
    MOE_FFN_F32 = 0,
    MOE_FFN_BF16 = 1,
    MOE_FFN_I32 = 2, /* topk_ids */
    MOE_FFN_I64 = 3  /* topk_ids */
} moe_ffn_dtype;

typedef enum {
    MOE_FFN_OK = 0,
    MOE_FFN_ERR_NULL = 1,      /* a required pointer is NULL */
    MOE_FFN_ERR_SHAPE = 2,     /* a size is out of the supported range */
    MOE_FFN_ERR_DTYPE = 3,     /* unsupported dtype combination */
    MOE_FFN_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
    MOE_FFN_ERR_WORKSPACE = 5, /* ws_bytes (or saved) smaller than required */
    MOE_FFN_ERR_EXPERT_ID = 6, /* a topk_ids value outside [0, E) (found on the device) */
    MOE_FFN_ERR_SAVED = 7,     /* the saved context does not belong to this problem */
    MOE_FFN_ERR_HIP = 8,       /* a HIP runtime call failed; see moe_ffn_last_error() */
    MOE_FFN_ERR_DEVICE = 9,    /* the current device is not a gfx950 GPU */
    MOE_FFN_ERR_TIMEOUT = 10   /* a wait of the pipelined forward hit its watchdog */
} moe_ffn_status;

/* Problem description.  Limits: 0 <= T, 1 <= K <= 32, 1 <= E <= 1024,
 * T·K < 2^31, 8 <= H, 8 <= I, H % 8 == 0, I % 8 == 0, H·2I < 2^31. */
typedef struct {
    int64_t T, H, I, E, K;
    int32_t dtype;     /* MOE_FFN_F32 or MOE_FFN_BF16 */
    int32_t ids_dtype; /* MOE_FFN_I32 or MOE_FFN_I64 */
    int64_t Is;        /* intermediate width of the shared expert, a multiple of I with
                          E + Is / I <= 1024; 0: no shared expert (the *_shared calls) */
} moe_ffn_problem;

/* Flags. */
#define MOE_FFN_CHECK_IDS 0x1u /* fwd: after routing, synchronise the stream and return
                                  MOE_FFN_ERR_EXPERT_ID before any GEMM runs if an id was
                                  out of range (the call is then synchronous). */
/* fwd, bf16 with H % 256 == 0 and I % 128 == 0: run GEMM1 and GEMM2 as ONE
 * persistent launch with tile-granular release (the overlap explainer page,
 * sections 5-6: a consumer tile starts once the producer tiles it reads have
 * signalled, instead of at a launch boundary), followed by the combine
 * launch.  Device counters in `ws`, zeroed by the routing step of the same
 * call, record per GEMM1 M-tile how many of its N-tiles are done, and a
 * GEMM2 tile waits for all GEMM1 N-tiles of its M-tile.  Tiles are handed out
 * by ticket counters (one per XCD slice of the tile order, a workgroup whose
 * slice is exhausted drawing from the others), and GEMM2 tickets only after
 * every GEMM1 tile has been claimed: a tile is only ever waited for once a
 * running workgroup owns it, so the waits do not depend on how many of the
 * launch's workgroups are resident (another stream's kernel, a partitioned
 * device).  Every wait is also bounded by a watchdog (2 s): on expiry the
 * status word gets MOE_FFN_DEV_TIMEOUT and the kernel still runs to its end,
 * so a stream never hangs; read it with moe_ffn_read_status, or pass
 * MOE_FFN_CHECK_STATUS.  Otherwise (and for other shapes, or with a shared
 * expert) GEMM1 and GEMM2 are separate launches.  Both give bitwise identical
 * outputs.  Without MOE_FFN_PIPELINE or MOE_FFN_BULK the library chooses: the
 * pipelined launch for problems on 64-row tiles (at most 64 routed rows per
 * expert on average, where streaming the weights from HBM bounds both GEMMs
 * and the one launch measured faster), the separate launches otherwise. */
#define MOE_FFN_PIPELINE 0x2u
/* fwd: always run GEMM1 and GEMM2 as separate launches (the bulk twin of the
 * pipelined forward).  MOE_FFN_PIPELINE and MOE_FFN_BULK together are
 * rejected with MOE_FFN_ERR_SHAPE. */
#define MOE_FFN_BULK 0x10u
/* fwd: after the launches, synchronise the stream and read the device status
 * word: MOE_FFN_ERR_TIMEOUT if a pipelined wait hit its watchdog (y is then
 * unreliable), MOE_FFN_ERR_EXPERT_ID if an expert id was out of range (its
 * slot was dropped).  The call is then synchronous. */
#define MOE_FFN_CHECK_STATUS 0x8u
/* Test hook, never for production: the pipelined forward drops the release
 * of one GEMM1 tile and uses a 20 ms watchdog, so that the waits behind it
 * time out (status MOE_FFN_DEV_TIMEOUT) while every kernel still ends. */
#define MOE_FFN_TEST_DROP_RELEASE 0x100u
/* Test hook: the fast-path forward kernels run as 16 workgroups (2 per XCD),
 * so that each workgroup walks many tiles (and, in the pipelined launch, waits
 * on many releases) at sizes a CPU reference checks in full. */
#define MOE_FFN_TEST_SMALL_GRID 0x200u
/* Test hook: the pipelined forward runs as ONE workgroup, which must then
 * claim every tile of every XCD slice itself (its ticket draws move on to the
 * other slices) and still end with the exact result. */
#define MOE_FFN_TEST_ONE_WORKGROUP 0x400u
/* bwd: read the saved context's header on the host first (synchronising the
 * stream) and return MOE_FFN_ERR_SAVED, before anything is launched, if it was
 * not written by a forward of this problem.  Without the flag the same check
 * runs on the device: on a mismatch the backward reads nothing else from
 * `saved`, every output is zero and the workspace status word gets
 * MOE_FFN_DEV_BAD_SAVED. */
#define MOE_FFN_CHECK_SAVED 0x4u
/* Bits of the device status word (moe_ffn_read_status). */
#define MOE_FFN_DEV_BAD_ID 0x1    /* an expert id was outside [0, E); its slot was dropped */
#define MOE_FFN_DEV_TIMEOUT 0x2   /* a pipelined wait hit the watchdog; outputs are unreliable */
#define MOE_FFN_DEV_BAD_SAVED 0x4 /* bwd: the saved context did not belong to this problem */
#define MOE_FFN_DEV_BAD_WS 0x8    /* bwd_w: the workspace did not hold moe_ffn_bwd_d's result for
                                     this saved context; the weight gradients were zeroed */

/* Stages of the forward, for the timing hook below. */
enum {
    MOE_FFN_STAGE_ROUTE = 0,   /* counts, offsets, permutation, inverse index */
    MOE_FFN_STAGE_GEMM1 = 1,   /* gathered up_proj GEMM with the SwiGLU epilogue */
    MOE_FFN_STAGE_GEMM2 = 2,   /* down_proj GEMM */
    MOE_FFN_STAGE_COMBINE = 3, /* unpermute + gate-weighted sum */
    MOE_FFN_STAGE_PIPELINE = 4, /* the pipelined forward's single launch (GEMM1, GEMM2 and
                                   combine); stages 1-3 are then not recorded */
    MOE_FFN_NUM_FWD_STAGES = 5
};

/* Stages of the backward, for the timing hook below. */
enum {
    MOE_FFN_STAGE_BWD_ACT_GRAD = 0,   /* dY gather, dY·W2^T with the SwiGLU backward epilogue */
    MOE_FFN_STAGE_BWD_INPUT_GRAD = 1, /* dh·W1^T per permuted row */
    MOE_FFN_STAGE_BWD_COMBINE = 2,    /* dx k-ordered sum and d_topk_weights */
    MOE_FFN_STAGE_BWD_W2_GRAD = 3,    /* d_down_proj_weight */
    MOE_FFN_STAGE_BWD_W1_GRAD = 4,    /* d_up_proj_weight */
    MOE_FFN_NUM_BWD_STAGES = 5
};

/* Optional per-stage timing: hipEvent_t handles created by the caller (see
 * moe_ffn_event_create).  When an entry is non-NULL the library records it on
 * `stream` right before (begin) / after (end) that stage's launches. */
typedef struct {
    void *begin[8];
    void *end[8];
} moe_ffn_stage_events;

/* ---- forward ------------------------------------------------------------ */

/* Sizes of the forward workspace and of the saved context that the backward
 * needs (a header naming the problem, the route arrays and the pre-activation
 * h = x·up_proj_weight in the problem dtype).  The query half of the
 * two-phase operator interface (HyperMegaMoE issue page, section 2.3: a
 * workspace-size entry and an execute entry per direction; section 5.3: the
 * host computes the workspace size).  Pure host function; no device is
 * touched; errors as moe_ffn_fwd's host checks. */
int moe_ffn_fwd_workspace_size(const moe_ffn_problem *p, uint32_t flags, size_t *ws_bytes,
                               size_t *saved_bytes);

/* y [T, H] = layer(x [T, H], topk_ids [T, K], topk_weights [T, K] fp32,
 *                  up_proj_weight [E, H, 2I], down_proj_weight [E, I, H]).
 * `saved` may be NULL (inference).  When non-NULL it must hold saved_bytes
 * and receives what moe_ffn_bwd needs; it stays owned by the caller.
 * An expert id outside [0, E) never causes an out-of-bounds access: the slot
 * is dropped, a status word in `ws` records it (moe_ffn_read_status) and,
 * with MOE_FFN_CHECK_IDS, the call fails with MOE_FFN_ERR_EXPERT_ID. */
int moe_ffn_fwd(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                const float *topk_weights, const void *up_proj_weight,
                const void *down_proj_weight, void *y, void *saved, void *ws, size_t ws_bytes,
                uint32_t flags, void *stream);

/* Where an inference forward (saved = NULL) leaves its intermediate stages in
 * `ws`, for checking the path stage by stage against a reference (the overlap
 * explainer page, section 6: validate a pipelined operator against the plain
 * stage sequence one stage at a time).  Byte offsets into ws, valid for that
 * problem and flags until ws is used again: counts [E] and offsets [E+1]
 * (int32), sorted_slot [T·K] and slot_pos [T·K] (int32, the routing of
 * moe_ffn_route), act [T·K, I] and o [T·K, H] (problem dtype, rows in the
 * permuted, expert-major order of sorted_slot).  With a shared expert the
 * arrays continue with its Is / I chunks of T rows each.  Also the tile
 * height and the kernel family the forward runs for this problem and flags.
 * Pure host function; a test and debugging hook, not needed to run the
 * layer. */
typedef struct {
    size_t counts, offsets, sorted_slot, slot_pos, act, o;
    int32_t tile_rows; /* rows per M-tile of GEMM1 (and of GEMM2, but for
                          MOE_FFN_KERNEL_TILES_BIG_GEMM2, whose GEMM2 tiles
                          have 256 rows) */
    int32_t kernel;    /* their kernel: MOE_FFN_KERNEL_* */
} moe_ffn_fwd_stage_layout;
#define MOE_FFN_KERNEL_GENERIC 0   /* fp32 */
#define MOE_FFN_KERNEL_ENGINE 1    /* bf16, H % 256 or I % 128 != 0 */
#define MOE_FFN_KERNEL_TILES 2     /* bf16 tile kernel: 64 or 128-row tiles */
#define MOE_FFN_KERNEL_BIG_TILES 3 /* bf16 256 x 256 tile kernel */
#define MOE_FFN_KERNEL_PIPELINED 4 /* bf16 one-launch forward (MOE_FFN_PIPELINE) */
#define MOE_FFN_KERNEL_TILES_BIG_GEMM2 5 /* bf16: GEMM1 on 128-row tiles, GEMM2 on 256 x 256 */
int moe_ffn_fwd_stages(const moe_ffn_problem *p, uint32_t flags, moe_ffn_fwd_stage_layout *layout);

/* moe_ffn_fwd with the per-stage timing hook (ev may be NULL). */
int moe_ffn_fwd_ex(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, void *y, void *saved, void *ws, size_t ws_bytes,
                   uint32_t flags, void *stream, const moe_ffn_stage_events *ev);
/* moe_ffn_fwd, moe_ffn_fwd_ex, moe_ffn_bwd, moe_ffn_bwd_ex, moe_ffn_bwd_d and
 * moe_ffn_bwd_w take problems without a shared expert (Is == 0;
 * MOE_FFN_ERR_SHAPE otherwise). */

/* ---- forward without allocation ------------------------------------------- */

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops and harnesses that forbid hipMalloc.  The
 * inference forward (moe_ffn_fwd with saved = NULL) with its workspace taken
 * from a scratch array the library keeps in device memory:
 * MOE_FFN_NOALLOC_WS_BYTES (64 MiB) per GPU, one copy on each GPU the library
 * runs on, held until the process ends.  Enough for decode-sized batches
 * (T = 128, H = 7168, I = 2048, E = 32, K = 8 needs about 19 MB).  A problem
 * whose workspace (moe_ffn_fwd_workspace_size) exceeds it is rejected with
 * MOE_FFN_ERR_WORKSPACE before anything is launched; so is Is != 0 and
 * MOE_FFN_CHECK_IDS (it copies to the host), with MOE_FFN_ERR_SHAPE.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call);
 * the first call on a device resolves the array's address there.  Every
 * call on one GPU uses the same array, which keeps the last call's contents
 * (the forward initialises everything it reads): calls that overlap on one
 * GPU (different streams, or threads) race and must be serialised by the
 * caller.  Arguments, layout, ownership and the device status word
 * (moe_ffn_read_status is not available: the workspace is private) are
 * otherwise those of moe_ffn_fwd; y is written on `stream`. */
#define MOE_FFN_NOALLOC_WS_BYTES ((size_t)64 << 20)
int moe_ffn_fwd_noalloc(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                        const float *topk_weights, const void *up_proj_weight,
                        const void *down_proj_weight, void *y, uint32_t flags, void *stream);

/* ---- shared expert -------------------------------------------------------- */

/* The optional shared expert (issue page, section 6.1 "shared-expert fused
 * MoE"; the EP overlap issue, section 4.3: its output is added to the combined
 * routed output): a SwiGLU feed-forward that every token passes through,
 *   y[t] = Σ_k g[t,k] · FFN_{e[t,k]}(x[t]) + FFN_s(x[t]),
 *   FFN_s(x) = (silu(x · Ws1[:, :Is]) ⊙ (x · Ws1[:, Is:])) · Ws2,
 * with Ws1 = up_proj_weight [H, 2·Is] and Ws2 = down_proj_weight [Is, H] in
 * the problem dtype, row-major, 16-byte aligned, owned by the caller.  The
 * problem's Is must be a multiple of I: the kernels run the shared expert as
 * Is / I extra experts (column chunk c of the gate and of the up half, row
 * chunk c of Ws2) whose tiles are scheduled with the routed experts' and whose
 * outputs the combine adds after the routed terms (gate 1, chunk order).
 * Workspace and saved sizes (moe_ffn_fwd_workspace_size,
 * moe_ffn_bwd_workspace_size) depend on Is.  MOE_FFN_PIPELINE is ignored here
 * (the bulk launches run). */
typedef struct {
    const void *up_proj_weight;   /* [H, 2·Is] */
    const void *down_proj_weight; /* [Is, H] */
} moe_ffn_shared_weights;
typedef struct {
    void *d_up_proj_weight;   /* [H, 2·Is], overwritten */
    void *d_down_proj_weight; /* [Is, H], overwritten */
} moe_ffn_shared_grads;

/* moe_ffn_fwd_ex with a shared expert (p->Is > 0; with Is == 0 it is
 * moe_ffn_fwd_ex); ev may be NULL. */
int moe_ffn_fwd_shared(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                       const float *topk_weights, const void *up_proj_weight,
                       const void *down_proj_weight, const moe_ffn_shared_weights *shared,
                       void *y, void *saved, void *ws, size_t ws_bytes, uint32_t flags,
                       void *stream, const moe_ffn_stage_events *ev);
/* moe_ffn_bwd_ex with a shared expert (ev may be NULL): also the shared weights' gradients; dx
 * includes the shared expert's contribution, d_topk_weights does not involve
 * it.  `saved` must come from moe_ffn_fwd_shared for the same problem. */
int moe_ffn_bwd_shared(const moe_ffn_problem *p, const void *dy, const void *x,
                       const void *topk_ids, const float *topk_weights,
                       const void *up_proj_weight, const void *down_proj_weight,
                       const moe_ffn_shared_weights *shared, const void *saved, void *dx,
                       void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                       const moe_ffn_shared_grads *d_shared, void *ws, size_t ws_bytes,
                       uint32_t flags, void *stream, const moe_ffn_stage_events *ev);

/* ---- routing alone -------------------------------------------------------- */

/* Workspace for moe_ffn_route. */
int moe_ffn_route_workspace_size(const moe_ffn_problem *p, size_t *ws_bytes);

/* The routing step alone (section 4.1 "routing and expert parallelism"):
 * counts [E], offsets [E+1] (offsets[E] = number of valid slots), the stable
 * permutation sorted_slot [T·K] (position p -> slot s, ordered by expert then
 * by s) and its inverse slot_pos [T·K] (slot s -> position p, -1 for a slot
 * whose id is out of range).  All int32 device arrays owned by the caller. */
int moe_ffn_route(const moe_ffn_problem *p, const void *topk_ids, int32_t *counts,
                  int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, void *ws,
                  size_t ws_bytes, void *stream);

/* ---- backward ------------------------------------------------------------- */

/* Size of the backward workspace: the query half of the backward's
 * two-phase interface (HyperMegaMoE issue page, section 2.3).  Pure host
 * function.  The backward supports bf16 problems (MOE_FFN_ERR_DTYPE for
 * fp32). */
int moe_ffn_bwd_workspace_size(const moe_ffn_problem *p, uint32_t flags, size_t *ws_bytes);

/* Gradients of y with respect to the inputs, given dy [T, H] and the `saved`
 * context written by moe_ffn_fwd for the same problem and inputs (section 2.2):
 * dx [T, H], d_up_proj_weight [E, H, 2I], d_down_proj_weight [E, I, H] in the
 * problem dtype and d_topk_weights [T, K] fp32.  Outputs are overwritten, not
 * accumulated; an expert that received no slot gets exact zero gradients.
 * The weight gradients run beside input_grad and the dx combine (section
 * 2.2): on a second stream the library creates per device (default
 * priority, on the first call), forked from and joined back to `stream` by
 * events, so the outputs are valid once `stream` reaches the call and the
 * call can be captured into a graph like any single-stream work. */
int moe_ffn_bwd(const moe_ffn_problem *p, const void *dy, const void *x, const void *topk_ids,
                const float *topk_weights, const void *up_proj_weight,
                const void *down_proj_weight, const void *saved, void *dx,
                void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                void *ws, size_t ws_bytes, uint32_t flags, void *stream);

/* moe_ffn_bwd with the per-stage timing hook (ev may be NULL; stages
 * MOE_FFN_STAGE_BWD_*). */
int moe_ffn_bwd_ex(const moe_ffn_problem *p, const void *dy, const void *x, const void *topk_ids,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, const void *saved, void *dx,
                   void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                   void *ws, size_t ws_bytes, uint32_t flags, void *stream,
                   const moe_ffn_stage_events *ev);

/* The backward split into its two halves (EP overlap issue, section 2.3
 * "W/D split + deferred W queue" and section 4.5's interface draft: a
 * D-only entry that yields the input gradient, and a W-only entry that a
 * scheduler can defer into an idle window).  Together they compute exactly
 * what moe_ffn_bwd computes, bit for bit.
 *
 * moe_ffn_bwd_d: dx [T, H] and d_topk_weights [T, K] (fp32), from dy, the
 * gates, both weight tensors and `saved`.  It leaves in `ws` (sized by
 * moe_ffn_bwd_workspace_size) the intermediate gradients the weight half
 * reads, stamped with the saved context's identity; the caller must keep
 * `ws` untouched until the matching moe_ffn_bwd_w has been issued.
 *
 * moe_ffn_bwd_w: d_up_proj_weight [E, H, 2I] and d_down_proj_weight [E, I, H],
 * from dy, x, the same `saved` and the `ws` of the moe_ffn_bwd_d call, issued
 * after it on the same stream (or after an event recorded behind it).  If `ws`
 * does not carry the stamp of that `saved` context, nothing is read from it:
 * the weight gradients are written as zeros and the workspace status word
 * gets MOE_FFN_DEV_BAD_WS (with MOE_FFN_CHECK_SAVED the call returns
 * MOE_FFN_ERR_SAVED before launching instead).  Outputs are overwritten, not
 * accumulated.  Pointer, size and error rules are those of moe_ffn_bwd. */
int moe_ffn_bwd_d(const moe_ffn_problem *p, const void *dy, const float *topk_weights,
                  const void *up_proj_weight, const void *down_proj_weight, const void *saved,
                  void *dx, float *d_topk_weights, void *ws, size_t ws_bytes, uint32_t flags,
                  void *stream);
int moe_ffn_bwd_w(const moe_ffn_problem *p, const void *dy, const void *x, const void *saved,
                  void *d_up_proj_weight, void *d_down_proj_weight, void *ws, size_t ws_bytes,
                  uint32_t flags, void *stream);

/* ---- status and measurement helpers ---------------------------------------- */

/* Synchronises `stream`, then reads the device status word that the last
 * forward, route or backward call on this workspace left: 0, or an OR of
 * MOE_FFN_DEV_BAD_ID and MOE_FFN_DEV_TIMEOUT (forward, route) or
 * MOE_FFN_DEV_BAD_SAVED, MOE_FFN_DEV_BAD_WS (backward).  The status word lives
 * in the caller's workspace of the two-phase interface (HyperMegaMoE issue
 * page, section 2.3); conditions only the device can see (an expert id out
 * of range, issue page section 4.2) are reported there instead of failing a
 * call that has already returned.  `ws` is a device pointer; device_status a
 * host pointer; MOE_FFN_ERR_NULL or MOE_FFN_ERR_HIP on failure. */
int moe_ffn_read_status(const void *ws, void *stream, int32_t *device_status);

/* Static text for a status code. */
const char *moe_ffn_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char *moe_ffn_last_error(void);

/* hipEvent helpers for the timing hook, so a caller needs no other HIP
 * binding: create / destroy an event and read the elapsed milliseconds
 * between two recorded events (synchronises on `end`).  For an event that
 * was never recorded (a stage the call's path does not run) the elapsed
 * query returns MOE_FFN_ERR_HIP and leaves no error behind for later calls. */
int moe_ffn_event_create(void **event);
int moe_ffn_event_destroy(void *event);
int moe_ffn_event_elapsed_ms(void *begin, void *end, float *ms);

/* Library version, "major.minor.patch". */
const char *moe_ffn_version(void);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
