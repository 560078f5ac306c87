/*
 * ep.h -- C ABI of libep_mi355x.so: MoE expert-parallel token dispatch,
 * combine, combine backward, static-shape planning and duplicated-expert
 * gradient reduction, as hand-written HIP kernels for MI355X (gfx950).
 *
 * Logical expert-parallel ranks are regions of one receive buffer in the
 * GPU's HBM; nothing here talks to another GPU.
 *
 * Sources the operations follow (cited by page title and section):
 *   NCCL EP paper listing (arXiv 2603.13606): abstract (low-latency and
 *     high-throughput modes), Table II (long-lived groups, per-pass
 *     handles; combine gathers expert outputs back to token order),
 *     Figure 2 (group once, then handle -> dispatch -> expert FFN ->
 *     combine), Table III (LL: 3D expert-major output; HT: 2D output with
 *     token counts), Table IV (tensor tags: tokens, top-k indices, top-k
 *     weights, FP8 scales), Table V (dispatch returns received tokens,
 *     indices and weights plus the handle), Figure 5 (one handle shared by
 *     the forward and backward passes).
 *   MoonEP article (Open Source For You), paragraphs 3-5: fixed per-rank
 *     workload from a GPU planner that picks redundant experts from the
 *     current routing; rows written straight to expert-grouped positions;
 *     static shapes, no per-layer host synchronisation; redundant experts'
 *     weights prefetched into dedicated slots, at most E/R per rank in
 *     training, a small fixed number in inference with the overflow read
 *     from the owner directly; duplicated-expert gradients folded into the
 *     owner's gradients through a reduce buffer.
 *
 * Conventions shared by every call
 *   Memory.     Every tensor is a non-owning view of caller-allocated device
 *               memory, row-major and contiguous.  The library never
 *               allocates or frees device memory.  A handle borrows the
 *               caller's workspace until ep_handle_destroy.
 *   Streams.    `stream` is a hipStream_t (NULL = the default stream).  All
 *               compute calls only enqueue work and return at once.
 *   Errors.     Argument errors are found on the host and returned before
 *               anything is enqueued.  A failed kernel launch returns
 *               EP_ERR_HIP.  Conditions only the data reveals (an expert id
 *               out of range, an LL expert over capacity, a receiver needing
 *               more replica slots than it has) are OR-ed into a device
 *               status word as EP_FLAG_* bits and read with
 *               ep_handle_status, the only call that waits for the GPU.
 *   Dtypes.     tokens bf16; top-k indices int32; top-k weights fp32; FP8
 *               rows OCP e4m3fn (bias 7, max 448); FP8 scales fp32.
 *   Sizes.      H % 8 == 0 (16-byte rows); H % 128 == 0 for FP8 dispatch;
 *               1 <= top_k <= 16; 1 <= E <= 1024; E % R == 0.
 *   Threads.    A handle is used by one stream at a time; calls on one
 *               handle from two streams without ordering race.
 */
#ifndef EP_MI355X_EP_H
#define EP_MI355X_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1,         /* null pointer, bad size or inconsistent config */
  EP_ERR_BAD_TAG = 2,             /* tensor tag does not match the argument's role */
  EP_ERR_BAD_DTYPE = 3,
  EP_ERR_BAD_SHAPE = 4,
  EP_ERR_NOT_PLANNED = 5,         /* dispatch/combine before any ep_plan on the handle */
  EP_ERR_WORKSPACE_TOO_SMALL = 6,
  EP_ERR_UNSUPPORTED = 7,         /* a valid request the library does not serve */
  EP_ERR_HIP = 8                  /* a HIP launch or copy failed */
} ep_status_t;

/* Device-detected conditions (bits of the status word, see ep_handle_status). */
#define EP_FLAG_INDEX_RANGE 1u  /* a top-k index outside [0, E) other than -1; entry skipped */
#define EP_FLAG_CAPACITY 2u     /* LL: an expert got more than `capacity` entries; extra dropped */
#define EP_FLAG_SLOT_BUDGET 4u  /* STATIC, training slot mode: a rank needs more replica slots
                                   than slots_per_rank (the plan is still complete) */
#define EP_FLAG_PLAN_STALL 8u   /* the layout's workgroups, which wait for each other, could not
                                   all run at once within about half a second (the GPU was held
                                   by other work): the layout of that call is incomplete and must
                                   be planned again */
#define EP_FLAG_SCALE_FORMAT 16u /* a group with EP_FP8_SCALES_POW2 (or _AMAX_POW2_WEIGHTS, for the
                                    weights' scales): an FP8 scale handed to the
                                    grouped GEMM was not a positive normal power of two (its
                                    block was taken at the scale's exponent) */

/* Tensor roles (NCCL EP paper listing, Table IV).  EP_TAG_EXPERT_GRADS,
 * EP_TAG_ROUTER_LOGITS and EP_TAG_EXPERT_WEIGHTS are this library's additions
 * for the duplicated-expert gradient reduce, the routing step and the
 * replica-weight prefetch. */
typedef enum ep_tensor_tag {
  EP_TAG_TOKENS = 0,        /* token rows: dispatch in/out, combine in/out, their grads */
  EP_TAG_TOPK_IDX = 1,      /* expert ids (int32); -1 = no expert */
  EP_TAG_TOPK_WEIGHTS = 2,  /* router weights (fp32) and their gradients */
  EP_TAG_FP8_SCALES = 3,    /* one fp32 scale per 128 channels of an FP8 row */
  EP_TAG_EXPERT_GRADS = 4,  /* expert parameter gradients */
  EP_TAG_ROUTER_LOGITS = 5,  /* router scores per token and expert (fp32) */
  EP_TAG_EXPERT_WEIGHTS = 6  /* expert parameters: owners' weights and prefetch slots */
} ep_tensor_tag_t;

typedef enum ep_dtype {
  EP_DTYPE_BF16 = 0,
  EP_DTYPE_FP32 = 1,
  EP_DTYPE_FP8_E4M3 = 2,
  EP_DTYPE_INT32 = 3
} ep_dtype_t;

/* Receive-buffer layouts (NCCL EP listing, Table III; MoonEP article, par. 3-4). */
typedef enum ep_layout {
  EP_LAYOUT_LL = 0,     /* [E, capacity, H]: expert-major, row e*capacity + position */
  EP_LAYOUT_HT = 1,     /* [T*k, H]: rows grouped by expert, expert e from offsets[e] */
  EP_LAYOUT_STATIC = 2  /* [R, C, H], C = ceil(T*k / R): every rank holds exactly its
                           share of rows; hot experts' tail rows go to replicas */
} ep_layout_t;

/* What a STATIC plan does with a replica past a rank's S-th slot (MoonEP
 * article, par. 5).  The plan's rows are the same in both modes. */
typedef enum ep_slot_mode {
  EP_SLOTS_TRAINING = 0,  /* every duplicate needs a slot: overflow sets EP_FLAG_SLOT_BUDGET */
  EP_SLOTS_INFERENCE = 1  /* a small fixed S; overflow segments read the owner's weights
                             directly (seg_slot -1) and set no flag */
} ep_slot_mode_t;

/* How dispatch writes the receive rows.  Cached stores leave the rows in the
 * 256 MB Infinity Cache for the next kernel; past about twice its size they
 * only leave write-backs for that kernel to pay, and non-temporal stores
 * win; small dispatches are latency-bound and gain nothing.  AUTO picks
 * cached stores when one dispatch writes between 64 MiB and 512 MiB of rows,
 * counting the rows of every pass in flight (passes_in_flight): several
 * passes overlapped on their own streams share the cache. */
typedef enum ep_dispatch_stores {
  EP_STORES_AUTO = 0,
  EP_STORES_CACHED = 1,
  EP_STORES_STREAMING = 2  /* non-temporal */
} ep_dispatch_stores_t;

/* How ep_combine writes the token rows it outputs (weighted, and with NULL
 * weights as the backward of dispatch), with the same three values.  AUTO
 * and CACHED leave the rows in the Infinity Cache, where the next layer,
 * which reads them, finds them.  STREAMING writes them non-temporally: a
 * caller whose next kernels stream much more than the cache holds (a
 * training step's backward pass) takes it, since the rows would otherwise be
 * written back while those kernels run. */

/* Format of the fp32 scales of FP8 rows (one per row and 128 channels).
 * The pages fix only that FP8 rows travel with scales (NCCL EP listing,
 * Table IV); both formats are readings.  AMAX: scale = amax / 448, the
 * block's largest value lands on the largest e4m3 code.  POW2: the smallest
 * power of two at or above amax / 448 (at least 2^-126; 1 for an all-zero
 * block), so a scale is an 8-bit exponent and the grouped GEMM's matrix
 * cores apply it themselves: with POW2 the FP8 GEMM of large groups takes
 * the 256 x 256 kernel with no per-block rescaling, and the weights' scales
 * must be powers of two too (ep_quantize_fp8 with POW2 makes such). */
typedef enum ep_fp8_scales {
  EP_FP8_SCALES_AMAX = 0,
  EP_FP8_SCALES_POW2 = 1,
  /* AMAX rows (dispatch and row quantiser as AMAX) against weights whose
   * scales are powers of two (ep_quantize_fp8 with POW2): the FP8 GEMM's
   * matrix cores apply the weight scales and only the row scales are folded
   * per 128-channel block, one fused multiply-add per output element.  A
   * weight scale that is not a power of two raises EP_FLAG_SCALE_FORMAT. */
  EP_FP8_SCALES_AMAX_POW2_WEIGHTS = 2
} ep_fp8_scales_t;

/* Non-owning view of a contiguous row-major device tensor.  data must be
 * 16-byte aligned for the tags TOKENS, EXPERT_WEIGHTS and EXPERT_GRADS (rows
 * move as 16-byte vectors) and 4-byte aligned for the others; a misaligned
 * view is rejected with EP_ERR_INVALID_ARG. */
typedef struct ep_tensor {
  void *data;           /* device pointer (may be NULL only if the tensor is empty) */
  int32_t dtype;        /* ep_dtype_t */
  int32_t tag;          /* ep_tensor_tag_t */
  int32_t ndim;         /* 1..4 */
  int32_t reserved;     /* must be 0 */
  int64_t sizes[4];     /* sizes[0..ndim-1], outermost first */
} ep_tensor_t;

/* Long-lived configuration (NCCL EP listing, Table II: groups). */
typedef struct ep_group_config {
  int32_t num_experts;     /* E, 1..1024 */
  int32_t num_ranks;       /* R logical ranks, E % R == 0; expert e lives on rank e / (E/R) */
  int32_t hidden;          /* H, multiple of 8 */
  int32_t top_k;           /* k, 1..16 */
  int32_t max_tokens;      /* largest T a handle of this group may take */
  int32_t layout;          /* ep_layout_t */
  int32_t capacity;        /* LL only: rows per expert, >= 1 */
  int32_t slots_per_rank;  /* STATIC only: replica slots S per rank, >= 0 */
  int32_t slot_mode;       /* ep_slot_mode_t (STATIC only; 0 otherwise) */
  int32_t dispatch_stores; /* ep_dispatch_stores_t */
  int32_t passes_in_flight; /* passes of this group the caller runs at once (e.g. micro-batches
                               on several streams); 0 or 1 = one.  EP_STORES_AUTO weighs the
                               receive rows of all of them against the Infinity Cache. */
  int32_t fp8_scales;      /* ep_fp8_scales_t: FP8 dispatch scales and the FP8 GEMM's path */
  int32_t combine_stores;  /* ep_dispatch_stores_t: how ep_combine writes its token rows */
} ep_group_config_t;

typedef struct ep_group *ep_group_t;
typedef struct ep_handle *ep_handle_t;

/* Device pointers into a handle's workspace, valid while the handle lives.
 * Contents are defined once the producing call has completed on the stream. */
typedef struct ep_handle_view {
  int32_t num_tokens;      /* T */
  int32_t top_k;           /* k */
  int32_t num_experts;     /* E */
  int32_t num_ranks;       /* R */
  int64_t recv_rows;       /* rows of the receive buffer: T*k (HT), E*cap (LL), R*C (STATIC) */
  int32_t rank_rows;       /* STATIC: C; LL: capacity; HT: T*k */
  int32_t max_segments;    /* STATIC: E + R (size of the segment table), else 0 */
  int32_t *counts;         /* [E]   entries routed to each expert (ep_plan) */
  int32_t *offsets;        /* [E+1] exclusive prefix sum of counts; offsets[E] = total */
  int32_t *dst;            /* [T*k] receive row of entry t*k+j, -1 if skipped/dropped */
  int32_t *recv_src;       /* [recv_rows] entry t*k+j held by each row; written only
                              for rows that hold one: HT rows < offsets[E], LL slots
                              < min(counts[e], capacity) of expert e, STATIC rows
                              < load[r] of rank r.  Other rows are left unchanged. */
  uint32_t *status;        /* [1]   EP_FLAG_* bits of the last ep_plan (+ dup reduce);
                              EP_FLAG_PLAN_STALL is reported by ep_handle_status only */
  /* STATIC only (NULL otherwise): */
  int32_t *keep;           /* [E] rows of e kept on its home rank */
  int32_t *native_row;     /* [E] first row of e's kept rows inside its home rank */
  int32_t *seg_first;      /* [E] first segment of e (segments of e are consecutive) */
  int32_t *seg_count;      /* [E] number of segments of e */
  int32_t *segments;       /* [max_segments][5]: expert, rank, pos_begin, len, row_begin */
  int32_t *n_segments;     /* [1] */
  int32_t *load;           /* [R] rows used on each rank */
  int32_t *replica;        /* [R][S] expert held in each replica slot, -1 if empty */
  int32_t *seg_slot;       /* [max_segments] slot of segment i on its rank (segments[i][1]),
                              -1 if it has none (past the S-th: overflow) */
} ep_handle_view_t;

/* Human-readable name of a status code (static string, never NULL).  The
 * codes are this library's own; the pages name no error interface. */
const char *ep_status_string(ep_status_t st);

/* Validate `cfg` and create a group (host memory only): the long-lived
 * object of the NCCL EP listing's Table II, made once and used by every
 * per-pass handle (Figure 2).
 * Errors: EP_ERR_INVALID_ARG for a NULL argument or a value outside the
 * ranges above; EP_ERR_UNSUPPORTED if the planner's on-chip tables for E
 * and R would not fit. */
ep_status_t ep_group_create(const ep_group_config_t *cfg, ep_group_t *out);
ep_status_t ep_group_destroy(ep_group_t g);

/* Bytes of device workspace a handle for `num_tokens` tokens needs.  The
 * size depends only on the group and num_tokens, so a caller sizes one fixed
 * buffer per pass shape up front and nothing is allocated per layer (MoonEP
 * article, paragraph 4: static shapes avoid per-layer allocation and
 * fragmentation). */
ep_status_t ep_handle_workspace_bytes(ep_group_t g, int32_t num_tokens, size_t *bytes);

/* Rows of the receive buffer for `num_tokens` tokens (see recv_rows): T*k
 * (HT), E*capacity (LL, the 3D expert-major buffer of the NCCL EP listing's
 * Table III) or R*C (STATIC, the fixed per-rank shape of the MoonEP
 * article, paragraphs 3-4). */
ep_status_t ep_group_recv_rows(ep_group_t g, int32_t num_tokens, int64_t *rows);

/* Create a per-pass handle (NCCL EP listing, Table II: handles) over a
 * caller-owned device workspace of `workspace_bytes` bytes, 256-byte
 * aligned and zero-filled when the handle is created (the status word then
 * holds the EP_FLAG_* bits of each call; the layout's handshake words start
 * from zero and are kept consistent by every later call, so a workspace is
 * zeroed once, not per call).  Host bookkeeping only: nothing is
 * enqueued.  Errors: EP_ERR_INVALID_ARG (NULL, misaligned, num_tokens < 0 or
 * > max_tokens), EP_ERR_WORKSPACE_TOO_SMALL. */
ep_status_t ep_handle_create(ep_group_t g, int32_t num_tokens, void *workspace,
                             size_t workspace_bytes, ep_handle_t *out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * handle as ep_handle_create, but its workspace is the library's static
 * device scratch of 16 MiB (EP_SCRATCH_BYTES) on the current device, held by
 * each GPU the library runs on until the process ends, and the handle itself
 * lives in static storage.  Enqueues one zero-filling kernel on `stream`
 * (the workspace contract); calls on the handle must follow it on that
 * stream or after it.  Nothing is allocated, on the device or the host.
 * The device has ONE such handle and ONE scratch: every call returns the
 * same handle object, re-made for the new arguments, and the scratch keeps
 * the last call's contents, so using two of these handles on one device at
 * once, or a handle after the next ep_handle_create_static on that device,
 * races.  ep_handle_destroy on it does nothing.
 * Errors: EP_ERR_INVALID_ARG (NULL, num_tokens < 0 or > max_tokens),
 * EP_ERR_WORKSPACE_TOO_SMALL (the workspace ep_handle_workspace_bytes gives
 * for num_tokens exceeds EP_SCRATCH_BYTES), EP_ERR_HIP (no device, or the
 * clearing kernel failed to launch). */
#define EP_SCRATCH_BYTES ((size_t)16 << 20)
ep_status_t ep_handle_create_static(ep_group_t g, int32_t num_tokens, void *stream,
                                    ep_handle_t *out);
ep_status_t ep_handle_destroy(ep_handle_t h);

/* Device pointers to every table of the handle's last plan (counts, offsets,
 * destinations, the static plan), the routing state that the forward and
 * the backward pass share (NCCL EP listing, Figure 5: one handle for both).
 * Host bookkeeping only; the tables hold valid data once the stream has run
 * the plan.  Errors: EP_ERR_INVALID_ARG for a NULL argument. */
ep_status_t ep_handle_query(ep_handle_t h, ep_handle_view_t *view);

/* Wait for `stream`, then return the status word's EP_FLAG_* bits in *flags.
 * The only blocking call of the library; meant for tests and error checks.
 * Every other call sizes and checks its work on the device, so a pass needs
 * no per-layer host synchronisation (MoonEP article, paragraph 4); data
 * errors are latched in the status word and read here when the caller
 * chooses.  Errors: EP_ERR_INVALID_ARG (NULL), EP_ERR_HIP (the copy or the
 * wait failed). */
ep_status_t ep_handle_status(ep_handle_t h, void *stream, uint32_t *flags);

/* Top-k routing, the gate step before ep_plan ("Ultra-Large MoE Models"
 * article, sections 2.1 and 3.1-3.2: top-k selection over the gate scores,
 * a fused top-k + routing operator).  For every token: the k experts with the
 * largest logits, in descending order (equal logits: lower expert id first;
 * choice 0 is the largest), and weights = softmax over those k logits (fp32,
 * they sum to 1).  With fewer than k experts (E < k) the extra choices are
 * -1 with weight 0.  Logits must be finite.
 * logits:       fp32 [T, E], tag ROUTER_LOGITS.
 * topk_idx:     int32 [T, k] output, tag TOPK_IDX (the input of ep_plan).
 * topk_weights: fp32 [T, k] output, tag TOPK_WEIGHTS.
 * Needs no ep_plan; T, E and k are the handle's. */
ep_status_t ep_route(ep_handle_t h, const ep_tensor_t *logits, ep_tensor_t *topk_idx,
                     ep_tensor_t *topk_weights, void *stream);

/* Routing and layout together: the result of ep_route followed by ep_plan
 * on its topk_idx, with the routing done inside the layout kernel (the
 * fused top-k + routing operator of the "Ultra-Large MoE Models" article,
 * sections 3.1-3.2, carrying on into the per-expert histogram of the NCCL
 * EP listing's Table III layouts): the tile of entries a workgroup ranks is
 * routed by that workgroup, so the ids are ranked from LDS and the pass
 * takes one launch fewer.  Same arguments, outputs and errors as ep_route;
 * afterwards the handle is planned as by ep_plan.  E > 512 routes in a
 * launch of its own first (same results).
 * Cost: the routing then runs on the layout's workgroups (one per 2048
 * entries) instead of one per few tokens, so this is faster than ep_route +
 * ep_plan only when the routing work per tile is small (a few tokens times
 * few experts, such as T = 64, E = 8, k = 2); for decode-sized batches with
 * hundreds of experts the two calls are faster. */
ep_status_t ep_route_plan(ep_handle_t h, const ep_tensor_t *logits, ep_tensor_t *topk_idx,
                          ep_tensor_t *topk_weights, void *stream);

/* Layout (and, for EP_LAYOUT_STATIC, the static-shape plan) of one pass.
 * topk_idx: int32 [T, k], tag EP_TAG_TOPK_IDX.  Writes counts, offsets,
 * dst, recv_src (rows that hold an entry) and the status word; STATIC also
 * writes the plan tables.
 * Rows inside one expert keep the order of the flat entry index t*k + j.
 * HT:     dst = offsets[e] + position of the entry among e's entries.
 * LL:     dst = e*capacity + position; entries past capacity are dropped
 *         (dst = -1, EP_FLAG_CAPACITY).
 * STATIC: every rank r gets exactly floor(N/R) + (r < N mod R) rows (N =
 *         valid entries).  Ranks whose own experts exceed that shed the last
 *         rows of their hottest experts (count descending, id ascending);
 *         the shed runs fill the short ranks in rank order, behind their own
 *         rows; each short rank numbers the distinct experts it receives as
 *         replica slots 0, 1, ...; a segment past the S-th slot has none
 *         (seg_slot -1), which sets EP_FLAG_SLOT_BUDGET in the training
 *         slot mode and is the direct-read overflow in the inference mode.
 * Entries equal to -1 are skipped; other ids outside [0, E) are skipped and
 * set EP_FLAG_INDEX_RANGE.
 * Enqueues one kernel while ceil(T*k / 2048) tiles fit the device's compute
 * units (T*k <= 524288 on MI355X): the tiles wait for each other inside it,
 * a wait bounded so that it ends with EP_FLAG_PLAN_STALL rather than hangs
 * when other work holds the GPU; above that, two kernels.
 * Re-planning a handle invalidates the layout every earlier output used. */
ep_status_t ep_plan(ep_handle_t h, const ep_tensor_t *topk_idx, void *stream);

/* Write every routed token row to its receive row (MoonEP article, par. 4:
 * straight into the expert-grouped position, no staging copy).
 * tokens:            bf16 [T, H], tag TOKENS.
 * topk_weights:      fp32 [T, k], tag TOPK_WEIGHTS; needed only for
 *                    recv_topk_weights, may be NULL otherwise.
 * recv_tokens:       tag TOKENS, [recv_rows, H] or any shape whose leading
 *                    sizes multiply to recv_rows (e.g. [E, cap, H],
 *                    [R, C, H]); bf16 (bit copy) or, when recv_scales is not
 *                    NULL, FP8 e4m3: per token and 128-channel block,
 *                    scale = amax/448 (fp32 division; 1 if amax == 0),
 *                    code = e4m3(clamp(x / scale, -448, 448)), round to
 *                    nearest even.
 * recv_scales:       NULL or fp32 [recv_rows, H/128], tag FP8_SCALES.
 * recv_topk_idx:     NULL or int32 [recv_rows], tag TOPK_IDX: the expert of
 *                    each row, -1 for rows no entry maps to.
 * recv_topk_weights: NULL or fp32 [recv_rows], tag TOPK_WEIGHTS: the router
 *                    weight of each row's entry, 0 for rows no entry maps to.
 * Rows no entry maps to are not written.  EP_ERR_NOT_PLANNED before ep_plan. */
ep_status_t ep_dispatch(ep_handle_t h, const ep_tensor_t *tokens,
                        const ep_tensor_t *topk_weights, ep_tensor_t *recv_tokens,
                        ep_tensor_t *recv_scales, ep_tensor_t *recv_topk_idx,
                        ep_tensor_t *recv_topk_weights, void *stream);

/* ep_plan followed by ep_dispatch, as one call: the same tables and rows,
 * bit for bit.  For the low-latency regime (NCCL EP listing, abstract and
 * Table III: LL mode for small decode batches, where latency is the figure of
 * merit) the layout runs inside the dispatch launch when the layout is LL or
 * HT and T*k <= 2048: every token's workgroup places its own entries by
 * counting, over all T*k ids, the earlier entries of its expert (and, HT,
 * the entries of lower experts), and one more workgroup writes counts,
 * offsets and flags; one launch instead of two (plus the per-row outputs'
 * launch when asked for).  Otherwise it enqueues ep_plan's kernels, then
 * the dispatch.  Arguments, outputs and errors: those of ep_plan (topk_idx)
 * and ep_dispatch (the rest); afterwards the handle is planned. */
ep_status_t ep_plan_dispatch(ep_handle_t h, const ep_tensor_t *topk_idx,
                             const ep_tensor_t *tokens, const ep_tensor_t *topk_weights,
                             ep_tensor_t *recv_tokens, ep_tensor_t *recv_scales,
                             ep_tensor_t *recv_topk_idx, ep_tensor_t *recv_topk_weights,
                             void *stream);

/* FP8 e4m3 quantisation of bf16 rows with the FP8 dispatch's recipe (NCCL EP
 * listing, Table IV: FP8 codes travel with one fp32 scale per 128 channels):
 * per row and 128-wide block, scale = amax/448 (fp32 division; 1 if amax ==
 * 0), code = e4m3(clamp(x / scale, -448, 448)), round to nearest even --
 * bit for bit what ep_dispatch writes for the same row.  For rows that do
 * not come from a dispatch: the activation between the expert FFN's two
 * grouped GEMMs ("Ultra-Large MoE Models" article, section 3.1), so that the
 * second GEMM runs on FP8 operands (ep_expert_gemm_fp8).  Needs no handle.
 * tokens: bf16 [rows, K] (any leading shape), tag TOKENS; K % 128 == 0.
 * codes:  e4m3, the same shape, tag TOKENS.
 * scales: fp32 [rows, K/128] (any leading shape), tag FP8_SCALES.
 * fp8_scales: ep_fp8_scales_t, the scale format (AMAX as above; POW2 the
 *             power of two at or above amax/448, as a POW2 group's dispatch).
 * Errors: EP_ERR_BAD_TAG / _BAD_DTYPE / _BAD_SHAPE / _INVALID_ARG.
 * Enqueues one kernel. */
ep_status_t ep_quantize_fp8(const ep_tensor_t *tokens, ep_tensor_t *codes, ep_tensor_t *scales,
                            int32_t fp8_scales, void *stream);

/* Gather each token's expert outputs back to its place (NCCL EP listing,
 * Table II):  out[t, :] = sum_j w[t, j] * expert_out[dst[t*k+j], :], j
 * ascending, skipped entries contribute nothing, accumulated in fp32.
 * expert_out:   bf16 [recv_rows, H] (any leading shape), tag TOKENS.
 * topk_weights: fp32 [T, k], tag TOPK_WEIGHTS; NULL = all weights 1, which
 *               is the backward of dispatch (sum of a token's row grads).
 * out_tokens:   bf16 or fp32 [T, H], tag TOKENS (rounded to nearest even). */
ep_status_t ep_combine(ep_handle_t h, const ep_tensor_t *expert_out,
                       const ep_tensor_t *topk_weights, ep_tensor_t *out_tokens,
                       void *stream);

/* Backward of ep_combine (NCCL EP listing, Figure 5: same handle as the
 * forward pass).  For every routed entry f = t*k + j with row d = dst[f]:
 *   grad_expert_out[d, h] = bf16(w[t, j] * grad_tokens[t, h])  (the exact
 *                           product rounded once, to nearest even)
 *   grad_topk_weights[t, j] = sum_h grad_tokens[t, h] * expert_out[d, h]
 *                           (fp32 accumulation; 0 for skipped entries)
 * grad_tokens bf16 [T, H] tag TOKENS; expert_out bf16 [recv_rows, H] tag
 * TOKENS; topk_weights fp32 [T, k]; grad_expert_out bf16 [recv_rows, H]
 * tag TOKENS (rows no entry maps to are not written); grad_topk_weights
 * fp32 [T, k] tag TOPK_WEIGHTS. */
ep_status_t ep_combine_bwd(ep_handle_t h, const ep_tensor_t *grad_tokens,
                           const ep_tensor_t *expert_out, const ep_tensor_t *topk_weights,
                           ep_tensor_t *grad_expert_out, ep_tensor_t *grad_topk_weights,
                           void *stream);

/* Fold duplicated-expert gradients into the owners' gradients (MoonEP
 * article, paragraph 5):
 *   owner[e, p] <- fp32(owner[e, p] + sum_{i : expert[i] == e} replica[i, p])
 * the sum taken in fp64 in replica order and rounded once.
 * replica_grads:  bf16 [n, P...], tag EXPERT_GRADS.
 * replica_expert: int32 [n], tag TOPK_IDX (owner expert of each replica,
 *                 -1 = skip; other out-of-range ids are skipped and set
 *                 EP_FLAG_INDEX_RANGE), or NULL to use the handle's STATIC
 *                 replica table, in which case n must be R*S (slot-major).
 * owner_grads:    fp32 [E_owner, P...], tag EXPERT_GRADS; same P.
 * Does not need ep_plan unless replica_expert is NULL. */
ep_status_t ep_dup_grad_reduce(ep_handle_t h, const ep_tensor_t *replica_grads,
                               const ep_tensor_t *replica_expert, ep_tensor_t *owner_grads,
                               void *stream);

/* Replica-weight prefetch (MoonEP article, par. 3 and 5: the planner's
 * redundant experts get their weights prefetched into dedicated slots; each
 * expert projection's weights are contiguous).  After ep_plan of a STATIC
 * handle: for every segment i with seg_slot[i] = s >= 0 on rank
 * r = segments[i][1], slot (r, s) becomes a byte copy of expert
 * segments[i][0]'s row of expert_weights.  Slots the plan leaves empty, and
 * segments without a slot, are not touched (the overflow of the inference
 * slot mode reads the owner's row directly).  Call it once per projection
 * (for FP8 weights, once for the codes and once for their scales).
 * expert_weights: [E, P...], tag EXPERT_WEIGHTS, dtype bf16, fp32 or FP8;
 *                 or the scales of FP8 weights: tag FP8_SCALES, fp32.
 * slot_weights:   [R, S, P...] output, same tag and dtype; the 2-D form
 *                 [R*S, P] is accepted too.
 * A row (P elements) must be a multiple of 4 bytes (rows that are a
 * multiple of 16 bytes take the 16-byte vector path).  Errors:
 * EP_ERR_UNSUPPORTED for a non-STATIC handle, EP_ERR_NOT_PLANNED before
 * ep_plan, EP_ERR_BAD_SHAPE for mismatched sizes.  Reads only the plan
 * tables on the device; enqueues one kernel (none if R*S or P is 0). */
ep_status_t ep_prefetch_replicas(ep_handle_t h, const ep_tensor_t *expert_weights,
                                 ep_tensor_t *slot_weights, void *stream);

/* Grouped GEMM of the experts ("Ultra-Large MoE Models" article, section
 * 3.1: the tokens grouped by expert are multiplied by their expert's
 * weights, one irregularly sized product per expert; NCCL EP listing,
 * Figure 2: the expert FFN between dispatch and combine).  After ep_plan,
 * for every group of receive rows that share a weight matrix and every
 * row i of it, column n < N:
 *   out[i, n] = bf16( sum_c recv_tokens[i, c] * W[n, c] )  (fp32 MFMA
 *   accumulation, rounded once to nearest even)
 * Groups: HT -- expert e's rows [offsets[e], offsets[e+1]); LL -- rows
 * [e*cap, e*cap + min(counts[e], cap)); STATIC -- e's kept rows on its home
 * rank and each segment's rows on its receiving rank, with W the segment's
 * prefetch slot when slot_weights is given and the segment has one, else
 * the owner's matrix (the inference overflow reads the owner directly).
 * recv_tokens:    bf16 [recv_rows, K] (e.g. the dispatch output), tag TOKENS;
 *                 K % 64 == 0.
 * expert_weights: bf16 [E, N, K] (each expert's [N, K] matrix, K
 *                 contiguous), tag EXPERT_WEIGHTS.
 * slot_weights:   NULL, or (STATIC only) bf16 [R, S, N, K] or [R*S, N, K],
 *                 tag EXPERT_WEIGHTS (filled by ep_prefetch_replicas).
 * out:            bf16 [recv_rows, N], tag TOKENS; rows no group covers are
 *                 not written.
 * Errors: EP_ERR_BAD_SHAPE, EP_ERR_UNSUPPORTED (slots for a non-STATIC
 * handle), EP_ERR_NOT_PLANNED.  Enqueues two kernels (the tile table of the
 * current plan, then the GEMM). */
ep_status_t ep_expert_gemm(ep_handle_t h, const ep_tensor_t *recv_tokens,
                           const ep_tensor_t *expert_weights, const ep_tensor_t *slot_weights,
                           ep_tensor_t *out, void *stream);

/* The expert FFN's first GEMM with its activation fused into the store
 * ("Ultra-Large MoE Models" article, section 3.1, names the grouped GEMM as
 * the core of the expert computation; the activation is not given there,
 * and this library reads it as SwiGLU).  The weight rows interleave the two
 * projections: row 2j of each [N, K] matrix is the gate of output j, row
 * 2j + 1 its up projection.  With h[i, n] the bf16 result ep_expert_gemm
 * would write, for every group row i and j < N/2:
 *   out[i, j] = bf16( silu(h[i, 2j]) * h[i, 2j + 1] ),
 *   silu(g) = g / (1 + e^-g) in fp32, the reciprocal to about 1 ulp of
 *   fp32 (for g < -87.34 the reciprocal flushes to zero and so does the
 *   result, where the exact value is below 1.1e-36 |u|).
 * Arguments as for ep_expert_gemm, except out: bf16 [recv_rows, N/2], tag
 * TOKENS, and N % 16 == 0 (else EP_ERR_BAD_SHAPE).  The FFN's second GEMM
 * is ep_expert_gemm over out with K = N/2. */
ep_status_t ep_expert_gemm_swiglu(ep_handle_t h, const ep_tensor_t *recv_tokens,
                                  const ep_tensor_t *expert_weights,
                                  const ep_tensor_t *slot_weights, ep_tensor_t *out,
                                  void *stream);

/* The same grouped GEMM on FP8 operands ("Ultra-Large MoE Models" article,
 * section 3.1, over the receive rows the FP8 dispatch delivers: e4m3 codes
 * with one fp32 scale per 128 channels, NCCL EP listing, Table IV).  The
 * weights come in the same format: one scale per output row n and 128-wide
 * block of K.  A code stands for code * scale, so for every group (as in
 * ep_expert_gemm), row i and column n < N:
 *   out[i, n] = bf16( sum_b recv_scales[i, b] * W_scales[n, b] *
 *                     sum_{c in block b} recv_tokens[i, c] * W[n, c] )
 * (exact e4m3 products, fp32 accumulation, one rounding to nearest even).
 * recv_tokens:   e4m3 [recv_rows, K], tag TOKENS; K % 128 == 0, K <= 2^24.
 * recv_scales:   fp32 [recv_rows, K/128], tag FP8_SCALES.
 * expert_weights: e4m3 [E, N, K], tag EXPERT_WEIGHTS.
 * expert_scales: fp32 [E, N, K/128], tag FP8_SCALES.
 * slot_weights, slot_scales: both NULL, or (STATIC only) e4m3 [R, S, N, K]
 *                and fp32 [R, S, N, K/128] (or [R*S, ...]) filled by
 *                ep_prefetch_replicas, tags EXPERT_WEIGHTS and FP8_SCALES.
 * out:           bf16 [recv_rows, N], tag TOKENS; rows no group covers are
 *                not written.
 * Errors: EP_ERR_BAD_SHAPE, EP_ERR_INVALID_ARG (only one of the slot
 * tensors given), EP_ERR_UNSUPPORTED (slots for a non-STATIC handle, or
 * K > 2^24),
 * EP_ERR_NOT_PLANNED.  Enqueues two kernels (tile table, GEMM). */
ep_status_t ep_expert_gemm_fp8(ep_handle_t h, const ep_tensor_t *recv_tokens,
                               const ep_tensor_t *recv_scales, const ep_tensor_t *expert_weights,
                               const ep_tensor_t *expert_scales, const ep_tensor_t *slot_weights,
                               const ep_tensor_t *slot_scales, ep_tensor_t *out, void *stream);

/* ep_expert_gemm_fp8 with the SwiGLU store of ep_expert_gemm_swiglu: the
 * same interleaved weight rows (codes and scales), out bf16 [recv_rows, N/2],
 * N % 16 == 0 (else EP_ERR_BAD_SHAPE); other arguments and errors as for
 * ep_expert_gemm_fp8. */
ep_status_t ep_expert_gemm_fp8_swiglu(ep_handle_t h, const ep_tensor_t *recv_tokens,
                                      const ep_tensor_t *recv_scales,
                                      const ep_tensor_t *expert_weights,
                                      const ep_tensor_t *expert_scales,
                                      const ep_tensor_t *slot_weights,
                                      const ep_tensor_t *slot_scales, ep_tensor_t *out,
                                      void *stream);

/* ------------------------------------------------------------------------
 * Recorded calls.  A launch-bound loop -- a low-latency decode step, a few
 * kernels of a few microseconds each (NCCL EP listing, Table III: the LL
 * mode for batches of 1 to 128 tokens) -- spends about as much host time
 * entering the library once per operation as the GPU spends on the
 * operations.  A caller can describe the step's calls once and pass the
 * whole list to ep_run_calls every step: one entry into the library, the
 * same work. */

/* The entry point a recorded call makes. */
typedef enum ep_op {
  EP_OP_ROUTE = 1,
  EP_OP_ROUTE_PLAN = 2,
  EP_OP_PLAN = 3,
  EP_OP_DISPATCH = 4,
  EP_OP_PLAN_DISPATCH = 5,
  EP_OP_QUANTIZE_FP8 = 6,
  EP_OP_COMBINE = 7,
  EP_OP_COMBINE_BWD = 8,
  EP_OP_DUP_GRAD_REDUCE = 9,
  EP_OP_PREFETCH_REPLICAS = 10,
  EP_OP_EXPERT_GEMM = 11,
  EP_OP_EXPERT_GEMM_SWIGLU = 12,
  EP_OP_EXPERT_GEMM_FP8 = 13,
  EP_OP_EXPERT_GEMM_FP8_SWIGLU = 14
} ep_op_t;

/* One recorded call.  p holds the entry point's pointer arguments in its
 * own order -- the handle first where it takes one, the tensor views (NULL
 * where the entry point accepts NULL), the stream last; i0 holds its one
 * integer argument (ep_quantize_fp8's fp8_scales; p is then tokens, codes,
 * scales, stream).  Slots past the entry point's arguments are ignored. */
typedef struct ep_call {
  int32_t op; /* ep_op_t */
  int32_t i0;
  void *p[9];
} ep_call_t;

/* Makes calls[0 .. n-1] in order, each exactly as its entry point would be
 * called with those arguments (the same checks, kernels and streams), and
 * stops at the first one that does not return EP_OK.
 * failed: if not NULL, receives the index of that call, or n.
 * Returns the failing call's status, or EP_OK.  EP_ERR_INVALID_ARG for
 * n < 0, for calls == NULL with n > 0, and for a call with an unknown op
 * (its index in *failed).  The list and everything it points to stay the
 * caller's and must stay valid during the call; the kernels it enqueues
 * read the tensors later, as with the entry points themselves. */
ep_status_t ep_run_calls(const ep_call_t *calls, int32_t n, int32_t *failed);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_EP_H */
