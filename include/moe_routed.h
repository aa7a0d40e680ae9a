/*
 * moe_routed.h -- C ABI of the routed mixture-of-experts layer for AMD
 * Instinct MI355X (gfx950): routing plan, activation gather, grouped expert
 * FFN (gate/up projection + SwiGLU, weighted down projection) and a
 * fixed-order combine.
 *
 * Sources of the operations (web pages, cited by title and section):
 *  [P1] "Round 4 Track C: Prefill MoE Plan (mm_clear + mm_hist + mm_scan +
 *       mm_place) & Epilogue / Gather Audit" -- s.1 findings 1-4, s.2
 *       Table 2.1, s.3 Bitwise & Numerical Parity.
 *  [P3] "Batched resident MoE experts on Apple Silicon: a flat parallel expert
 *       pass" -- s.1 Contribution (job list of (token, expert, weight);
 *       gate/up -> gated activation -> weighted down projection), s.3
 *       Results (fixed per-token top-k summation order).
 *  [P4] "Add --moe-mode sweep-prefill: streamed expert supply for CPU
 *       mul_mat_id" -- Mechanism (experts in ascending id order over
 *       contiguous slices).
 *
 * Common conventions
 *  - Entry i = t*K + k: token t's k-th routed expert (token-major), k in the
 *    router's order.
 *  - Element types (enum moe_dtype): activations x, gathered rows xs, expert
 *    weights and the SwiGLU output h share one type D. Accumulation is fp32.
 *    Router weights w, the per-row weight sw, expert outputs y and the layer
 *    output are fp32.
 *  - Weight layouts, row-major: w_gate and w_up [E][d][f] (input index, then
 *    output index), w_down [E][f][d].
 *  - Pointers: every array argument is a DEVICE pointer (hipMalloc'd or
 *    equivalent), owned by the caller. The library allocates and frees no
 *    device memory and keeps no state between calls. Arrays must not alias,
 *    except that a scratch/workspace buffer may be reused by later calls on
 *    the same stream. Structs passed by pointer (sizes, timers) live on the
 *    host.
 *  - Streams: every call enqueues its kernels on `stream` (a hipStream_t; NULL
 *    is the default stream) and returns without waiting. Data-dependent
 *    scalars (row counts) stay on the device in `meta` and are read there by
 *    later calls.
 *  - Outputs need no clearing: every element a call defines is written on
 *    every call.
 *  - Errors: each call returns MOE_OK or an error code; nothing prints, throws
 *    or aborts. MOE_EINVAL: a NULL or misaligned pointer (data arrays need
 *    16-byte alignment, index arrays 4-byte), a size out of range, an
 *    undersized scratch or workspace. MOE_EUNSUPPORTED: a valid request this
 *    build does not implement (E > MOE_MAX_EXPERTS). MOE_EHIP: the HIP
 *    runtime refused a launch (e.g. no device). Argument checks happen before
 *    any HIP call.
 *  - Ids: -1 marks a skipped entry ([P1] s.3: experts skipped by tail
 *    skipping); it gets no row and pos = -1. Any other id outside [0, E) is
 *    counted in meta[MOE_META_NBAD] and treated the same way.
 *  - Inconsistent plan arrays passed to the later calls (made up rather than
 *    produced by moe_plan) give unspecified values but never an access
 *    outside the stated array sizes: row and token indices are clamped to
 *    their bounds on the device.
 */
#ifndef MOE_ROUTED_H
#define MOE_ROUTED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moe_stream_t; /* hipStream_t */

enum moe_dtype { MOE_F32 = 0, MOE_F16 = 1, MOE_BF16 = 2 };

enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = 1,
    MOE_EUNSUPPORTED = 2,
    MOE_EHIP = 3,
    MOE_ENOSPACE = 4 /* larger than the fixed buffer of moe_forward_packed_noalloc */
};

/* Fields of the device array meta[MOE_META_N] written by moe_plan. */
enum moe_meta_field {
    MOE_META_NENT = 0,    /* T*K entries */
    MOE_META_NBLK = 1,    /* plan blocks of MOE_PLAN_BLOCK entries */
    MOE_META_NR = 2,      /* rows of the expert-sorted list, pads included */
    MOE_META_NT = 3,      /* tiles of tm rows: nr / tm */
    MOE_META_NACTIVE = 4, /* experts with at least one entry */
    MOE_META_MAXCNT = 5,  /* largest entry count of one expert */
    MOE_META_NSKIP = 6,   /* entries with id -1 */
    MOE_META_NBAD = 7,    /* entries with another id outside [0, E) */
    MOE_META_TM = 8,
    MOE_META_E = 9,
    MOE_META_K = 10,
    MOE_META_N = 11
};

#define MOE_MAX_EXPERTS 1024 /* one plan counter per expert in LDS ([P1] s.1 finding 1: 1024 counters) */
#define MOE_PLAN_BLOCK 1024  /* entries per plan block (the page's block size) */

#define MOE_ROUTE_MAX_K 64     /* picks per token of moe_route_topk (one wave lane each) */

/*
 * moe_route_topk -- the router step before the plan ([P1] s.1 finding 5 and
 * s.3 name route_topk, which writes the routed ids). Per token: a softmax over
 * the E logits, the K largest probabilities kept and renormalised to sum to
 * one -- equivalently the K largest logits, weight k = exp(l_k - m) / sum over
 * the K picks of exp(l_j - m), m the largest logit. Picks are in descending
 * order; equal logits go to the lower expert id; NaN logits are never picked
 * and if fewer than K logits are not NaN the remaining picks are id -1 with
 * weight 0. fp32 arithmetic, exponentials summed in pick order.
 * In:  logits [T][E] fp32. Out: ids [T*K] int32, w [T*K] fp32 (the inputs of
 * moe_plan / moe_forward).
 * Errors: MOE_EINVAL for T, E or K < 1, K > E, NULL/misaligned pointers;
 * MOE_EUNSUPPORTED for E > MOE_MAX_EXPERTS or K > MOE_ROUTE_MAX_K; MOE_EHIP
 * on a failed launch.
 */
int moe_route_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                   moe_stream_t stream);

/* Host-side sizes of a plan. */
typedef struct {
    int64_t nent;         /* T*K */
    int64_t nblk;         /* ceil(nent / MOE_PLAN_BLOCK) */
    int64_t max_rows;     /* upper bound of nr: rows to allocate for stok, sw, xs, h, y */
    int64_t max_tiles;    /* max_rows / tm */
    size_t scratch_bytes; /* device scratch moe_plan needs */
} moe_plan_sizes_t;

/*
 * moe_plan_sizes -- host only, no HIP call.
 * max_rows = ceil((T*K + min(E, T*K)*(tm-1)) / tm) * tm: every valid entry has
 * a row and each active expert adds at most tm-1 pad rows.
 * Returns MOE_EINVAL if T, K, E or tm < 1, T*K >= 2^31 or max_rows >= 2^31;
 * MOE_EUNSUPPORTED if E > MOE_MAX_EXPERTS.
 */
int moe_plan_sizes(int T, int K, int E, int tm, moe_plan_sizes_t *out);

/*
 * moe_plan -- the routing plan ([P1] s.1 findings 1 and 2; s.3 lists the
 * outputs): a per-block expert histogram, a prefix scan of the per-expert
 * counts padded up to a multiple of tm (pad rows marked -1 in the same pass),
 * and a placement of every entry into an expert-sorted row list. Experts are
 * laid out in ascending id order ([P4] Mechanism). Inside one expert the rows
 * follow entry order (stable by token, then k), so the plan is unique.
 *
 * In:  ids [T*K] int32, w [T*K] fp32 (router weight of each entry).
 * Out: cnt [E]            entries per expert
 *      eoff [E+1]         first row of each expert; eoff[E] = nr
 *      tiles [max_tiles]  expert of each tm-row tile, tiles [0, nt) written
 *      stok [max_rows]    token of each row; -1 on pad rows; rows [0, nr) written
 *      sw [max_rows]      router weight of each row (bit copy of w); +0.0 on pad rows
 *      pos [T*K]          row of each entry; -1 for skipped/bad entries
 *      boff [nblk*E]      entries of expert e in the blocks before block b, at [b*E + e]
 *      meta [MOE_META_N]  see enum moe_meta_field
 * scratch: device buffer of at least moe_plan_sizes().scratch_bytes.
 * Errors: as moe_plan_sizes, plus MOE_EINVAL for NULL/misaligned pointers or
 * a small scratch; MOE_EHIP on a failed launch.
 */
int moe_plan(const int32_t *ids, const float *w, int T, int K, int E, int tm, int32_t *cnt,
             int32_t *eoff, int32_t *tiles, int32_t *stok, float *sw, int32_t *pos, int32_t *boff,
             int32_t *meta, void *scratch, size_t scratch_bytes, moe_stream_t stream);

/*
 * moe_gather -- [P1] s.1 finding 4: copy each routed token's row of the
 * half-precision activation into expert-contiguous rows, bit for bit.
 * xs[r][:] = x[stok[r]][:] for r < min(meta[MOE_META_NR], max_rows); pad rows
 * (stok[r] < 0) become all-zero bits. Rows >= nr are not touched.
 * In:  x [T][d] of dtype, stok [max_rows], meta [MOE_META_N] (device, from moe_plan).
 * Out: xs [max_rows][d] of dtype.
 * Errors: MOE_EINVAL for d < 8 or d % 8 != 0, T < 1, max_rows < 1, bad dtype,
 * NULL/misaligned pointers; MOE_EHIP on a failed launch.
 */
int moe_gather(const void *x, int dtype, int T, int d, const int32_t *stok, const int32_t *meta,
               int64_t max_rows, void *xs, moe_stream_t stream);

/*
 * moe_ffn_scratch_bytes -- host only: scratch moe_expert_ffn needs for a plan
 * of at most max_rows rows over E experts with tile tm, hidden size d,
 * intermediate size f and element type dtype (the work list, plus fp32
 * partial sums when a projection is split along its reduction, see
 * moe_ffn_splits).
 * Errors: MOE_EINVAL for NULL bytes, E/tm/max_rows < 1, d or f not positive
 * multiples of 8, bad dtype; MOE_EUNSUPPORTED for E > MOE_MAX_EXPERTS.
 */
int moe_ffn_scratch_bytes(int E, int d, int f, int tm, int64_t max_rows, int dtype,
                          size_t *bytes);

/*
 * moe_ffn_splits -- host only: into how many reduction ranges moe_expert_ffn
 * (and moe_forward) split the gate/up projection (over d) and the down
 * projection (over f) for these sizes. A projection is split when the bound on
 * its work items is too small to occupy the GPU (decode-sized batches); the
 * partial sums are then added in a fixed order, so results stay deterministic
 * run to run but differ in rounding from the unsplit order. Same argument
 * checks as moe_ffn_scratch_bytes.
 */
int moe_ffn_splits(int E, int d, int f, int tm, int64_t max_rows, int dtype, int *split_gateup,
                   int *split_down);

/*
 * moe_ffn_big_cells -- host only: which projections of the packed entry
 * points (moe_expert_ffn_packed, moe_forward_packed) with fp16 or bf16 run
 * each expert's runs of 4 work items (256 rows) on 512-thread workgroups of
 * 256 rows x 256 weight columns whose operands are staged in LDS (a separate
 * launch before the other work items): *on bit 0 = the gate/up projection,
 * bit 1 = the down projection. Used when the plan bound averages at least 64
 * rows per expert, for a projection that is not split. The results are the
 * same bits either way. Same argument checks as moe_ffn_scratch_bytes.
 */
int moe_ffn_big_cells(int E, int d, int f, int tm, int64_t max_rows, int dtype, int *on);

/*
 * moe_expert_ffn -- the grouped expert FFN over the expert-sorted rows
 * ([P3] s.1: gate/up projection, gated activation, weighted down projection
 * per job; [P1] s.1 finding 5 names the SwiGLU and down-projection epilogue
 * kernels). For every row r in expert e's range [eoff[e], eoff[e+1]):
 *   g = xs[r] . w_gate[e],  u = xs[r] . w_up[e]            (fp32 accumulation)
 *   h[r][j] = D( silu(g[j]) * u[j] ),  silu(z) = z / (1 + exp(-z))
 *   y[r][c] = sw[r] * sum_j h[r][j] * w_down[e][j][c]      (fp32)
 * h is stored in D (the operand type of the down projection, like the page's
 * half SwiGLU output) for every row of every expert range; y is stored only
 * on rows with stok[r] >= 0 (pad rows are never read by moe_combine).
 * In:  xs [max_rows][d], w_gate/w_up [E][d][f], w_down [E][f][d] (dtype),
 *      eoff [E+1], stok [max_rows], sw [max_rows], meta [MOE_META_N].
 * Out: h [max_rows][f] (dtype), y [max_rows][d] fp32.
 * scratch: at least moe_ffn_scratch_bytes().
 * Errors: MOE_EINVAL for d or f not positive multiples of 8 or above 2^22,
 * one expert matrix of 2 GiB or more, bad dtype, NULL/misaligned pointers,
 * small scratch, tm < 1; MOE_EUNSUPPORTED for E > MOE_MAX_EXPERTS; MOE_EHIP on
 * a failed launch.
 */
int moe_expert_ffn(const void *xs, const void *w_gate, const void *w_up, const void *w_down,
                   int dtype, int E, int d, int f, int tm, const int32_t *eoff, const int32_t *stok,
                   const float *sw, const int32_t *meta, int64_t max_rows, void *h, float *y,
                   void *scratch, size_t scratch_bytes, moe_stream_t stream);

/* Which matrices a packed weight buffer holds. */
enum moe_wkind {
    MOE_W_GATE_UP = 0, /* W_gate or W_up: [E][d][f] */
    MOE_W_DOWN = 1     /* W_down: [E][f][d] */
};

/*
 * moe_packed_weight_bytes -- host only: size of one packed matrix set (see
 * moe_pack_weights) for E experts, hidden size d, intermediate size f, dtype.
 * Errors: MOE_EINVAL for NULL bytes, E < 1, d or f not positive multiples of
 * 8, bad dtype or kind; MOE_EUNSUPPORTED for E > MOE_MAX_EXPERTS.
 */
int moe_packed_weight_bytes(int E, int d, int f, int dtype, int kind, size_t *bytes);

/*
 * moe_pack_weights -- rearrange one set of expert matrices, once (at model
 * load), into the tile layout the grouped FFN streams: for each expert,
 * column group of 4 slices, K-step and slice, one contiguous 4 KB tile per
 * 64-column stream (gate/up: one stream of 64 columns per slice; down: two)
 * holding, for each of the 64 MFMA lanes, the 4 B-operand words of that step
 * in the order the lane consumes them (16-bit types: 8 consecutive K of one
 * column; fp32: 4 consecutive columns of one K-row). Bits are copied, nothing
 * is converted; positions past d or f hold zeros. The grouped GEMMs then read
 * each workgroup's K range of a column group as one contiguous run, with
 * 16-byte loads and no transposes: a reorganisation of [P3]'s resident expert
 * weights for the MI355X memory system, not a change of the arithmetic
 * (moe_forward_packed returns the same bits as moe_forward).
 * In:  w = W_gate or W_up [E][d][f] (kind MOE_W_GATE_UP) or W_down [E][f][d]
 *      (MOE_W_DOWN) of dtype, 16-byte aligned.
 * Out: packed [moe_packed_weight_bytes], 16-byte aligned; owned by the caller.
 * Errors: as moe_packed_weight_bytes, plus MOE_EINVAL for misaligned pointers,
 * packed_bytes too small, or one matrix of 2 GiB or more; MOE_EHIP on a failed
 * launch.
 */
int moe_pack_weights(const void *w, int dtype, int E, int d, int f, int kind, void *packed,
                     size_t packed_bytes, moe_stream_t stream);

/*
 * moe_expert_ffn_packed -- moe_expert_ffn with packed expert weights
 * (pw_gate, pw_up: moe_pack_weights(..., MOE_W_GATE_UP); pw_down:
 * MOE_W_DOWN). Same arguments, results (bit for bit) and errors otherwise.
 */
int moe_expert_ffn_packed(const void *xs, const void *pw_gate, const void *pw_up,
                          const void *pw_down, int dtype, int E, int d, int f, int tm,
                          const int32_t *eoff, const int32_t *stok, const float *sw,
                          const int32_t *meta, int64_t max_rows, void *h, float *y, void *scratch,
                          size_t scratch_bytes, moe_stream_t stream);

/*
 * moe_combine -- sum each token's expert outputs in the fixed top-k order
 * ([P3] s.3: the same per-token top-k summation order gives bit-identical
 * results): out[t][c] = +0.0f, then += y[pos[t*K+k]][c] for k = 0..K-1 in fp32,
 * skipping pos < 0 (and pos >= max_rows). One correct fp32 result exists for
 * this order, and this call produces it.
 * In:  y [max_rows][d] fp32, pos [T*K]. Out: out [T][d] fp32.
 * Errors: MOE_EINVAL for d % 8 != 0, T/K < 1, NULL/misaligned pointers;
 * MOE_EHIP on a failed launch.
 */
int moe_combine(const float *y, int64_t max_rows, const int32_t *pos, int T, int K, int d,
                float *out, moe_stream_t stream);

/*
 * moe_forward_workspace -- host only: bytes of the workspace moe_forward
 * carves its intermediates from (plan arrays, xs, h, y, scratch).
 */
int moe_forward_workspace(int T, int K, int E, int d, int f, int tm, int dtype, size_t *bytes);

/*
 * moe_forward -- one routed MoE layer: the results of moe_plan, moe_gather,
 * moe_expert_ffn and moe_combine in sequence on one stream, intermediates in
 * `workspace`. Fewer launches than calling them one by one: for T*K <= 32768
 * the plan is one kernel that also writes the FFN's work list; for T*K <= 64
 * with tm dividing 64 (and x below 2 GiB) that plan runs inside the gate/up
 * kernel, whose workgroups find their work items from the ids themselves (the
 * workspace's plan arrays get the same values); and when x is smaller than 2
 * GiB the gate/up kernel reads its rows from x through stok (the gather is
 * fused; the workspace's xs rows are then left unwritten).
 * For fp16 and bf16 layers the expert outputs y are kept in a compact format,
 * half the bytes of fp32 rows: each row is cut into blocks of 128 columns, a
 * block holds binary16 values s and one exponent e (int8) and stands for
 * s * 2^-e exactly; e puts the block's largest magnitude in [2^14, 2^15) (e =
 * 15 - k for a maximum m * 2^k, m in [1/2, 1), clamped to [-112, 100]; 0 for
 * an all-zero or infinite block) and s = y * 2^e rounded to binary16 (nearest
 * even), a relative error of at most 2^-12 per value near the block maximum.
 * The combine decodes each value exactly and sums in the same fixed order, so
 * the result is deterministic; it differs in rounding from the four calls
 * (whose y is fp32) but not from the same call again. In the workspace
 * (moe_forward_layout) the y region then holds the binary16 rows [max_rows][d]
 * followed by their exponents, block-major: [ceil(d/128)][max_rows]. fp32
 * layers keep fp32 y and equal the four calls bit for bit.
 * In:  x [T][d] (dtype), ids [T*K], w [T*K], expert weights as above.
 * Out: out [T][d] fp32.
 * Errors: the union of the four calls' errors.
 */
int moe_forward(const void *x, const int32_t *ids, const float *w, const void *w_gate,
                const void *w_up, const void *w_down, int dtype, int T, int K, int E, int d, int f,
                int tm, void *workspace, size_t ws_bytes, float *out, moe_stream_t stream);

/*
 * moe_forward_packed -- moe_forward with packed expert weights (see
 * moe_pack_weights); same workspace, results (bit for bit) and errors.
 */
int moe_forward_packed(const void *x, const int32_t *ids, const float *w, const void *pw_gate,
                       const void *pw_up, const void *pw_down, int dtype, int T, int K, int E,
                       int d, int f, int tm, void *workspace, size_t ws_bytes, float *out,
                       moe_stream_t stream);

/*
 * Expert weights in host memory, for layers whose experts do not all fit in
 * device memory ("#372 Prompt path: an MMQ group's experts gathered in one
 * launch, after one wait, released by one event", description: the routed
 * experts are streamed into a ring of device slots, ring entries the routing
 * does not use are skipped; "Add --moe-mode sweep-prefill: streamed expert
 * supply for CPU mul_mat_id", Mechanism: the used experts in ascending order).
 * The weights stay in host memory that is pinned and mapped for the device
 * (hipHostMalloc; torch pin_memory): w_gate_host, w_up_host [E][d][f] and
 * w_down_host [E][f][d], or the packed arrays of moe_pack_weights (packed = 1).
 * A device cache holds `slots` experts (each slot one expert's three
 * matrices) and the state of a ring over the slots.
 *
 * moe_host_cache_bytes -- host only: the cache's device bytes for `slots`
 * slots (0: the fewest that serve a call of T tokens, min(E, T*K)).
 * Errors: MOE_EINVAL / MOE_EUNSUPPORTED as moe_forward_workspace; MOE_EINVAL
 * also for packed other than 0 or 1 and for slots (other than 0) below
 * min(E, T*K) or above E.
 *
 * moe_host_cache_init -- mark every slot of a cache empty (one launch on
 * `stream`). Needed before a cache's first use, and again after the host
 * weights it has copied change. Errors: MOE_EINVAL for a small or unaligned
 * cache or bad sizes (1 <= slots <= E).
 *
 * moe_forward_host_weights -- moe_forward (packed = 0) or moe_forward_packed
 * (packed = 1) with the weights in host memory. After the plan, one launch
 * keeps the slot of every routed expert the cache already holds, gives every
 * other routed expert (ascending) the next slot of the ring that holds no
 * expert this call routes to (evicting the expert it held), and renumbers the
 * work list to slots; a second launch copies the newly placed experts'
 * matrices from host memory, the GPU reading it over the host link. The
 * grouped FFN then reads the cache. The call enqueues on the stream like
 * moe_forward and never waits for the GPU. Calls that share a cache must be
 * ordered (one stream).
 * In:  the host weights as above; slots as at moe_host_cache_init (>=
 *      min(E, T*K)); the rest as moe_forward.
 * cache: device, 256-byte aligned, >= moe_host_cache_bytes for `slots`, made
 *      by moe_host_cache_init with the same sizes; updated by the call.
 * Out: out [T][d] fp32, the same bits as moe_forward / moe_forward_packed on
 *      device copies of the same weights, whatever the cache held.
 * Errors: those of moe_forward; MOE_EINVAL also for a small or unaligned
 *      cache, slots below min(E, T*K), and weight pointers that are not
 *      pinned, device-mapped host memory (pageable memory is refused before
 *      any launch).
 */
int moe_host_cache_bytes(int T, int K, int E, int d, int f, int dtype, int packed, int slots,
                         size_t *bytes);
int moe_host_cache_init(void *cache, size_t cache_bytes, int E, int d, int f, int dtype,
                        int packed, int slots, moe_stream_t stream);
int moe_forward_host_weights(const void *x, const int32_t *ids, const float *w,
                             const void *w_gate_host, const void *w_up_host,
                             const void *w_down_host, int packed, int dtype, int T, int K, int E,
                             int d, int f, int tm, int slots, void *cache, size_t cache_bytes,
                             void *workspace, size_t ws_bytes, float *out, moe_stream_t stream);

/* Byte offsets of moe_forward's intermediates inside the workspace (host only),
 * so that a caller can inspect them after a call. */
typedef struct {
    size_t cnt, eoff, tiles, stok, sw, pos, boff, meta, plan_scratch, xs, h, y, ffn_scratch, total;
} moe_forward_layout_t;
int moe_forward_layout(int T, int K, int E, int d, int f, int tm, int dtype,
                       moe_forward_layout_t *out);

/* ---- per-kernel timing (HIP events recorded around each kernel) ---- */

enum moe_stage {
    MOE_STAGE_HIST = 0,
    MOE_STAGE_SCAN,
    MOE_STAGE_PLACE,
    MOE_STAGE_GATHER,
    MOE_STAGE_WORKLIST,
    MOE_STAGE_GATEUP,
    MOE_STAGE_DOWN,
    MOE_STAGE_COMBINE,
    MOE_STAGE_N
};

typedef struct moe_timer moe_timer_t;

/* Create a timer that can hold `capacity` recorded calls (host object; its
 * HIP events are created on the current device). Only the stages whose bit
 * (1 << stage) is set in stage_mask are timed, so that a caller timing one
 * kernel adds no event records around the others. */
int moe_timer_create(moe_timer_t **out, int capacity, unsigned stage_mask);
int moe_timer_destroy(moe_timer_t *timer);
/* Wait for the recorded events, add each stage's elapsed milliseconds into
 * total_ms[MOE_STAGE_N] and its launch count into launches[MOE_STAGE_N], then
 * forget the recorded calls. */
int moe_timer_read(moe_timer_t *timer, double *total_ms, int64_t *launches);

/* moe_forward with an event pair recorded around every kernel into `timer`
 * (NULL: identical to moe_forward). MOE_EINVAL when the timer is full. */
int moe_forward_timed(const void *x, const int32_t *ids, const float *w, const void *w_gate,
                      const void *w_up, const void *w_down, int dtype, int T, int K, int E, int d,
                      int f, int tm, void *workspace, size_t ws_bytes, float *out,
                      moe_stream_t stream, moe_timer_t *timer);

/* moe_forward_packed with an event pair recorded around every kernel into
 * `timer` (NULL: identical to moe_forward_packed). */
int moe_forward_packed_timed(const void *x, const int32_t *ids, const float *w,
                             const void *pw_gate, const void *pw_up, const void *pw_down,
                             int dtype, int T, int K, int E, int d, int f, int tm,
                             void *workspace, size_t ws_bytes, float *out, moe_stream_t stream,
                             moe_timer_t *timer);

/*
 * moe_forward_packed_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_forward_packed with its workspace taken from a fixed buffer
 * inside this library instead of a caller argument. The caller still passes
 * the inputs and `out`, as for moe_forward_packed; results are the same bits.
 *  - The buffer is MOE_NOALLOC_WORKSPACE_BYTES of device memory per GPU,
 *    reserved when the library's code is loaded on that GPU and held until the
 *    process ends. It covers decode-sized batches (e.g. 4 tokens, hidden 2816,
 *    128 experts, top-8, intermediate 704 needs 22.7 MiB).
 *  - A request whose moe_forward_workspace() exceeds the buffer returns
 *    MOE_ENOSPACE before any HIP call.
 *  - The first call on each device looks up that device's buffer address
 *    (hipGetSymbolAddress); make that first call outside graph capture. Later
 *    calls allocate nothing, clear nothing with memset and never wait on the
 *    host, so they can be captured.
 *  - `stream` must belong to the current device (MOE_EINVAL otherwise); NULL
 *    is the current device's default stream.
 *  - All calls on one GPU share that GPU's buffer, which keeps the last call's
 *    contents (nothing in it needs to start at zero): calls that can overlap on
 *    one GPU (different streams or threads without ordering between them) race
 *    on it and must be serialised by the caller.
 * Errors: those of moe_forward_packed, plus MOE_ENOSPACE, and
 * MOE_EUNSUPPORTED for a device ordinal of 64 or more.
 */
#define MOE_NOALLOC_WORKSPACE_BYTES (64u * 1024u * 1024u)
int moe_forward_packed_noalloc(const void *x, const int32_t *ids, const float *w,
                               const void *pw_gate, const void *pw_up, const void *pw_down,
                               int dtype, int T, int K, int E, int d, int f, int tm, float *out,
                               moe_stream_t stream);

/* Static description of a status code. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTED_H */
