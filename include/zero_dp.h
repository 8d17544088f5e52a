/*
 * zero_dp.h -- C ABI of the ZeRO-DP owned-partition step on one AMD
 * Instinct MI355X (gfx950).
 *
 * The method (ZeRO-DP, "Zero Redundancy Optimizer", data-parallel stages
 * Pos / Pos+g / Pos+g+p) partitions the model states of Psi parameters over
 * Nd data-parallel ranks.  Each rank owns a contiguous window of the flat
 * parameter buffer; per training step it
 *   1. receives and sums the Nd ranks' fp16 gradient contributions for its
 *      window (the local half of the reduce-scatter),
 *   2. unscales by the loss scale, flags inf/NaN and forms sum(g^2),
 *   3. runs mixed-precision Adam on its fp32 master / momentum / variance
 *      (16 bytes per parameter: fp16 param + fp16 grad + 12 bytes of Adam
 *      state), and
 *   4. writes its updated fp16 parameters into the flat all-gather buffer at
 *      its window's offset (the local half of the all-gather).
 * Sources: upskillscore.com "ZeRO: partitioning training state across GPUs",
 * section "How it works"; the trishampatil.com engineering dissection of ZeRO
 * (page zero-memory-optimization-training-large-models), sections "The Real
 * Problem", "ZeRO-1/2/3", "The Full Progression, in One View" and
 * "Forward/Backward Under ZeRO-3"; the
 * anthology note on ZeRO (dmarx.github.io note-103), "Assumptions" and
 * "Method".
 *
 * Conventions
 *   - Every call returns an int status: ZERO_OK (0) or a negative ZERO_E*.
 *   - "device" pointers are HIP device memory (e.g. from hipMalloc or a
 *     PyTorch CUDA/HIP tensor); "host" pointers are ordinary CPU memory.
 *   - Asynchronous calls validate their arguments on the host, enqueue work
 *     on `stream` (a hipStream_t; NULL = the legacy default stream) and
 *     return without synchronising.  Results are valid once the stream has
 *     reached them.  On a non-OK return nothing was enqueued, except for
 *     ZERO_EHIP, which reports a failed launch (see zero_last_hip_error);
 *     launches of the same call before the failed one may have been
 *     enqueued, and the step must then be treated as not taken.
 *   - The library allocates nothing and only borrows the caller's buffers for
 *     the duration of the enqueued work.  Its only mutable state is a
 *     per-device cache of launch sizes (filled once, thread-safe) and the
 *     per-thread last HIP error.
 *   - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *   - Element counts and offsets are int64_t; sizes up to 2^62 elements.
 *   - A data pointer may be NULL when its element count is 0 (empty window).
 */
#ifndef ZERO_DP_H
#define ZERO_DP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_DP_ABI_VERSION 7

/* ---- status codes --------------------------------------------------- */
#define ZERO_OK          0
#define ZERO_EINVAL     -1  /* null pointer, nd < 1, n < 0, bad stage/align, bad hyperparameter */
#define ZERO_EALIGN     -2  /* a vector operand is not 16-byte aligned, or an offset/stride is not a multiple of 8 elements */
#define ZERO_EOVERFLOW  -3  /* an int64 size or offset computation would overflow */
#define ZERO_ECAPACITY  -4  /* the caller's fragment array is too small (*n_frags holds the needed count),
                              or the library's fixed scratch is too small for the device */
#define ZERO_EALIAS     -5  /* an output buffer overlaps an input it must not overlap */
#define ZERO_EHIP       -6  /* a HIP launch or runtime call failed; see zero_last_hip_error() */

/* Message for a status code (static string, never NULL). */
const char* zero_strerror(int status);
/* hipError_t of the last ZERO_EHIP returned on the calling thread (0 if none). */
int zero_last_hip_error(void);
/* ZERO_DP_ABI_VERSION of the loaded library. */
int zero_abi_version(void);

/* ---- partition plan (host, synchronous) ------------------------------
 * The flat parameter buffer holds the tensors packed in list order; it is
 * split into Nd equal windows, window i held by rank i (trishampatil "ZeRO's
 * Core Idea"; upskillscore "How it works": the optimizer state is divided
 * among the Nd data-parallel ranks).  The pages leave padding open; this library pads the total to
 * S = align * ceil(Psi / (Nd * align)) elements per rank, so rank r owns flat
 * elements [r*S, (r+1)*S) and all padding sits at the tail of rank Nd-1.
 */
typedef struct zero_plan {
    int64_t psi;      /* sum of tensor sizes (real parameters) */
    int32_t nd;       /* data-parallel degree */
    int32_t align;    /* alignment of S in elements */
    int64_t part;     /* S: elements owned by each rank */
    int64_t padded;   /* Nd * S */
    int64_t pad;      /* padded - psi, 0 <= pad < Nd * align */
} zero_plan;

/* One piece of a tensor that lies inside one rank's window. */
typedef struct zero_frag {
    int32_t tensor;       /* index into the tensor list */
    int32_t rank;         /* owning rank */
    int64_t tensor_off;   /* first element of the piece inside the tensor */
    int64_t flat_off;     /* first element inside the flat buffer */
    int64_t local_off;    /* first element inside the owner's window (flat_off - rank*S) */
    int64_t len;          /* elements in the piece, > 0 */
} zero_frag;

/*
 * numels:    host array of n_tensors sizes (>= 0); may be NULL if n_tensors == 0.
 * nd:        >= 1.   align_elems: >= 8 and a multiple of 8 (keeps every
 *            window 16-byte aligned for fp16 and fp32 data).
 * plan:      host, written on success.
 * frags:     host array of frag_cap entries, written in tensor order and,
 *            within a tensor, in rank order.  May be NULL if frag_cap == 0.
 * n_frags:   host, receives the number of fragments.  If it exceeds
 *            frag_cap the call returns ZERO_ECAPACITY after filling *plan and
 *            *n_frags (call again with a larger array).
 * Errors: ZERO_EINVAL, ZERO_EOVERFLOW, ZERO_ECAPACITY.
 */
int zero_plan_partitions(const int64_t* numels, int32_t n_tensors, int32_t nd,
                         int32_t align_elems, zero_plan* plan, zero_frag* frags,
                         int64_t frag_cap, int64_t* n_frags);

/* ---- memory / communication model (host, synchronous, pure) ----------
 * Per-device model-state bytes of mixed-precision Adam, K bytes of optimizer
 * state per parameter (K = 12: fp32 copy, momentum, variance):
 *   stage 0 (DP)        2Psi + 2Psi + K Psi
 *   stage 1 (Pos)       2Psi + 2Psi + K Psi/Nd
 *   stage 2 (Pos+g)     2Psi + (2+K) Psi/Nd
 *   stage 3 (Pos+g+p)   (2+2+K) Psi/Nd
 * and the per-step communication volume in elements: 2Psi for stages 0-2
 * (reduce-scatter Psi + all-gather Psi), 3Psi for stage 3 (two parameter
 * all-gathers + one reduce-scatter).  trishampatil "The Real Problem",
 * "ZeRO-1", "ZeRO-2", "ZeRO-3", "The Full Progression, in One View";
 * upskillscore "How it works".
 */
typedef struct zero_mem_report {
    double params_bytes;     /* fp16 parameters held per device */
    double grads_bytes;      /* fp16 gradients held per device */
    double optim_bytes;      /* optimizer state held per device */
    double total_bytes;
    double comm_elems;       /* nominal per-rank volume: 2Psi or 3Psi */
    double comm_elems_ring;  /* comm_elems * (Nd-1)/Nd, what a ring moves per rank */
    double reduction_vs_dp;  /* (4+K)Psi / total_bytes */
} zero_mem_report;

/* psi >= 0 and finite; nd >= 1; stage in 0..3; k >= 0.  Errors: ZERO_EINVAL. */
int zero_memory_model(double psi, int32_t nd, int32_t stage, int32_t k, zero_mem_report* out);

/* ---- gradient source --------------------------------------------------
 * The Nd ranks' fp16 contributions to the owned window, as the
 * reduce-scatter delivers them: slice k (rank k) starts at
 * base + k*slice_stride, and the owned window is elements
 * [elem_off, elem_off + n) of every slice.  (Measured at Nd = 400: a
 * slice_stride that is an exact power of two reads 2-3% slower than one
 * padded off it by a few thousand elements.)
 */
typedef struct zero_grad_src {
    const uint16_t* base;   /* device, fp16 bit patterns, 16-byte aligned */
    int64_t slice_stride;   /* elements between slices; multiple of 8 (any value if nd == 1) */
    int64_t elem_off;       /* window offset inside each slice; multiple of 8 */
    int64_t n;              /* window length S >= 0 (any value; a tail of n % 8 is handled) */
    int32_t nd;             /* number of slices, 1 <= nd < 8192 (the float64 sum is exact below 2^13 terms) */
    int32_t reserved;       /* must be 0 */
    double loss_scale;      /* L > 0, L and 1/L finite; g = s * (1/L) */
} zero_grad_src;

/* ---- workspace ----------------------------------------------------------
 * Device scratch for per-workgroup partial results, a completion counter
 * and the element count of a bucketed or split step.
 * Allocate zero_workspace_bytes() bytes of device memory (16-byte aligned),
 * zero it ONCE before first use, and never share one workspace between calls
 * that may run concurrently (different streams).  Every call leaves it ready
 * for the next call.
 */
int64_t zero_workspace_bytes(void);

/* ---- reduce (decomposed path) ---------------------------------------
 * s_j = G_0[j] + ... + G_{Nd-1}[j] (exact, float64), g_j = s_j * (1/L),
 * *overflow = 1 if any fp32(g_j) is inf/NaN (so any inf/NaN s_j) else 0, *sumsq = sum_j g_j^2 (float64,
 * deterministic order).  Pos+g: a gradient partition is summed on its
 * owning rank alone (upskillscore "How it works").
 *   grad_out: device float[n], 16-byte aligned, receives fp32(g); may be NULL.
 *   overflow: device int32 (4-byte aligned), required.  sumsq: device double
 *   (8-byte aligned), required.  workspace: see above.  No output may
 *   overlap the slices, another output or the workspace.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
int zero_reduce_owned(const zero_grad_src* src, float* grad_out, int32_t* overflow,
                      double* sumsq, void* workspace, void* stream);

/* ---- Adam state of one owned shard -----------------------------------
 * fp32 master weights, momentum and variance (12 bytes per parameter:
 * anthology note "Assumptions"; trishampatil "The Real Problem"), held twice
 * (ping-pong) so that a step found to overflow after its single pass can be
 * dropped: each step reads set ctl->cur and writes set 1 - ctl->cur, and the
 * step's commit (on the device, after the pass) sets cur ^= 1 and t += 1
 * only when no element overflowed.  The control block lives in device memory; initialise it with
 * zero_ctl_init() on the host and copy it to the device.
 */
typedef struct zero_step_ctl {
    int32_t cur;         /* index (0/1) of the buffers holding the committed state */
    int32_t t;           /* committed optimizer steps */
    int32_t overflow;    /* 0: the last step was committed; 1: skipped (inf/NaN gradient);
                            2: skipped (a bucketed step's buckets did not cover the window) */
    int32_t good_steps;  /* dynamic loss scaling: consecutive clean steps since the last change */
    double beta1_pow;    /* beta1^t, as t successive products from 1.0 */
    double beta2_pow;    /* beta2^t */
    double sumsq;        /* sum g^2 of the last step (meaningful when overflow == 0) */
    int64_t skipped;     /* number of skipped steps */
    double loss_scale;   /* dynamic loss scaling: the scale the next step's gradients carry */
    double clip_coef;    /* coefficient the last clipped step applied (1 = not clipped) */
} zero_step_ctl;

/* Fills *ctl (host) with t = 0, cur = 0, powers 1.0, loss_scale as given
 * (used only with dynamic loss scaling), clip_coef 1. */
void zero_ctl_init(zero_step_ctl* ctl, double loss_scale);

typedef struct zero_adam_state {
    float* master[2];      /* device float[n] each, 16-byte aligned */
    float* exp_avg[2];     /* momentum m */
    float* exp_avg_sq[2];  /* variance v */
    zero_step_ctl* ctl;    /* device */
} zero_adam_state;

/* Hyperparameters; beta1/beta2 must stay constant over the life of a ctl.
 * weight_decay is decoupled (AdamW): p <- p*(1 - lr*wd) - ... ; 0 = Adam.
 *
 * Dynamic loss scaling (scale_interval > 0; the practice of the
 * mixed-precision training the anthology note's "Connections" cites): the
 * gradients carry ctl->loss_scale (src->loss_scale is then ignored); after
 * each step the commit kernel multiplies the scale by scale_backoff if the
 * step overflowed (and resets good_steps), else counts the clean step and
 * multiplies the scale by scale_growth after scale_interval of them (and
 * resets good_steps), keeping the old scale if the grown one is not finite
 * (as torch's amp scaler does).  A scale backed off to 0 (or to a value
 * whose reciprocal overflows) makes every g non-finite, so every later step
 * is skipped and the state is never written with inf/NaN.
 *
 * Global-norm clipping (max_grad_norm > 0) is applied only by
 * zero_adam_step_clipped, which needs the norm before the update. */
typedef struct zero_adam_hp {
    double lr;
    double beta1;          /* in [0, 1) */
    double beta2;          /* in [0, 1) */
    double eps;            /* > 0 */
    double weight_decay;   /* >= 0 */
    double max_grad_norm;  /* > 0 for zero_adam_step_clipped; must be 0 for zero_adam_step */
    double scale_growth;   /* > 0 (e.g. 2), used when scale_interval > 0 */
    double scale_backoff;  /* > 0 (e.g. 0.5), used when scale_interval > 0 */
    int32_t scale_interval;/* 0: static scale src->loss_scale; > 0: dynamic scaling */
    int32_t reserved;      /* must be 0 */
} zero_adam_hp;

/* ---- fused step (hot path) -------------------------------------------
 * One pass over the owned window: exact Nd-way sum -> unscale -> overflow
 * flag and sum g^2 -> Adam/AdamW in float64 (m' = b1 m + (1-b1) g;
 * v' = b2 v + (1-b2) g^2; d = sqrt(v') / sqrt(1-b2^t) + eps;
 * p' = p (1 - lr wd) - lr/(1-b1^t) * m'/d; state stored as fp32, RNE) ->
 * allgather[allgather_off + j] = fp16_RNE(fp32 p'_j).  Two launches: the
 * fused pass (each workgroup leaves its partial sum of g^2 and flag in the
 * workspace) and a small commit kernel that sums them in a fixed order and
 * commits the step in ctl (see zero_adam_state), or skips it and re-emits
 * the all-gather window from the committed master.  A long window takes its
 * fused pass in consecutive launches (measured faster than one long
 * launch): of about 2^24 elements when it is longer than 2^25 and Nd < 32,
 * of about 2^23 when it is longer than 2^24 and 32 <= Nd < 256, of about
 * 2^22 when it is longer than 2^23 and Nd >= 256.  Their partials
 * accumulate in the workspace; the results are the same element for
 * element, and the sum of g^2 differs only in its rounding order.  A rank steps its own
 * partition alone and the new parameters then reach every rank by
 * all-gather (upskillscore "How it works"; trishampatil "Forward/Backward
 * Under ZeRO-3": reduce-scatter, update the shard, all-gather).
 *   src: gradient source, src->n = window length.
 *   st:  ping-pong state; neither set may overlap the other, the slices or
 *        the all-gather window.  st->ctl is 8-byte aligned, and neither it
 *        nor the workspace may overlap any of these.
 *   allgather: device uint16 buffer; the window [allgather_off,
 *        allgather_off + n) is written (16-byte aligned start).  NULL skips
 *        the emit.
 * On an overflowing step the state is untouched (not committed) and the
 * all-gather window holds the committed parameters again once the call's
 * work has run; no host synchronisation or restore call is needed.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
int zero_adam_step(const zero_grad_src* src, const zero_adam_state* st,
                   const zero_adam_hp* hp, uint16_t* allgather, int64_t allgather_off,
                   void* workspace, void* stream);
/* (hp->max_grad_norm must be 0 here; dynamic loss scaling is applied when
 * hp->scale_interval > 0.) */

/* ---- fused step without a workspace argument ---------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The step
 * of zero_adam_step, with its workspace replaced by a device array the
 * library holds, zero_workspace_bytes() bytes (98,560) per GPU, kept until
 * the process ends; the call itself allocates nothing.  The first call on
 * a device looks up that device's copy (hipGetSymbolAddress).  Every call
 * on one GPU shares that GPU's copy and leaves the last call's partials in
 * it: calls that may overlap on one GPU (several streams, or host threads
 * without ordering) race and must not be made; calls in one stream's
 * order are fine.  Nothing needs clearing between calls (each step's
 * first launch writes every slot its commit reads).  The array holds the
 * partials of up to 8192 workgroups, more than a step launches on any
 * device (one per CU: 256 on MI355X); a device that would need more gets
 * ZERO_ECAPACITY.  The window length is not limited by it.  Arguments,
 * results and the other errors are those of zero_adam_step.
 */
int zero_adam_step_noalloc(const zero_grad_src* src, const zero_adam_state* st,
                           const zero_adam_hp* hp, uint16_t* allgather, int64_t allgather_off,
                           void* stream);

/* ---- clipped step (two passes) ----------------------------------------
 * Global-norm clipping needs the norm of the whole gradient before any
 * element is updated, so this path materialises the reduced gradient:
 *   pass 1: g32_j = fp32(s_j * (1/L)) into grad_buf, flag, sumsq = sum g32^2
 *           (float64, deterministic order);
 *   pass 2: if the flag is set, the step is skipped (state and all-gather
 *           window untouched, no restore needed); otherwise
 *           coef = min(1, max_grad_norm / (sqrt(sumsq) + 1e-6)) and the
 *           update of zero_adam_step runs on g = g32 * coef (float64);
 *   then a one-workgroup commit; ctl->clip_coef records coef.
 * A long window takes each pass in consecutive launches: the first pass
 * as zero_adam_step's fused pass, the second in launches of about 2^24
 * elements when the window is longer than 2^25.
 * L is src->loss_scale or, with dynamic scaling, ctl->loss_scale.
 * Traffic (2*Nd + 4) + 30 bytes per element instead of 2*Nd + 26.
 *   grad_buf: device float[n], 16-byte aligned, must not overlap any other
 *   operand.  Other arguments as for zero_adam_step; hp->max_grad_norm > 0.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
int zero_adam_step_clipped(const zero_grad_src* src, const zero_adam_state* st,
                           const zero_adam_hp* hp, float* grad_buf, uint16_t* allgather,
                           int64_t allgather_off, void* workspace, void* stream);

/* ---- bucketed step (constant-size fused buffers) ---------------------
 * The reduce-scatter delivers the owned gradient partition bucket by bucket
 * (dmarx anthology note, "Method": constant-size fused buffers, CB); this
 * steps one bucket as soon as it has arrived, so the step overlaps the rest
 * of the ingest.  The buckets of one step partition the window
 * [0, window_n): bucket b covers window elements [win_off, win_off + n)
 * and its gradients come from src (n = src->n; typically the same
 * constant-size receive buffer [Nd, B] for every bucket).  Each bucket runs
 * the fused update of zero_adam_step on its elements, reading state
 * buffer ctl->cur and writing the other one plus
 * allgather[allgather_off + win_off + j]; nothing is committed until the
 * last bucket.  Each workgroup's sum of g^2 and flag accumulate in its
 * workspace slot across the step's buckets (all bucket launches run on the
 * same grid), and the elements covered in a counter, in stream order
 * (deterministic for a given bucket order).  The call flagged
 * ZERO_BUCKET_LAST also launches the commit: the whole step is committed as
 * zero_adam_step would, or skipped if any bucket overflowed
 * (ctl->overflow = 1, the loss scale backs off) or if the buckets covered
 * fewer or more than window_n elements (ctl->overflow = 2, the loss scale
 * is left alone); a skip re-emits the whole all-gather window.
 *   st: the window's state, as for zero_adam_step (n = window_n).
 *   allgather, allgather_off: the whole window's all-gather range (its
 *   start 16-byte aligned); bucket b writes from allgather_off + win_off.
 *   win_off: multiple of 8.  phase: ZERO_BUCKET_FIRST on the step's first
 *   bucket, ZERO_BUCKET_LAST on its last (both for a single bucket), 0 in
 *   between.  Every bucket of a step runs on one stream with one
 *   workspace, and no other call may use that workspace between the step's
 *   first and last bucket; the buckets may come in any order but must not
 *   overlap (an overlap that keeps the count equal to window_n is not
 *   detected).
 *   hp->max_grad_norm must be 0: clipping needs the whole norm before any
 *   bucket is updated.
 * Errors: ZERO_EINVAL (also win_off + n > window_n), ZERO_EALIGN,
 * ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
#define ZERO_BUCKET_FIRST 1
#define ZERO_BUCKET_LAST  2
int zero_adam_step_bucket(const zero_grad_src* src, const zero_adam_state* st,
                          const zero_adam_hp* hp, int64_t win_off, int64_t window_n,
                          uint16_t* allgather, int64_t allgather_off, int32_t phase,
                          void* workspace, void* stream);

/* ---- several arrived buckets in one call ------------------------------
 * The same step as a sequence of zero_adam_step_bucket calls, one per
 * bucket in list order, for the buckets that have arrived together: their
 * elements are stepped in as few launches as fit (consecutive buckets
 * share a launch up to 16 runs and one launch length, about 2^24 elements
 * below Nd = 32; a bucket longer than two launch lengths is cut as a long
 * window is).  A bucket's fixed cost is then paid per launch rather than
 * per bucket: the launch, the ramp of its first loads and the drain of its
 * last stores (for Nd <= 16 a launch walks the elements of all its buckets
 * as one sequence, so its loads run ahead across bucket edges).  Per element the results are those of the one-bucket calls
 * bit for bit; the sum of g^2 differs only in its rounding order.  phase
 * applies to the call: ZERO_BUCKET_FIRST if its first bucket is the step's
 * first, ZERO_BUCKET_LAST to commit after its last bucket.  Calls and
 * one-bucket calls may be mixed within a step (all on the same stream and
 * workspace).  A bucket b reads b->src (its receive buffer; nd and
 * loss_scale equal across the call) for window elements
 * [b->win_off, b->win_off + b->src.n); the buckets of a call may not cover
 * the same element twice (ZERO_EINVAL).  Other arguments and rules are
 * those of zero_adam_step_bucket (window_n, allgather, allgather_off the
 * whole window's).  1 <= nb <= ZERO_MAX_BUCKETS_PER_CALL.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
typedef struct zero_bucket {
    zero_grad_src src;   /* the bucket's slices (src.n elements of each) */
    int64_t win_off;     /* window offset of its first element; multiple of 8 */
} zero_bucket;
#define ZERO_MAX_BUCKETS_PER_CALL 1024
int zero_adam_step_buckets(const zero_bucket* buckets, int32_t nb, const zero_adam_state* st,
                           const zero_adam_hp* hp, int64_t window_n, uint16_t* allgather,
                           int64_t allgather_off, int32_t phase, void* workspace, void* stream);

/* Re-emits allgather[off + j] = fp16_RNE(master[ctl->cur][j]) for j < n when
 * ctl->overflow != 0 (the step was skipped), and does nothing otherwise; the
 * decision is taken on the device, so no host synchronisation is needed.
 * The steps restore their window themselves; this call is for a window
 * that must be re-derived from the committed master at another time (for
 * example a second copy of the window).
 * The window must not overlap either master or the control block.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP. */
int zero_restore_skipped(const zero_adam_state* st, int64_t n, uint16_t* allgather,
                         int64_t allgather_off, void* stream);

/* ---- Pos+g+p on-demand parameter gather -------------------------------
 * With the parameters partitioned too (Pos+g+p), rank r keeps only its
 * fp16 window of the flat parameter buffer, and a layer's parameters are
 * gathered when the computation reaches the layer, used, then released
 * (trishampatil dissection, sections "ZeRO-3" and "Forward/Backward Under
 * ZeRO-3"; the two gathers per step are the extra Psi of the 3Psi volume).
 * This copies flat elements [lo, hi) from their owners' windows into dst:
 *   dst[i] = windows[f / part][f % part] with f = lo + i, for i < hi - lo.
 * A layer is the flat range of its tensors (the fragments
 * zero_plan_partitions reports give the offsets).  Release is the caller
 * reusing dst (a constant-size layer buffer) for the next layer.
 *   windows: host array of nd device pointers, each to `part` fp16
 *     elements (2-byte aligned); only the windows that [lo, hi) touches
 *     are read, the others may be NULL.
 *   part: S, elements per window (zero_plan.part).  0 <= lo <= hi <= nd*part.
 *   dst: device, hi - lo elements, 2-byte aligned, overlapping no window
 *     piece it reads.  A piece whose source and dst addresses agree modulo
 *     16 bytes moves 16-byte vectors (always the case for windows and dst
 *     that are 16-byte aligned and lo a multiple of 8); others move
 *     element-wise.
 * One launch for every 16 windows touched (one for any layer that spans
 * at most 16 windows), in stream order.  Errors: ZERO_EINVAL,
 * ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP (nothing is launched
 * unless every piece is valid).
 */
int zero_gather_params(const uint16_t* const* windows, int32_t nd, int64_t part,
                       int64_t lo, int64_t hi, uint16_t* dst, void* stream);

/* Several layers' gathers in one call: range q is flat elements
 * [ranges[2q], ranges[2q+1]) into dsts[q] (host array of nranges device
 * pointers), as zero_gather_params would copy it.  The ranges' window
 * pieces share launches, up to 16 pieces per launch, so gathering a few
 * short layers at once (the current layer with the next ones, ahead of
 * use) pays one launch's fixed cost instead of one per layer.  No
 * destination may overlap another or a window piece any range reads.  An
 * empty range copies nothing.  nranges >= 0.  Errors as zero_gather_params.
 */
int zero_gather_layers(const uint16_t* const* windows, int32_t nd, int64_t part, const int64_t* ranges,
                       int32_t nranges, uint16_t* const* dsts, void* stream);

/* ---- emit (all-gather half) ------------------------------------------
 * allgather[allgather_off + j] = fp16_RNE(master[j]) for j < n (IEEE
 * round-to-nearest-even, overflow to inf).  Initial fill of the all-gather
 * buffer from the fp32 master (upskillscore "How it works").
 *   master: device float[n], 16-byte aligned.  allgather: device, window
 *   start 16-byte aligned.  Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW,
 *   ZERO_EHIP.
 */
int zero_emit_fp16(const float* master, int64_t n, uint16_t* allgather,
                   int64_t allgather_off, void* stream);

/* ---- bandwidth calibration (for benchmarks; not part of the step) ------
 * What HBM attains on the running GPU, beside the step: STREAM's triad
 * a[i] = b[i] + q*c[i] (fp32; 8 bytes read and 4 written per element), and
 * a kernel that moves exactly the fused step's streams with no arithmetic
 * (per element: the Nd fp16 slice reads of src, reads of in[0..2] (fp32),
 * writes of out[0..2] (fp32) and out16 (fp16); 2*Nd + 26 bytes) in the
 * fused step's launch shape, visit order and launch pieces.  It writes
 * out[0] = in[0], out[1] = in[1], out[2] = in[2] with the XOR of the
 * element's slices folded into its bits, and out16 = the top 16 bits of
 * in[0] (values with no meaning: only the traffic matters).
 *   triad: a, b, c device float[n], 16-byte aligned; a overlaps neither b
 *   nor c.  mix: src as for the step (src->loss_scale is not used but must
 *   be valid); in, out: host arrays of 3 device pointers to n floats each,
 *   16-byte aligned; out16 device uint16[n], 16-byte aligned; no output
 *   overlaps another output or any input.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
int zero_calib_triad(float* a, const float* b, const float* c, float q, int64_t n, void* stream);
int zero_calib_stream_mix(const zero_grad_src* src, const float* const* in, float* const* out,
                          uint16_t* out16, void* stream);

/* The fused step's slice reads alone: the Nd fp16 slices of src's window
 * (2*Nd bytes per element), read in the fused step's launch shape, visit
 * order and launch pieces, with no state streams and no stores beside
 * them.  The words read are folded with XOR and XORed into *sink (one
 * atomic per workgroup and launch): bits 0-15 of the folded word are the
 * XOR of the fp16 bit patterns of every slice at the window's even
 * elements (counted from the window's first element), bits 16-31 those at
 * its odd elements.  Clear *sink first to read that value; it has no other
 * meaning.  The rate is what the step's slice streams attain on the GPU.
 *   src as for the step (src->loss_scale is not used but must be valid);
 *   sink: device uint32, 4-byte aligned, outside the slices' span.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EOVERFLOW, ZERO_EALIAS, ZERO_EHIP.
 */
int zero_calib_slice_read(const zero_grad_src* src, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_DP_H */
