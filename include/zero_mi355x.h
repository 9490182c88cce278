/*
 * zero_mi355x.h -- C ABI of the ZeRO partitioned mixed-precision Adam step on
 * one data-parallel rank's flat shard, for AMD Instinct MI355X (gfx950).
 *
 * The model state the pages fix (ZeRO paper card, section "Bottleneck"):
 * fp16 parameters and fp16 gradients plus fp32 master parameters, fp32
 * momentum and fp32 variance -- 16 bytes per parameter.  ZeRO partitions that
 * state across the Nd data-parallel ranks instead of replicating it (paper
 * card, "Method": stage 1 optimizer state, stage 2 gradients, stage 3
 * parameters).  One rank therefore steps only its own contiguous slice of n
 * parameters: this library is that step.
 *
 * The step is three calls, all asynchronous on one HIP stream, with no host
 * synchronisation between them:
 *   1. zero_flatten_bucket      pack per-layer fp16 gradient tensors into the
 *                               rank's contiguous gradient partition
 *                               (contiguous, defragmented buffers: paper card,
 *                               "Method", ZeRO-R paragraph);
 *   2. zero_shard_norm_overflow exact squared L2 norm + inf/NaN flag of that
 *                               partition, then the step decision (dynamic
 *                               loss scale, skip, clip factor, bias
 *                               corrections) kept in device memory;
 *   3. zero_shard_adam_step     one fused pass: unscale + clip + Adam with
 *                               bias correction and decoupled weight decay,
 *                               fp32 master/momentum/variance update and the
 *                               fp16 parameter copy (28 bytes per parameter).
 * zero_state_bytes gives the per-rank model-state bytes for each ZeRO stage.
 *
 * Two further forms of the same step:
 *   - fused: zero_flatten_norm_bucket computes the exact-norm partials while
 *     it flattens and zero_shard_decide folds them, so the norm needs no
 *     second pass over the partition;
 *   - gradient accumulation (the DeepSpeed article leaves gradient
 *     accumulation to the library): micro-batch fp16 gradients are added
 *     into an fp32 partition (zero_flatten_bucket with ZERO_F32, or the
 *     fused zero_flatten_norm_bucket_f32 for the last micro-batch), and the
 *     *_f32 reduction and update read that fp32 gradient (30 bytes per
 *     parameter in the update);
 *   - 1-bit Adam (DeepSpeed article): zero_onebit_step runs ordinary steps
 *     for a warm-up, then compresses the momentum to one bit per element
 *     with error feedback and updates with the frozen variance;
 *   - host step (ZeRO-Offload, in the DeepSpeed article: ZeRO-2 plus CPU
 *     memory): the fp32 master parameters, momentum and variance live in host
 *     memory and the CPU steps them (zero_host_*, zero_offload_step), with
 *     the fp16 gradient partition copied down and the fp16 parameters copied
 *     back up.
 *
 * Conventions for every entry point:
 *   - pointers named dev_* or documented as device memory are HIP device
 *     pointers; everything else is host memory;
 *   - the caller owns and allocates every buffer; the library allocates
 *     nothing and keeps no pointer to a caller's buffer after a call
 *     returns.  Two exceptions, both owned by the library: a host context
 *     (zero_host_create: its worker threads and, after zero_offload_step,
 *     HIP events), and the fixed device array of
 *     zero_shard_norm_overflow_noalloc (4 KiB per GPU, held until the
 *     process ends);
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     device work is enqueued there and the call returns without waiting;
 *   - return value: ZERO_OK (0) or a negative ZERO_E* code; argument errors
 *     are detected on the host before any device work is enqueued; a fault
 *     inside a kernel surfaces at the caller's next synchronisation;
 *   - calls on different streams with disjoint buffers may run concurrently;
 *     two calls that share a zero_step_state_t must be ordered on one stream.
 */
#ifndef ZERO_MI355X_H
#define ZERO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------- */
#define ZERO_OK       0
#define ZERO_EINVAL  (-1)   /* null pointer, bad dtype/stage/hyperparameter */
#define ZERO_EALIGN  (-2)   /* a buffer is not aligned as required */
#define ZERO_ERANGE  (-3)   /* a size or segment is out of the allowed range */
#define ZERO_EHIP    (-4)   /* the HIP runtime refused a launch or a copy */
#define ZERO_ENOTSUP (-5)   /* the host CPU lacks an instruction set the host step needs */
#define ZERO_ENOMEM  (-6)   /* out of host memory */

/* Human-readable text for a status code (static storage; never NULL).
 * For ZERO_EHIP the text of the last HIP error seen by this thread. */
const char* zero_status_string(int code);

/* ---- element types of a flatten destination ------------------------- */
#define ZERO_F16 1          /* IEEE binary16, stored as uint16_t bit patterns */
#define ZERO_F32 2          /* IEEE binary32 */

/* One piece of a per-layer gradient tensor that lands in the partition:
 * count elements from src[src_off ...] go to dst[dst_off ...].
 * src is a DEVICE pointer to binary16 data; offsets and count are elements. */
typedef struct {
    const uint16_t* src;
    uint64_t src_off;
    uint64_t dst_off;
    uint64_t count;
} zero_segment_t;

/* Hyperparameters of one step (host struct, passed by pointer).
 * lr, beta1, beta2, eps, weight_decay: AdamW (Kingma & Ba 2015 with the
 *   decoupled decay of Loshchilov & Hutter 2019, schedule multiplier = lr);
 * max_grad_norm: clip threshold on the unscaled gradient norm, <= 0 = off;
 * backoff, growth, growth_interval, min_scale: dynamic loss scaling
 *   (Micikevicius et al. 2018) -- on an inf/NaN gradient the step is skipped
 *   and S <- max(S*backoff, min_scale); after growth_interval consecutive
 *   clean steps S <- S*growth (growth_interval <= 0: never grow). */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    double max_grad_norm;
    double backoff, growth, min_scale;
    int32_t growth_interval;
    int32_t reserved;
} zero_hparams_t;

/* Step state in DEVICE memory (128 bytes, 8-byte aligned).  Initialise it
 * with zero_step_state_init.  It carries the loss scaler and the Adam step
 * count between steps, and the last decision from zero_shard_norm_overflow to
 * zero_shard_adam_step.  The caller may copy it to the host to read it (after
 * synchronising the stream) and may save/restore it bytewise. */
typedef struct {
    /* carried from step to step */
    double   loss_scale;        /* S: gradients arrive multiplied by S */
    double   beta1_pow;         /* beta1^t, running binary64 product */
    double   beta2_pow;         /* beta2^t */
    int64_t  step;              /* t: applied (not skipped) steps */
    int32_t  good_steps;        /* clean steps since the last scale change */
    int32_t  skipped_total;     /* skipped steps so far */
    /* written by the last reduction (zero_shard_norm_overflow, its fp32
       form, or zero_shard_decide) */
    double   sumsq;             /* exact sum of squares of the scaled
                                   gradient, rounded once to binary64;
                                   +inf when overflow is set */
    double   grad_norm;         /* sqrt(sumsq) / S (unscaled norm); +inf on overflow */
    int32_t  overflow;          /* 1 if the gradient holds an inf or NaN */
    int32_t  skip;              /* 1 if this step is skipped (== overflow,
                                   or while wide_pending) */
    float    gmul;              /* fp32(coef / S): unscale and clip factor */
    float    bc1, bc2;          /* fp32(1 - beta1^t), fp32(1 - beta2^t) */
    float    lr, beta1, beta2;  /* fp32 hyperparameters of this step */
    float    omb1, omb2;        /* fp32(1 - beta1), fp32(1 - beta2) */
    float    eps, wd;
    uint32_t done_blocks;       /* internal arrival counter; 0 between calls */
    uint32_t wide_pending;      /* internal: 1 while an fp32 reduction waits
                                   for its wide pass (see
                                   zero_shard_norm_overflow_f32); 0 after it */
    uint64_t sumsq_units[2];    /* the exact sum in units of 2^-48 (low,
                                   high) when it is a whole number of them
                                   below 2^128 (always, for binary16
                                   gradients); otherwise both words are
                                   all ones */
} zero_step_state_t;

/* ---- model-state arithmetic (host only, no device work) ------------- */

/* Per-rank model-state bytes for a model of psi parameters over nd
 * data-parallel ranks, with k optimizer bytes per parameter (k = 12 for the
 * fp32 master, momentum and variance of mixed-precision Adam; paper card,
 * "Bottleneck").  A rank owns P = ceil(psi/nd) parameters.
 *   stage 0 (plain data parallel): (2 + 2 + k) * psi
 *   stage 1 (optimizer state):     4 * psi + k * P
 *   stage 2 (+ gradients):         2 * psi + (2 + k) * P
 *   stage 3 (+ parameters):        (2 + 2 + k) * P
 * (paper card, "Method": 4x, 8x and Nd-proportional reductions; "Evidence":
 * 1T parameters -> about 16 TB, about 16 GB per GPU over 1024 GPUs.)
 * Errors: ZERO_EINVAL (out_bytes NULL, nd == 0, stage not 0..3),
 *         ZERO_ERANGE (the result does not fit in 64 bits). */
int zero_state_bytes(uint64_t psi, uint32_t nd, uint32_t k, int stage, uint64_t* out_bytes);

/* Cut a segment list (sorted or not) to the destination window
 * [begin, end): every part of a segment whose dst range falls inside the
 * window is written to out (host array of cap entries), in input order.
 * This is how a partition is flattened in fixed-size buckets (paper card,
 * "Method": temporary buffers sized to balance memory and throughput).
 * Errors: ZERO_EINVAL (NULL pointers, begin > end), ZERO_ERANGE (more than
 * cap pieces; *out_n then holds the number needed). */
int zero_bucket_segments(const zero_segment_t* segs, uint32_t nsegs, uint64_t begin,
                         uint64_t end, zero_segment_t* out, uint32_t cap, uint32_t* out_n);

/* ---- device step ----------------------------------------------------- */

/* Enqueue the initialisation of a step state: loss_scale = initial_scale,
 * beta powers 1, step and all counters 0.  dev_state: device, 8-byte aligned.
 * Errors: ZERO_EINVAL (NULL, initial_scale not finite and > 0),
 *         ZERO_EALIGN, ZERO_EHIP. */
int zero_step_state_init(zero_step_state_t* dev_state, double initial_scale, void* stream);

/* Flatten: for each segment, dst[dst_off + i] <- src[src_off + i], i < count.
 *   dst_dtype ZERO_F16, accumulate 0: bit copy of the binary16 values;
 *   dst_dtype ZERO_F16, accumulate 1: dst = fp16(dst + src) (correctly
 *                                     rounded binary16 addition);
 *   dst_dtype ZERO_F32, accumulate 0: dst = fp32(src) (exact);
 *   dst_dtype ZERO_F32, accumulate 1: dst = dst + fp32(src) (binary32 add).
 * segs: HOST array of nsegs entries (the src pointers inside are device
 * pointers); dst: device, dst_len elements, 16-byte aligned.  Destination
 * elements no segment covers are not touched.  Segment destinations must not
 * overlap each other (the result of overlapping segments is unspecified).
 * Any number of segments; the library may split them over several launches.
 * Errors: ZERO_EINVAL (NULL dst/segs with nsegs > 0, NULL src, bad dtype),
 *         ZERO_ERANGE (dst_off + count > dst_len), ZERO_EALIGN (dst base or
 *         a src pointer not 2-byte aligned, dst base not 16-byte aligned),
 *         ZERO_EHIP. */
int zero_flatten_bucket(const zero_segment_t* segs, uint32_t nsegs, void* dst, uint64_t dst_len,
                        int dst_dtype, int accumulate, void* stream);

/* ---- fused flatten + norm (the norm without a second pass) ----------- */

/* Bytes of one per-workgroup partial of the exact sum (opaque contents). */
#define ZERO_NORM_PARTIAL_BYTES 16

/* Number of partials zero_flatten_norm_bucket writes for this segment list
 * (one per workgroup it launches; host only, no device work).  0 for NULL. */
uint64_t zero_flatten_norm_partials(const zero_segment_t* segs, uint32_t nsegs);

/* The fp16 flatten of zero_flatten_bucket (bit copy, or fp16 accumulate),
 * which also computes, for every value it stores, the exact square and the
 * inf/NaN test, and writes one partial per workgroup to partials[0 ..
 * zero_flatten_norm_partials(segs, nsegs)).  For a step flattened in several
 * buckets, give each call its own stretch of one partials buffer and fold all
 * of them with zero_shard_decide.  The norm so obtained covers exactly the
 * elements the segments write (the whole partition when the segments cover
 * it, as in a ZeRO shard; paper card, "Method": contiguous buffers).
 * dst: device binary16, dst_len elements, 16-byte aligned; partials: device,
 * 16-byte aligned, partials_capacity entries of ZERO_NORM_PARTIAL_BYTES.
 * Errors: those of zero_flatten_bucket, and ZERO_EINVAL (NULL partials),
 *         ZERO_EALIGN, ZERO_ERANGE (partials_capacity too small). */
int zero_flatten_norm_bucket(const zero_segment_t* segs, uint32_t nsegs, uint16_t* dst, uint64_t dst_len,
                             int accumulate, void* partials, uint64_t partials_capacity, void* stream);

/* The fp32 flatten of zero_flatten_bucket (dst = fp32(src), or with
 * accumulate dst = dst + fp32(src) in binary32), which also computes the
 * exact-norm partials of every fp32 value it stores, under the rules of
 * zero_shard_norm_overflow_f32.  Used for the last micro-batch of a
 * gradient-accumulation step: the partials it writes, folded by
 * zero_shard_decide, give exactly the decision zero_shard_norm_overflow_f32
 * takes on the finished partition.  It writes
 * zero_flatten_norm_partials(segs, nsegs) partials, like the fp16 form.
 * dst: device binary32, dst_len elements, 16-byte aligned; the rest as for
 * zero_flatten_norm_bucket.  Errors: as zero_flatten_norm_bucket. */
int zero_flatten_norm_bucket_f32(const zero_segment_t* segs, uint32_t nsegs, float* dst, uint64_t dst_len,
                                 int accumulate, void* partials, uint64_t partials_capacity, void* stream);

/* Several buckets of one step in one call: the same stores (and, with
 * partials, the same partials) as calling zero_flatten_bucket -- or
 * zero_flatten_norm_bucket / zero_flatten_norm_bucket_f32 when partials is
 * not NULL -- once per bucket, in order, each bucket's partials right after
 * the previous bucket's (paper card, "Method": the partition is one
 * contiguous buffer; the buckets are windows of it).  The first launch waits
 * for the work queued earlier on the stream, like any launch; the launches
 * between the first and the last are issued without the dispatch barrier,
 * so consecutive buckets overlap on the GPU instead of draining it between
 * them; the last keeps the barrier, so its completion implies every
 * earlier one's and anything queued or waiting on the stream after the call
 * (kernels, copies, events, synchronisation) sees all of them.  That is only safe
 * because no two buckets touch a common element: every segment's
 * destination range must be disjoint from every other's, and the call
 * checks it.
 * segs: HOST array of the buckets' segment lists, one after another;
 * bucket_nsegs: HOST array of nbuckets counts; dst: device, binary16 or
 * binary32 (dst_dtype), dst_len elements, 16-byte aligned; partials: NULL
 * (no norm) or device, 16-byte aligned, partials_capacity entries of
 * ZERO_NORM_PARTIAL_BYTES, at least zero_flatten_norm_partials(segs, total
 * segments) of them.  dst_dtype and accumulate as for zero_flatten_bucket.
 * Errors: those of zero_flatten_bucket and zero_flatten_norm_bucket;
 *         ZERO_EINVAL also for NULL bucket_nsegs with nbuckets > 0 and for
 *         two segments whose destination ranges overlap; ZERO_ERANGE for
 *         more than 2^32 - 1 segments in all; ZERO_ENOMEM if the host
 *         cannot allocate the overlap check's list.  No device work is
 *         queued when an argument error is returned. */
int zero_flatten_buckets(const zero_segment_t* segs, const uint32_t* bucket_nsegs, uint32_t nbuckets, void* dst,
                         uint64_t dst_len, int dst_dtype, int accumulate, void* partials,
                         uint64_t partials_capacity, void* stream);

/* Bytes of device workspace zero_shard_decide needs to fold `count` partials. */
size_t zero_decide_workspace_bytes(uint64_t count);

/* Folds `count` partials written by zero_flatten_norm_bucket into the
 * exact sum and overflow flag, then takes exactly the decision that
 * zero_shard_norm_overflow takes (same fields of dev_state, bit for bit).
 * Partials of zero_flatten_norm_bucket_f32 go to zero_shard_decide_f32:
 * folded here, a partition off the fast path (see
 * zero_shard_norm_overflow_f32) leaves the step pending and skipped with
 * the loss scale and counters untouched.
 * partials, workspace: device, 16-byte aligned; hp: host; workspace of at
 * least zero_decide_workspace_bytes(count).
 * Errors: as zero_shard_norm_overflow (ZERO_ERANGE: count > 2^30 or
 *         workspace too small). */
int zero_shard_decide(const void* partials, uint64_t count, const zero_hparams_t* hp,
                      zero_step_state_t* dev_state, void* workspace, size_t workspace_bytes, void* stream);

/* The decision over the partials of zero_flatten_norm_bucket_f32 calls that
 * together wrote the fp32 partition grad32[0..n): the fold of
 * zero_shard_decide, then the wide pass over grad32 when the fold left the
 * step pending.  The result is exactly zero_shard_norm_overflow_f32's on
 * the same partition, bit for bit.  grad32: device, 4-byte aligned (NULL
 * allowed when n = 0); the rest as zero_shard_decide.
 * Errors: those of zero_shard_decide, and ZERO_ERANGE (n > 2^40). */
int zero_shard_decide_f32(const void* partials, uint64_t count, const float* grad32, uint64_t n,
                          const zero_hparams_t* hp, zero_step_state_t* dev_state, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of device workspace zero_shard_norm_overflow needs for n elements
 * (per-block partial sums; fixed for a given n). */
size_t zero_norm_workspace_bytes(uint64_t n);

/* Reduce and decide.  Over the n binary16 gradient elements at grad16:
 *   overflow = 1 if any element has an all-ones exponent (inf or NaN);
 *   sumsq    = the exact sum of squares, rounded once to binary64
 *              (+inf on overflow);
 * then, from the state in dev_state and the hyperparameters in hp:
 *   overflow -> skip = 1, S <- max(S*backoff, min_scale), good_steps <- 0;
 *   otherwise -> skip = 0, t += 1, beta powers advance,
 *               grad_norm = sqrt(sumsq)/S,
 *               coef = grad_norm > max_grad_norm > 0 ? max_grad_norm/grad_norm : 1,
 *               gmul = fp32(coef/S), bc1/bc2 = fp32(1 - beta^t),
 *               good_steps += 1 and S <- S*growth every growth_interval.
 * All of it is written into dev_state for zero_shard_adam_step.  Result bits
 * do not depend on the launch configuration (the sum is exact).
 * grad16: device, 16-byte aligned; n may be 0; hp: host;
 * dev_state: device, 8-byte aligned, initialised by zero_step_state_init;
 * workspace: device, 16-byte aligned, >= zero_norm_workspace_bytes(n),
 * contents need no initialisation.
 * Errors: ZERO_EINVAL (NULL, hyperparameters out of range: lr < 0,
 *         beta not in [0,1), eps <= 0, weight_decay < 0, backoff not in
 *         (0,1], growth < 1, min_scale <= 0, any non-finite value),
 *         ZERO_EALIGN, ZERO_ERANGE (workspace too small, n > 2^40),
 *         ZERO_EHIP. */
int zero_shard_norm_overflow(const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                             zero_step_state_t* dev_state, void* workspace,
                             size_t workspace_bytes, void* stream);

/* zero_shard_norm_overflow without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same reduction, same kernels,
 * same result bits and errors, except:
 *   - the per-workgroup partials live in a fixed device array inside the
 *     library (256 partials, 4 KiB), which each GPU the library runs on holds
 *     from the first call on that GPU until the process ends; its device
 *     address is looked up once per GPU, on that call, with that GPU current;
 *   - hence n <= 2^30 (ZERO_ERANGE above; the largest n whose grid of at
 *     most 256 workgroups fits the array);
 *   - every call on one GPU shares that array, and each call leaves its
 *     partials there: calls that overlap in time on one GPU (on different
 *     streams, or from different host threads) race and give undefined
 *     results -- order them on one stream.  Nothing in the array needs to
 *     start at zero (every partial a call reads, the same call wrote).
 * The call allocates nothing (no hipMalloc/hipFree, no allocating library
 * routine).  The stream must belong to the current device. */
int zero_shard_norm_overflow_noalloc(const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                                     zero_step_state_t* dev_state, void* stream);

/* Reduce and decide over an fp32 gradient partition (gradient
 * accumulation: a binary32 sum of micro-batch fp16 gradients).
 *   overflow = 1 if any element is inf or NaN;
 *   sumsq    = the exact sum of the squares of all n values, rounded once
 *              to binary64 (any finite binary32 values);
 * then the same decision as zero_shard_norm_overflow.  Two kernels: the
 * fast reduction sums exactly when every value is a multiple of 2^-24 below
 * 2^24 in magnitude (true of any binary32 sum of at most 256 binary16
 * values); when one is not, it leaves the decision pending
 * (wide_pending = 1) and the wide pass that follows sums the squares of any
 * binary32 values exactly (slower: LDS-atomic bound) and decides.  On the
 * fast path the wide pass returns at once.  sumsq_units holds the exact sum
 * in 2^-48 units when it is a whole number of them below 2^128, else all
 * ones.  grad32: device, 16-byte aligned; everything else as for
 * zero_shard_norm_overflow, including the workspace size
 * (zero_norm_workspace_bytes(n), which covers both kernels) and the
 * errors. */
int zero_shard_norm_overflow_f32(const float* grad32, uint64_t n, const zero_hparams_t* hp,
                                 zero_step_state_t* dev_state, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The fused element update, in binary32 with one rounding per operation and
 * this order (unless dev_state says skip, in which case nothing is written):
 *   g  = fp32(grad16[i]) * gmul
 *   m  = beta1*m32[i] + omb1*g
 *   v  = beta2*v32[i] + omb2*(g*g)
 *   u  = (m/bc1) / (sqrt(v/bc2) + eps) + wd*p32[i]
 *   p  = p32[i] - lr*u
 *   m32[i] = m; v32[i] = v; p32[i] = p; p16[i] = fp16(p) (round to nearest even)
 * It reads 2 + 12 bytes and writes 12 + 2 bytes per parameter.
 * All five arrays: device, n elements, 16-byte aligned, index-aligned with
 * each other and with the grad16 the decision was made on; n may be 0.
 * Placement (performance only): the five arrays are streamed together; on
 * MI355X the update is 1-5% faster when they share one allocation with array
 * k (p32, m32, v32, grad16, p16) starting at a 2 MiB boundary plus k * 64 KiB,
 * as the Python binding's StateArena lays them out.
 * dev_state: as left by zero_shard_norm_overflow (read only here).
 * Errors: ZERO_EINVAL (NULL), ZERO_EALIGN, ZERO_ERANGE (n above about 2^42:
 *         more than 2^31 - 1 workgroups of 2048 parameters), ZERO_EHIP. */
int zero_shard_adam_step(uint16_t* p16, float* p32, float* m32, float* v32,
                         const uint16_t* grad16, uint64_t n,
                         const zero_step_state_t* dev_state, void* stream);

/* The same update reading an fp32 gradient (gradient accumulation):
 *   g = grad32[i] * gmul, then exactly as zero_shard_adam_step.
 * It reads 4 + 12 bytes and writes 12 + 2 bytes per parameter (30).
 * dev_state: as left by zero_shard_norm_overflow_f32, or by
 * zero_shard_decide over zero_flatten_norm_bucket_f32 partials.
 * grad32: device, n elements, 16-byte aligned; the rest and the errors as
 * for zero_shard_adam_step. */
int zero_shard_adam_step_f32(uint16_t* p16, float* p32, float* m32, float* v32,
                             const float* grad32, uint64_t n,
                             const zero_step_state_t* dev_state, void* stream);

/* ---- 1-bit Adam, compression stage ------------------------------------ */

/* State of the compression stage in DEVICE memory (72 bytes, 8-byte
 * aligned; initialise with zero_onebit_state_init).  After each step it
 * holds the two scales and their exact sums. */
typedef struct {
    float    scale_w, scale_s;  /* worker and server scales of the last step */
    double   sumsq_w, sumsq_s;  /* the exact sums of squares, rounded once to binary64 */
    int32_t  qexp_w, qexp_s;    /* diagnostics of the fast windowed sums: the */
    uint32_t done_blocks;       /*   final window's unit 2^qexp; internal
                                     arrival counter (0 between calls) */
    uint32_t wide_pending;      /* internal: bit 0 / bit 1 while the worker /
                                   server scale waits for its wide pass */
    uint64_t units_w[2];        /* the windowed sums as integers of 2^qexp */
    uint64_t units_s[2];        /* units (low, high), before the wide pass */
} zero_onebit_state_t;

/* Enqueue the zeroing of a compression-stage state.
 * Errors: ZERO_EINVAL (NULL), ZERO_EALIGN, ZERO_EHIP. */
int zero_onebit_state_init(zero_onebit_state_t* dev_onebit, void* stream);

/* Bytes of device workspace zero_onebit_step needs for n elements. */
size_t zero_onebit_workspace_bytes(uint64_t n);

/* One step of 1-bit Adam (the DeepSpeed article: 1-bit Adam cuts
 * communication up to 5x with Adam-like convergence; the algorithm is Tang
 * et al. 2021, Algorithm 1), after zero_shard_decide (or
 * zero_shard_norm_overflow) has decided it.  The device chooses the stage
 * from the applied-step count in dev_state, so the host never reads it back
 * and one captured graph can cross from one stage to the other:
 *   warm-up (the applied steps before this one number fewer than `warmup`,
 *   i.e. dev_state->step <= warmup after the decision): the ordinary update
 *   of zero_shard_adam_step, which also builds the variance v32;
 *   compression stage (otherwise): v32 frozen, and with the decision in
 *   dev_state (gmul, beta1, lr, eps, wd), on this rank, its own server:
 *     g = fp32(grad16)*gmul;  m = beta1*m + (1-beta1)*g
 *     x = m + err_w;  s_w = S(x);  bits_w = sgn(x);  err_w = x - s_w*sgn(x)
 *     u = s_w*sgn(x) + err_s;  s_s = S(u);  bits_s = sgn(u)
 *     m = s_s*sgn(u);  err_s = u - m
 *     p = p - lr*(m/(sqrt(v)+eps) + wd*p);  p16 = fp16(p)
 * A skipped step (overflow) changes nothing, errors and bits included; the
 * kernels of the stage not taken return at once, before any load.
 * sgn(x) = +1 for x >= 0 (zeros too), -1 otherwise; bit k of byte j of a
 * bits array is element 8j+k, 1 for +1.  S(x) = fp32(sqrt(sum/n)) with the
 * sum of squares exact and rounded once to binary64.  The fast sum works in
 * windows: each workgroup of 4096 elements rounds its squares to multiples
 * of 2^(2E_b-80), 2^E_b <= its max|x| < 2^(E_b+1), and a fold moves those
 * integer sums onto the window of the largest E_b, rounding each to the
 * nearest unit; it keeps the result when the binary64 rounding is the same
 * at both ends of the error interval this leaves, and otherwise hands the
 * sum to a wide pass that is exact for any binary32 values.
 * Every elementwise operation is one binary32 operation in the order
 * above.  Results do not depend on the launch configuration.
 * p16, p32, m32, v32, err_w, err_s, grad16: device, n elements, 16-byte
 * aligned; bits_w, bits_s: device, (n+7)/8 bytes; workspace: device,
 * 256-byte aligned, >= zero_onebit_workspace_bytes(n).
 * Errors: ZERO_EINVAL (NULL, warmup < 0), ZERO_EALIGN, ZERO_ERANGE
 *         (n > 2^40, workspace too small), ZERO_EHIP. */
int zero_onebit_step(uint16_t* p16, float* p32, float* m32, float* v32, float* err_w, float* err_s,
                     const uint16_t* grad16, uint64_t n, uint8_t* bits_w, uint8_t* bits_s,
                     const zero_step_state_t* dev_state, zero_onebit_state_t* dev_onebit, int64_t warmup,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---- host step (ZeRO-Offload form) ----------------------------------- */

/* A host context: a pool of worker threads (and, once zero_offload_step has
 * run, the HIP events it pipelines with).  Calls that share a context must
 * not overlap; different contexts are independent.  Every zero_host_* call
 * runs on the calling thread plus the pool and returns when it is done. */
typedef struct zero_host_ctx zero_host_ctx_t;

/* Create a context with `threads` workers in all (the calling thread counts
 * as one; <= 0: every CPU this process may run on).
 * Errors: ZERO_EINVAL (out NULL), ZERO_ENOTSUP (the CPU lacks AVX-512 F, BW,
 *         VL, DQ, F16C or FMA), ZERO_ERANGE (threads > 1024), ZERO_ENOMEM. */
int zero_host_create(int threads, zero_host_ctx_t** out);

/* Stop the workers and free the context (NULL is allowed). */
void zero_host_destroy(zero_host_ctx_t* ctx);

/* Number of workers of a context (0 for NULL). */
int zero_host_threads(const zero_host_ctx_t* ctx);

/* zero_step_state_init for a step state in HOST memory (no device work).
 * Errors: ZERO_EINVAL (NULL, initial_scale not finite and > 0). */
int zero_host_state_init(zero_step_state_t* state, double initial_scale);

/* zero_shard_norm_overflow on the CPU: over the n binary16 values at grad16
 * (host memory, any alignment), the same overflow test and the same exact
 * sum of squares, then the same decision into the HOST step state, bit for
 * bit (one source for the decision; the sum is exact on both).
 * Errors: ZERO_EINVAL (NULL, hyperparameters out of range as for
 *         zero_shard_norm_overflow). */
int zero_host_norm_overflow(zero_host_ctx_t* ctx, const uint16_t* grad16, uint64_t n, const zero_hparams_t* hp,
                            zero_step_state_t* state);

/* zero_shard_adam_step on the CPU: the same element update, each operation
 * one binary32 round-to-nearest-even operation in the same order, the fp16
 * copy rounded to nearest even -- bit-identical to the device kernel.  All
 * arrays are host memory of n elements; any alignment works, and when p32,
 * m32, v32 are 64-byte aligned and p16 32-byte aligned at the same index the
 * stores bypass the caches.  Nothing is written when state->skip is set.
 * Errors: ZERO_EINVAL (NULL). */
int zero_host_adam_step(zero_host_ctx_t* ctx, uint16_t* p16, float* p32, float* m32, float* v32,
                        const uint16_t* grad16, uint64_t n, const zero_step_state_t* state);

/* The whole offloaded step for a partition whose fp16 gradient and fp16
 * parameters live on the device and whose fp32 master parameters, momentum
 * and variance live in host memory.  Two ways to decide:
 *   dev_state NULL: the CPU decides.  dev_grad16 is copied to host_grad16
 *     in chunks on `stream`, each chunk reduced on the CPU as soon as it has
 *     landed; then the decision into the host `state` (as
 *     zero_host_norm_overflow; `hp` is required);
 *   dev_state given: the device has already decided on `stream`
 *     (zero_shard_decide over zero_flatten_norm_bucket partials, or
 *     zero_shard_norm_overflow), bit-identically to the CPU's decision.  The
 *     128-byte device state is copied into `state` first, then the gradient
 *     chunks, and the CPU updates each chunk as soon as it has landed
 *     (`hp` is not used and may be NULL).
 * Unless the step is skipped, each chunk is updated on the CPU (as
 * zero_host_adam_step, fp16 parameters into host_p16) and its copy
 * host_p16 -> dev_p16 is enqueued on `stream` right away.  The call returns
 * once every update is done; copies may still be in flight on `stream`
 * (later work on `stream` sees them; the host must not touch host_grad16
 * or host_p16 before they complete).  host_grad16, host_p16 and `state`
 * should be pinned host memory (hipHostMalloc) for the copies to overlap.
 * chunk_elems is the largest chunk; the first chunks ramp up from
 * chunk_elems/16 (at least 64) by doubling and the last ones ramp down the
 * same way, so the CPU starts once a small chunk has landed and the last
 * parameters go up right after their update; every chunk boundary but n is a
 * multiple of 64 elements.  The results do not depend on the chunking.
 * dev_grad16, dev_p16, dev_state: device; the other arrays host memory.
 * Errors: ZERO_EINVAL (NULL, hyperparameters out of range), ZERO_EALIGN
 *         (chunk_elems 0 or not a multiple of 64, dev_state not 8-byte
 *         aligned), ZERO_ERANGE (n above 4096 * chunk_elems), ZERO_EHIP (a copy,
 *         event or synchronisation failed). */
int zero_offload_step(zero_host_ctx_t* ctx, const uint16_t* dev_grad16, uint16_t* dev_p16, uint16_t* host_grad16,
                      uint16_t* host_p16, float* p32, float* m32, float* v32, uint64_t n,
                      const zero_hparams_t* hp, zero_step_state_t* state, const zero_step_state_t* dev_state,
                      uint64_t chunk_elems, void* stream);

/* A streaming copy of `bytes` host bytes (dst, src 64-byte aligned, bytes a
 * multiple of 64) on the context's workers: the host memory bandwidth
 * reference next to the host step.  Errors: ZERO_EINVAL, ZERO_EALIGN. */
int zero_host_stream_copy(zero_host_ctx_t* ctx, void* dst, const void* src, uint64_t bytes);

/* ---- measurement reference ------------------------------------------ */

/* A plain streaming copy of `bytes` bytes (dst and src device, 16-byte
 * aligned, bytes a multiple of 16), used to measure the attainable HBM
 * bandwidth next to the step's kernels.  Errors: ZERO_EINVAL, ZERO_EALIGN,
 * ZERO_ERANGE (more than 2^31 - 1 workgroups), ZERO_EHIP. */
int zero_stream_copy(void* dst, const void* src, uint64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_MI355X_H */
