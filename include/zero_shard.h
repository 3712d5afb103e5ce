/*
 * zero_shard.h -- C ABI of libzeroshard.so: one data-parallel rank's ZeRO
 * partition step for mixed-precision Adam on an AMD MI355X (gfx950).
 *
 * Sources (three web pages; cited by title and section):
 *   [16B]  "Your 7.5B model's weights fit in 15 GB ... the 16-byte parameter
 *          and ZeRO's three-stage split" (blog.teqners.com)
 *   [ER10] "ZeRO and the Memory Tricks", The Engine Room ch. 10
 *          (hoshank.vercel.app)
 *   [DSZ]  "DeepSpeed ZeRO: account for every training state"
 *          (chenhuiyu.github.io)
 *
 * Conventions for every function:
 *  - Returns a status: ZERO_OK (0) or a negative ZERO_E* code; outputs are
 *    written only on ZERO_OK.  No C++ exception crosses this boundary.
 *  - "Device pointer" means memory of the current HIP device (hipMalloc'd,
 *    e.g. by PyTorch).  "Host pointer" means ordinary process memory.
 *  - fp16 arrays hold IEEE binary16 values (2 bytes each), fp32 arrays IEEE
 *    binary32 values, all contiguous, element i at byte offset i * size.
 *  - `stream` is a hipStream_t (NULL: the default stream).  Device work is
 *    enqueued on it and the call returns without synchronising; results are
 *    ready once the stream reaches that point.
 *  - The step and reduce entry points allocate nothing.  The library's only
 *    global state is, per device, the address of the fixed array that
 *    zero_adam_step_noalloc builds its table in (set once, on that entry
 *    point's first call on the device).
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK 0
#define ZERO_EINVAL (-1)    /* bad argument (null, range, alignment, aliasing) */
#define ZERO_EOVERFLOW (-2) /* a byte or element count exceeds 64 bits */
#define ZERO_EHIP (-3)      /* HIP runtime or launch error (captured, cleared) */
#define ZERO_ENOMEM (-4)    /* allocation failed (plan or offload creation only) */
#define ZERO_ENOTSUP (-5)   /* host CPU lacks AVX2 and F16C (host Adam, offload) */
#define ZERO_ERANGE (-6)    /* beyond the fixed limits of zero_adam_step_noalloc */

/* Largest N_d zero_reduce_grad_shard accepts (slice pointers travel as
 * kernel arguments). */
#define ZERO_MAX_SLICES 256

/* Slices from which zero_reduce_adam_step runs the reduce and the Adam
 * kernels in sequence instead of its fused kernel. */
#define ZERO_FUSED_SPLIT_SLICES 16

/* Shard of a flat buffer of psi elements split over nd ranks. */
typedef struct zero_layout {
    uint64_t padded_total; /* psi rounded up to a multiple of nd * align */
    uint64_t shard_len;    /* padded_total / nd, a multiple of align */
    uint64_t offset;       /* rank * shard_len: first element of this shard */
    uint64_t real_len;     /* elements of this shard below psi (rest: pad) */
} zero_layout;

/* Per-rank communication of one training step (see zero_comm_volume). */
typedef struct zero_comm {
    uint64_t passes;          /* reduce-scatter / all-gather passes: 2 or 3 */
    uint64_t volume_elems;    /* passes * psi: the pages' per-step volume */
    uint64_t ring_send_elems; /* passes * (nd - 1) * shard_len: what one rank
                                 sends in ring collectives over the padded
                                 layout (fp16: 2 bytes per element) */
} zero_comm;

/* One tensor of this rank's shard: five device arrays of n elements.
 * param_f16 is written, grad_f16 read, master/m/v read and written in
 * place.  The five ranges must not overlap.  The memory is borrowed: the
 * caller owns it and keeps it alive while a plan refers to it. */
typedef struct zero_tensor {
    void *param_f16;      /* fp16 parameter (written fresh each step) */
    const void *grad_f16; /* fp16 gradient of this rank's shard */
    float *master;        /* fp32 master copy of the parameter */
    float *m;             /* fp32 Adam first moment */
    float *v;             /* fp32 Adam second moment */
    uint64_t n;           /* elements; 0 is allowed (pointers then ignored) */
} zero_tensor;

/* Adam hyperparameters, as doubles; see zero_adam_scalars for how they
 * become the fp32 constants of the step. */
typedef struct zero_adam_hparams {
    double lr, beta1, beta2, eps;
    double weight_decay; /* must be 0: the pages define no weight decay */
} zero_adam_hparams;

/* Opaque multi-tensor plan (device-resident chunk table). */
typedef struct zero_plan zero_plan;

/* What a plan (or a would-be plan) contains. */
typedef struct zero_plan_stats {
    uint64_t n_tensors;
    uint64_t n_params;      /* sum of n over the tensors */
    uint64_t n_chunks;      /* work items; one workgroup handles one at a time */
    uint64_t chunk_elems;   /* elements per chunk (a tensor's first chunk also
                               holds its peeled head; its last may be short) */
    uint64_t vector_elems;  /* elements of tensors on the vector path (8-byte
                               fp16 and 16-byte fp32 vectors) outside their
                               single heads and tails; a partial last tile
                               or small chunk of more than 64 elements is
                               still updated element by element, in one
                               pass over memory */
    uint64_t scalar_elems;  /* elements done one at a time (heads, tails,
                               tensors whose arrays disagree in alignment,
                               except the 16-bit arrays alone on tensors of
                               1,024 elements or more: see zero_plan_create) */
    uint64_t table_bytes;   /* device bytes of the chunk table */
    uint64_t tile_elems;    /* elements one 64-lane wave of the step updates:
                               256 or 512 (see zero_plan_create) */
    uint64_t wg_per_cu;     /* one-wave workgroups of the step resident per CU
                               (its occupancy cap): 12 with 256-element
                               tiles; with 512-element tiles 7, or 14-27 for
                               lists of small tensors (see zero_plan_create) */
} zero_plan_stats;

/*
 * zero_shard_layout -- flat-buffer padding and this rank's shard.
 * Ranks own contiguous slices of the flattened state ([16B] "The part that
 * sounds too good: communication"; [DSZ] "ZeRO removes replicated state in
 * stages").  The buffer of psi elements is padded at its tail to
 * padded_total = ceil(psi / (nd * align)) * nd * align elements; every rank
 * gets shard_len = padded_total / nd elements starting at rank * shard_len,
 * of which real_len lie below psi (the padding sits in the last shards).
 * align is in elements.  psi = 0 is allowed (all zero).  align = 64 puts
 * every rank's fp16 view of a line-aligned buffer on a 128-byte line, which
 * the kernels stream fastest (a view off its lines costs the Adam step a
 * few percent and the gather more).
 * Pure host function.  Errors: EINVAL if out is NULL, nd = 0, align = 0 or
 * rank >= nd; EOVERFLOW if padded_total exceeds 2^64 - 1.
 */
int zero_shard_layout(uint64_t psi, uint32_t nd, uint32_t rank, uint32_t align,
                      zero_layout *out);

/*
 * zero_state_bytes -- model-state bytes resident on one rank.
 * [ER10] "The Mathematics", eq. M_states = (2 + 2 + K) Psi with K = 12 and
 * eq. M_states(p, N_d); [16B] "The replication nobody questioned", stage
 * table.  With S the padded shard length of zero_shard_layout:
 *   stage 0: 16 psi   1: 4 psi + 12 S   2: 2 psi + 14 S   3: 16 S
 * Activations, communication buffers and allocator effects are excluded
 * ([DSZ] "ZeRO removes replicated state in stages").
 * Pure host function.  Errors: EINVAL (out NULL, stage > 3, nd = 0,
 * align = 0); EOVERFLOW.
 */
int zero_state_bytes(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                     uint64_t *out_bytes);

/*
 * zero_comm_volume -- elements one rank moves per training step.
 * [16B] "The part that sounds too good: communication"; [ER10] "The
 * Mathematics", communication paragraph, and "What It Enabled", stage
 * table.  Each pass (a reduce-scatter or an all-gather; a ring all-reduce
 * runs one of each) moves Psi elements: plain data parallelism (stage 0)
 * and stages 1-2 (gradient reduce-scatter, fp16 parameter all-gather) move
 * 2 Psi; stage 3 adds the parameter all-gathers before the forward and the
 * backward pass: 3 Psi.
 * Volumes count elements (each fp16 element is 2 bytes).  ring_send_elems
 * is the exact count over the padded layout: every ring pass has each rank
 * send nd - 1 shards of shard_len elements.
 * Pure host function.  Errors: EINVAL (out NULL, stage > 3, nd = 0,
 * align = 0); EOVERFLOW.
 */
int zero_comm_volume(uint32_t stage, uint64_t psi, uint32_t nd, uint32_t align,
                     zero_comm *out);

/*
 * zero_plan_create -- chunk table for a list of tensors of mixed sizes.
 * tensors: host array of n_tensors descriptors (copied; the table does not
 * keep the host array).  Each tensor is cut into chunks of chunk_elems
 * elements after its peeled head, which rides in its first chunk (its
 * last chunk may be shorter); the step runs one 64-lane wave
 * per tile_elems consecutive elements of a chunk: 256 when at least 7/8 of
 * the plan's elements take the vector path and chunk_elems is 16384, else
 * 512 (the faster of the two, measured, for such plans).
 * chunk_elems: 0 lets the library choose: the largest of 16384, 8192, ...,
 * 512 whose 512-element tiles (counted over every chunk, a tensor's last
 * chunk included) exceed those with work by at most one eighth, so 16384 for
 * big tensors and smaller chunks for many small ones; otherwise a multiple
 * of 512 between 512 and 2^24.  Per tensor the library takes the vector path
 * (8-byte fp16 and 16-byte fp32 accesses) when all five arrays agree in
 * alignment after peeling at most 3 leading elements; when only the
 * 16-bit arrays disagree (views of full buffers at an offset that is not a
 * multiple of four elements), on a tensor of 1,024 elements or more, it
 * keeps the vector path, stores the parameter's 8-byte vectors shifted
 * across lanes and reads the gradient's four values per lane from two
 * whole aligned 8-byte words (measured 2-30% faster than single elements
 * there, slower on smaller tensors); otherwise it moves single elements.  On the vector path,
 * for a tensor of 1,024 elements or more, the peeled head runs on to the
 * element at which the tensor's master, m and v reach a 1 KiB boundary, when
 * they reach one at the same element (at most 255 elements, done by the
 * tensor's first tile), so that its chunks and tiles start there: a list
 * packed at offsets that are not multiples of 256 elements streams about 3%
 * faster so (measured).  The step keeps wg_per_cu one-wave workgroups
 * resident per CU: 12 with 256-element tiles, and with 512-element tiles 7
 * unless at least one tile in 200 holds a head or a tensor's partial last
 * tile, when the cap grows as the tiles' average element count e shrinks,
 * 7 * 512 / e + 7 within 14..27, 19 and 21 taken as 20 and 22 (lists of
 * small tensors wait on memory more per element; measured up to twice as
 * fast so).  The table is allocated on the current device (hipMalloc) and
 * filled with a synchronous copy; nothing else is allocated later.
 * Ownership: *out belongs to the caller until zero_plan_destroy.  The
 * tensors' memory stays the caller's and must outlive the plan.
 * Errors: EINVAL (NULL out or tensors with n_tensors > 0, a NULL array of
 * a non-empty tensor, fp16 arrays not 2-byte or fp32 arrays not 4-byte
 * aligned, overlapping arrays within or across tensors where one is
 * written, a bad chunk_elems); EOVERFLOW; ENOMEM; EHIP.
 */
int zero_plan_create(const zero_tensor *tensors, uint32_t n_tensors,
                     uint32_t chunk_elems, zero_plan **out);

/*
 * zero_plan_create_bf16 -- as zero_plan_create, for tensors whose parameter
 * and gradient arrays hold bfloat16 values (param_f16 and grad_f16 then
 * point to bfloat16): the variant that keeps the 16-byte ledger with
 * bfloat16 in place of fp16 ([DSZ] "Why parameter count is not training
 * memory": BF16 setups differ in which states they keep).  zero_adam_step
 * on such a plan widens the gradient from bfloat16 (exact), runs the same
 * fp32 update and rounds the parameter to the nearest bfloat16 (ties to
 * even); the non-finite flag tests the bfloat16 exponent field.
 */
int zero_plan_create_bf16(const zero_tensor *tensors, uint32_t n_tensors,
                          uint32_t chunk_elems, zero_plan **out);

/* zero_plan_stats_of -- fill *out for an existing plan.  Host only. */
int zero_plan_stats_of(const zero_plan *plan, zero_plan_stats *out);

/*
 * zero_plan_describe -- the same classification zero_plan_create would do,
 * without touching any device: pointers are only inspected as numbers.
 * Host only.  Errors as zero_plan_create minus ENOMEM and EHIP.
 */
int zero_plan_describe(const zero_tensor *tensors, uint32_t n_tensors,
                       uint32_t chunk_elems, zero_plan_stats *out);

/* zero_plan_destroy -- free the table.  No step using the plan may still be
 * in flight.  NULL is accepted.  Errors: EHIP. */
int zero_plan_destroy(zero_plan *plan);

/*
 * zero_adam_scalars -- the fp32 constants of step t (t >= 1).
 * out = {lr, b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, eps}; each is computed in
 * double from the double hyperparameters and rounded to fp32 once.
 * Host only.  Errors: EINVAL (NULL, t = 0, weight_decay != 0, lr or eps not
 * finite, eps < 0, betas outside [0, 1)).
 */
int zero_adam_scalars(const zero_adam_hparams *hp, uint64_t t, float out[8]);

/*
 * zero_adam_step -- one fused mixed-precision Adam step over every tensor of
 * the plan: this rank updates only its slice ([16B] "The part that sounds
 * too good: communication"), keeping fp32 master, momentum and variance and
 * writing fresh fp16 parameters ([16B] "Where 16 bytes per parameter comes
 * from", state table; "Why you can't just delete the fp32 copies").  Per
 * element, each an IEEE binary32 operation, in this order, without fused
 * multiply-add (Kingma and Ba, Algorithm 1; the pages print no equations):
 *   g = fp32(grad16);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g)
 *   u = (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps);  master = master - lr*u
 *   param16 = fp16(master), rounded to nearest even
 * Non-finite values propagate per IEEE.
 * nonfinite_flag: NULL or a device int32; if any gradient of the plan is
 *   infinite or NaN, 1 is OR-ed into it (the library never clears it).
 * skip_if_nonzero: NULL or a device int32 read when the step starts; if
 *   it is nonzero the step reads and writes nothing (e.g. chain it to the
 *   flag of zero_reduce_grad_shard).  It must not be nonfinite_flag.
 * Asynchronous on `stream`; allocates nothing.  A plan must not be stepped
 * on two streams at once.  Errors: EINVAL (NULL plan or hp, bad
 * hyperparameters as zero_adam_scalars, flag == skip, plan made on another
 * device); EHIP.
 */
int zero_adam_step(const zero_plan *plan, const zero_adam_hparams *hp,
                   uint64_t t, int32_t *nonfinite_flag,
                   const int32_t *skip_if_nonzero, void *stream);

/*
 * Dynamic loss scale.  The pages do not treat loss scaling; they say that
 * fp16 loses gradient values below 2^-24 ([16B] "Why you can't just delete
 * the fp32 copies"), which a power-of-two factor on the loss, and so on
 * every gradient, keeps inside fp16's range.  The scale is 2^log2_scale.
 * Lives in device memory (16 bytes, 4-byte aligned); the caller writes the
 * initial value (e.g. {16, 0, 0, 0}) and afterwards only
 * zero_loss_scale_update changes it.
 */
typedef struct zero_loss_scale {
    int32_t log2_scale;     /* the gradients carry a factor 2^log2_scale   */
    uint32_t good_steps;    /* finite steps since the scale last changed   */
    uint32_t skipped_steps; /* steps skipped for a non-finite gradient     */
    uint32_t applied_steps; /* steps applied (both counts wrap at 2^32)    */
} zero_loss_scale;

#define ZERO_LOG2_SCALE_MAX 100 /* |log2_scale| bound: 2^-k stays normal fp32 */

/*
 * zero_adam_step_scaled -- zero_adam_step on gradients that carry the loss
 * scale *scale: each widened gradient is multiplied by 2^-log2_scale in fp32
 * before the update, so the step equals the unscaled step on the true
 * gradient wherever that is representable.  The product is exact for every
 * finite fp16 value.  bfloat16 has fp32's exponent range: there it is exact
 * only while it stays a normal fp32 number (log2_scale > 0 can push small
 * values into the subnormals or to zero; log2_scale < 0 can carry large
 * ones to infinity).  The non-finite flag tests the gradient after the
 * multiply, so such an overflow raises it.
 * log2_scale is read on the device when the step starts and clamped to
 * [-ZERO_LOG2_SCALE_MAX, ZERO_LOG2_SCALE_MAX].  Plans of either format.
 * A step skipped through skip_if_nonzero leaves everything unchanged; the
 * caller chooses t, so a caller that wants t to count applied steps reads
 * the flag (or applied_steps) before the next step.
 * scale: device pointer (required, 4-byte aligned, read only); no other
 *   argument may point into it.
 * Errors: those of zero_adam_step; EINVAL (NULL or misaligned scale, the
 * flag or skip pointer inside *scale).
 */
int zero_adam_step_scaled(const zero_plan *plan, const zero_adam_hparams *hp,
                          uint64_t t, const zero_loss_scale *scale,
                          int32_t *nonfinite_flag, const int32_t *skip_if_nonzero,
                          void *stream);

/*
 * zero_loss_scale_update -- one update of *scale after a step, from the
 * non-finite flag of that step's gradients, then the flag is set to 0 so
 * that the next step's kernels can OR into it again.  On the device, one
 * thread:
 *   flag != 0:  log2_scale = max(min_log2, log2_scale - 1); good_steps = 0;
 *               skipped_steps += 1
 *   flag == 0:  applied_steps += 1; good_steps += 1;
 *               if good_steps >= interval:
 *                   log2_scale = min(max_log2, log2_scale + 1); good_steps = 0
 * Used as: reduce (flag) -> zero_adam_step_scaled (skip = the same flag) ->
 * zero_loss_scale_update (flag), all on one stream.
 * scale, nonfinite_flag: device pointers, 4-byte aligned, not overlapping.
 * Asynchronous; allocates nothing.  Errors: EINVAL (NULL or misaligned
 * pointer, overlap, interval = 0, min_log2 > max_log2, either outside
 * [-ZERO_LOG2_SCALE_MAX, ZERO_LOG2_SCALE_MAX]); EHIP.
 */
int zero_loss_scale_update(zero_loss_scale *scale, int32_t *nonfinite_flag,
                           uint32_t interval, int32_t min_log2, int32_t max_log2,
                           void *stream);

/*
 * zero_reduce_grad_shard -- this rank's final gradient for its partition
 * from the nd ranks' fp16 slices of it: the reduce-scatter leaves every
 * rank with the summed gradient of its own partition only ([16B] "The part
 * that sounds too good: communication"; [ER10] "The Mathematics",
 * communication paragraph).  Here the nd slices are given in local device memory.
 *   out[i] = fp16( (s_0[i] + s_1[i] + ... + s_{nd-1}[i]) / nd )
 * summed in fp32 in rank order starting from s_0, one IEEE division by nd,
 * rounded to nearest even fp16.
 * slices_f16: host array of nd device pointers to n fp16 each (read only;
 *   copied into the launch, so the host array may be reused at once).
 * out_f16: device pointer to n fp16 (written); must not overlap a slice.
 * nonfinite_flag: NULL or a device int32; 1 is OR-ed into it if any output
 *   is infinite or NaN.
 * Asynchronous; allocates nothing.  n = 0 launches nothing.
 * Fastest with every slice 16-byte aligned at the same phase as out; with
 * out alone 1-3 elements out of the slices' phase (and n >= 1,024), the
 * slices keep their vector loads and out is stored shifted across lanes
 * (measured 0.77-0.78 of 8 TB/s against 0.64-0.66 element by element).
 * Slices spaced an exact power of two apart (256 MiB, say) read about a
 * fifth slower than with a few KiB more between them.  Slices that share
 * only an 8-byte phase with out (nd slices back to back in one buffer with
 * a slice length of 4 mod 8) take 8-byte groups at about 0.74-0.80 of
 * 8 TB/s over 8-64 slices, against 0.80-0.85 in a common 16-byte phase.
 * Errors: EINVAL (NULL arrays, nd = 0 or > ZERO_MAX_SLICES, a pointer not
 * 2-byte aligned, out overlapping a slice); EHIP.
 */
int zero_reduce_grad_shard(const void *const *slices_f16, uint32_t nd,
                           uint64_t n, void *out_f16, int32_t *nonfinite_flag,
                           void *stream);

/*
 * zero_reduce_grad_shard_bf16 -- zero_reduce_grad_shard for bfloat16
 * slices and output: the same fp32 sum in rank order and one division by
 * nd, rounded to the nearest bfloat16 (the bfloat16 variant of the ledger,
 * see zero_plan_create_bf16).  Arguments and errors as
 * zero_reduce_grad_shard.
 */
int zero_reduce_grad_shard_bf16(const void *const *slices_bf16, uint32_t nd,
                                uint64_t n, void *out_bf16, int32_t *nonfinite_flag,
                                void *stream);

/*
 * zero_reduce_adam_step -- the stage-2 step of one rank over a flat shard
 * in one pass: the reduction of zero_reduce_grad_shard followed by the
 * update of zero_adam_step, without storing and re-reading the fp16
 * gradient ([16B] "The part that sounds too good: communication": each
 * rank owns the final gradients of its partition and updates only its
 * slice).  Per element i:
 *   g16 = fp16((s_0[i] + ... + s_{nd-1}[i]) / nd)   as zero_reduce_grad_shard
 *   then the Adam element of zero_adam_step with g = fp32(g16)
 * so the results are bit-identical to the two calls in sequence (without
 * a skip input).  Below ZERO_FUSED_SPLIT_SLICES (16) slices one kernel
 * does it all, reading the slices and the fp32 state in one pass (4 bytes
 * per element less than the two calls); from there on, where its mix of state writes
 * into the slice reads costs more than it saves, the call runs the reduce
 * kernel and then the Adam kernel, with the fp16 gradient passing through
 * grad_out_f16, or without it through param_f16, which then holds the
 * gradient until the Adam kernel overwrites it with the new parameter.
 * The 16-bit outputs may be out of phase with the slices and the state (a
 * parameter view at an offset that is not a multiple of four elements):
 * from 1,024 elements both routes keep their vector loads and store them
 * shifted, and the Adam kernel reads a gradient held in param_f16 shifted.
 * slices_f16: host array of nd device pointers to n fp16 each (read only).
 * param_f16: n fp16, written.  master, m, v: n fp32 each, updated in place.
 * grad_out_f16: NULL, or n fp16 that receive g16.
 * nonfinite_flag: NULL or a device int32; 1 is OR-ed into it if any g16 is
 *   infinite or NaN.  There is no skip input: a single pass cannot know
 *   before writing that a later element is non-finite; such elements
 *   propagate per IEEE (use the two separate calls to skip a whole step).
 * Asynchronous on `stream`; allocates nothing.  n = 0 launches nothing.
 * Errors: EINVAL (NULL slices or hp, nd = 0 or > ZERO_MAX_SLICES, a NULL
 * or misaligned array (fp16: 2 bytes, fp32: 4 bytes), a written array
 * overlapping another array, bad hyperparameters as zero_adam_scalars);
 * EOVERFLOW; EHIP.
 */
int zero_reduce_adam_step(const void *const *slices_f16, uint32_t nd, uint64_t n,
                          void *param_f16, float *master, float *m, float *v,
                          void *grad_out_f16, const zero_adam_hparams *hp,
                          uint64_t t, int32_t *nonfinite_flag, void *stream);

/*
 * zero_reduce_adam_step_bf16 -- zero_reduce_adam_step with bfloat16
 * slices, parameter and gradient output (fp32 master, m, v as before): the
 * reduction of zero_reduce_grad_shard_bf16 followed by the update of
 * zero_adam_step over a zero_plan_create_bf16 plan, bit-identical to those
 * two calls in sequence ([DSZ] "Why parameter count is not training
 * memory": BF16 setups keep different states; the variant keeps the whole
 * 16-byte ledger).  Arguments, ownership and errors as
 * zero_reduce_adam_step.
 */
int zero_reduce_adam_step_bf16(const void *const *slices_bf16, uint32_t nd, uint64_t n,
                               void *param_bf16, float *master, float *m, float *v,
                               void *grad_out_bf16, const zero_adam_hparams *hp,
                               uint64_t t, int32_t *nonfinite_flag, void *stream);

/*
 * zero_gather_shards -- the receive side of the all-gather of updated fp16
 * parameters: after it every rank holds the whole fp16 buffer, rank r's
 * shard at element r * shard_len ([16B] "The part that sounds too good:
 * communication": after the update, every rank receives every other
 * rank's fresh fp16 shard).
 * Here the nd shards are given in local device memory:
 *   full[r * shard_len + i] = shards[r][i],  r < nd, i < shard_len
 * A shard whose pointer already equals full + r * shard_len (this rank's
 * own shard, when its parameter is a view into the full buffer) is left
 * where it is and not read.
 * shards_f16: host array of nd device pointers (read only; they may
 *   overlap each other; a shard not already in place must not overlap any
 *   part of full).  Fastest when full sits on a 128-byte line and
 *   shard_len is a multiple of 64 (every destination on a line); from
 *   1,024 elements a source out of its destination's 4-element phase is
 *   read as whole aligned 8-byte words (which may reach up to 3 elements
 *   past either end of the shard; those values are not used).
 * full_f16: device pointer to nd * shard_len fp16, written.
 * Asynchronous; allocates nothing.  shard_len = 0 launches nothing.
 * Errors: EINVAL (NULL arrays, nd = 0 or > ZERO_MAX_SLICES, a pointer not
 * 2-byte aligned, a shard that is not in place overlapping full); EOVERFLOW;
 * EHIP.
 */
int zero_gather_shards(const void *const *shards_f16, uint32_t nd, uint64_t shard_len,
                       void *full_f16, void *stream);

/*
 * zero_adam_step_host -- the Adam step of zero_adam_step computed by the
 * host CPU over host arrays: the update that ZeRO-Offload moves to the CPU
 * together with the fp32 state ([ER10] "The Breakthrough": the optimizer's
 * fp32 states and the update run in host RAM on the CPU; [DSZ] "Offload
 * trades capacity against movement").  Same per-element operations in the
 * same order as zero_adam_step, so the results are bit-identical.
 * grad_f16: n fp16 (read); param_f16: n fp16 (written); master, m, v: n fp32
 * each, updated in place; all host memory, borrowed.  threads: 0 for
 * min(16, CPUs the process may run on), else the number of threads to use, at most
 * 1024 (the calling thread is one of them).  nonfinite_flag: NULL or a host int32 that 1 is
 * OR-ed into if any gradient is infinite or NaN.  Synchronous.
 * Errors: EINVAL (NULL or misaligned arrays, written arrays overlapping,
 * threads above 1024, bad hyperparameters as zero_adam_scalars); EOVERFLOW;
 * ENOTSUP (no AVX2 or F16C); ENOMEM (threads could not start).
 */
int zero_adam_step_host(const void *grad_f16, void *param_f16, float *master, float *m,
                        float *v, uint64_t n, const zero_adam_hparams *hp, uint64_t t,
                        uint32_t threads, int32_t *nonfinite_flag);

/*
 * zero_adam_step_host_bf16 -- zero_adam_step_host with bfloat16 gradient and
 * parameter (the bfloat16 variant of the ledger): the gradient widened
 * exactly, the parameter rounded to the nearest bfloat16, ties to even (a
 * NaN stays a quiet NaN with its sign); bit-identical to zero_adam_step over
 * a zero_plan_create_bf16 plan, NaN payloads aside.  Arguments, ownership
 * and errors as zero_adam_step_host.
 */
int zero_adam_step_host_bf16(const void *grad_bf16, void *param_bf16, float *master, float *m,
                             float *v, uint64_t n, const zero_adam_hparams *hp, uint64_t t,
                             uint32_t threads, int32_t *nonfinite_flag);

/* Opaque ZeRO-Offload pipeline: pinned staging, two copy streams and the
 * host threads of the CPU update. */
typedef struct zero_offload zero_offload;

/* How an offload pipeline was set up (see zero_offload_describe). */
typedef struct zero_offload_info {
    uint32_t threads;     /* host threads of the update, the caller's included */
    int32_t numa_node;    /* the GPU's NUMA node as the host reports it; -1: unknown */
    uint32_t pinned_cpus; /* CPUs of that node the worker threads are pinned to;
                             0: not pinned (node unknown, or none of its CPUs
                             is in the process's affinity) */
    uint32_t reserved;
    uint64_t chunk_elems; /* elements per pipeline chunk */
} zero_offload_info;

/*
 * zero_offload_create -- set up the offload pipeline on the current device.
 * chunk_elems: elements per pipeline chunk (0: 4 Mi; else a multiple of 8,
 * at most 2^32); three chunks of fp16 gradients and three of fp16
 * parameters are staged in pinned host memory (hipHostMalloc, 12 bytes per
 * chunk element).  threads: 0 for min(16, CPUs available), else as
 * zero_adam_step_host.  Where the host reports the GPU's NUMA node
 * ([DSZ] "Offload trades capacity against movement": NUMA placement is one
 * of offload's costs), the worker threads are pinned to that node's CPUs
 * (within the process's affinity) and "CPUs available" counts those; the
 * caller should first-touch the fp32 master, m and v from that node too.
 * *out belongs to the caller until zero_offload_destroy.
 * Errors: EINVAL; ENOTSUP; ENOMEM; EHIP.
 */
int zero_offload_create(uint64_t chunk_elems, uint32_t threads, zero_offload **out);

/* zero_offload_describe -- the threads, NUMA placement and chunk of an
 * offload pipeline.  Host only.  Errors: EINVAL (NULL). */
int zero_offload_describe(const zero_offload *off, zero_offload_info *out);

/* zero_offload_destroy -- wait for its copies and free everything.  NULL is
 * accepted.  Errors: EHIP. */
int zero_offload_destroy(zero_offload *off);

/*
 * zero_offload_step -- one ZeRO-Offload step over an n-element shard: the
 * GPU keeps the fp16 parameters and gradients, the host keeps the fp32
 * master, m and v and runs the update ([ER10] "The Breakthrough", "The
 * Mathematics", the ZeRO-Offload paragraph).  The fp16 gradients go to the
 * host, zero_adam_step_host's update runs there, the fresh fp16 parameters
 * come back: 4 bytes per parameter over PCIe, pipelined in chunks so the
 * copies in both directions overlap the CPU work.
 * grad_f16, param_f16: device arrays of n fp16 (grad read, param written);
 *   the gradients are read once the work already enqueued on `stream` is
 *   done.
 * master, m, v: host arrays of n fp32, updated in place.
 * nonfinite_flag: NULL or a host int32 (as zero_adam_step_host).
 * Host-synchronous: returns after the last parameters have reached the
 * device (any later work on any stream sees them).  An offload object runs
 * one step at a time.  Results are bit-identical to zero_adam_step.
 * Errors: EINVAL (NULL, misaligned or overlapping arrays, offload made on
 * another device, bad hyperparameters); EOVERFLOW; EHIP.
 */
int zero_offload_step(zero_offload *off, const void *grad_f16, void *param_f16,
                      float *master, float *m, float *v, uint64_t n,
                      const zero_adam_hparams *hp, uint64_t t, int32_t *nonfinite_flag,
                      void *stream);

/*
 * zero_offload_step_bf16 -- zero_offload_step with bfloat16 gradient and
 * parameter on the device and the update of zero_adam_step_host_bf16 on the
 * host.  Arguments, ownership and errors as zero_offload_step.
 */
int zero_offload_step_bf16(zero_offload *off, const void *grad_bf16, void *param_bf16,
                           float *master, float *m, float *v, uint64_t n,
                           const zero_adam_hparams *hp, uint64_t t, int32_t *nonfinite_flag,
                           void *stream);

/* Limits of zero_adam_step_noalloc: the bytes of its per-device table array
 * (64 per non-empty tensor + 16 per chunk) and the tensors of one call. */
#define ZERO_NOALLOC_SCRATCH_BYTES (8u << 20)
#define ZERO_NOALLOC_MAX_TENSORS 1024u

/*
 * zero_adam_step_noalloc -- zero_adam_step over a list of fp16 tensors
 * without a plan, allocating nothing.  For callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.
 * The chunk table that zero_plan_create keeps in an allocation of its own
 * is instead rebuilt on the device at every call, in a fixed array of
 * ZERO_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on until the process ends: the tensors' descriptors travel as
 * kernel arguments (one small launch per 32 non-empty tensors), then the
 * Adam kernel of zero_adam_step runs over that table.  The update, the
 * flag and the skip are those of zero_adam_step, and the results are
 * bit-identical to zero_plan_create (chunk_elems = 0) followed by
 * zero_adam_step on the same tensors.
 * tensors: host array of n_tensors descriptors, as zero_plan_create (read
 *   during the call only).  hp, t, nonfinite_flag, skip_if_nonzero: as
 *   zero_adam_step.
 * The array is shared by every call on a device and keeps the last call's
 * table: calls that may overlap on one device (two streams, or two threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe.  No device, pinned or heap memory is allocated:
 * hipMalloc, hipFree and allocating library routines are never called
 * (the host bookkeeping, about 190 KB, is on the calling thread's stack).
 * The first call on a device takes the array's device address
 * (hipGetSymbolAddress) with that device current.
 * Asynchronous on `stream`.
 * Errors: ERANGE (more than ZERO_NOALLOC_MAX_TENSORS tensors, or a table
 * larger than ZERO_NOALLOC_SCRATCH_BYTES; zero_plan_describe's table_bytes
 * gives its size), checked before anything is enqueued; EINVAL and
 * EOVERFLOW as zero_plan_create and zero_adam_step; EHIP.
 */
int zero_adam_step_noalloc(const zero_tensor *tensors, uint32_t n_tensors,
                           const zero_adam_hparams *hp, uint64_t t, int32_t *nonfinite_flag,
                           const int32_t *skip_if_nonzero, void *stream);

/* zero_status_str -- static description of a status code. */
const char *zero_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
