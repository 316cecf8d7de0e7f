/*
 * zero_flat.h -- C ABI for one data-parallel rank's share of a ZeRO
 * mixed-precision Adam step on MI355X (gfx950).
 *
 * The interface follows the pages' statement of the problem (ZeRO reading
 * notes 026, §三 pseudocode): partition the parameter indices and assign an
 * owner to each; decide per stage what is sharded; bring each shard's gradient
 * to its owner; let each owner update its shard with its local optimizer
 * state; gather the updated parameters.
 *
 * Pages cited by short name:
 *   L18 notes         CMU 11-868 Lecture 18 notes, "Memory Optimization in Distributed Training: ZeRO" (semidirectx.com)
 *   026 notes         "026｜ZeRO：数据并行中，没必要让每张卡保存全部训练状态" (wq-win.github.io)
 *   L3.2              "L3.2 显存优化与 ZeRO" (yulong.wang)
 *   Illustrated ZeRO  "图解分布式训练（八）—— ZeRO 学习" (llm.jiangnianmeng.cn)
 *   ZeRO paper notes  "ZeRO:" paper notes (puzhiyuan.github.io)
 *
 * Conventions for every function
 * ------------------------------
 * - Return value: ZERO_OK (0) or a negative ZERO_E* code; zero_last_error()
 *   then holds a message for the calling thread.  Every argument is checked
 *   BEFORE anything is enqueued: on error nothing has been launched and no
 *   output has been touched (the pages' validate-then-act rule: L18 notes §5.1
 *   and §5.4; fail explicitly, never partially: 026 notes §五).  The only
 *   exceptions are failures that can first appear part-way through a call
 *   that streams data (a checkpoint block found corrupt, a copy refused by
 *   the runtime); those functions say which outputs are then unusable.
 * - Device buffers are owned by the caller (allocated with any allocator,
 *   e.g. PyTorch).  The library allocates no device memory; kernels that need
 *   scratch use the caller's workspace (zero_workspace_bytes), except
 *   zero_grad_norm_noalloc, whose scratch is a static device array.
 * - Device work is enqueued asynchronously on `stream` (a hipStream_t passed
 *   as void*; NULL = the null stream) on the current HIP device.  Results are
 *   valid once the stream reaches that point.  Calls are re-entrant; calls
 *   that share a workspace or flag must be ordered on one stream.  The step's
 *   calls record no memset and no host synchronisation, so they can be
 *   captured in a HIP graph, except the reduce and the gathers with more than
 *   64 ranks (their pointer table is copied from host memory; they return
 *   ZERO_EINVAL on a capturing stream).
 * - 16-bit data: ZERO_F16 (IEEE binary16) or ZERO_BF16.  Optimizer state is
 *   always fp32.  Element counts are int64; n = 0 is a no-op (where a device
 *   output is defined for n = 0, e.g. the norm, it is still written).
 * - Alignment: 16-bit pointers 2-byte aligned, fp32 pointers 4-byte aligned.
 *   Any offset works; 16-byte-aligned buffers take the vector path.
 * - Inputs may not overlap outputs (ZERO_EALIAS).
 * - Host arrays passed in (sizes, device pointers per rank) are read before
 *   the call returns; the caller may reuse or free them at once.
 * - A non-finite gradient is not an error: it is reported through the
 *   caller's int32 device flag and the Adam kernel then skips the step.
 */
#ifndef ZERO_FLAT_H
#define ZERO_FLAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK 0
#define ZERO_EINVAL (-1)  /* bad pointer, size, rank count, stage or dtype */
#define ZERO_EALIAS (-2)  /* an output overlaps an input or another output */
#define ZERO_EHIP (-3)    /* the HIP runtime refused a launch or copy */
#define ZERO_ENOMEM (-4)  /* host allocation for a plan failed */
#define ZERO_EIO (-5)     /* a checkpoint file is missing, short, corrupt or unwritable */

#define ZERO_F16 1
#define ZERO_BF16 2

#define ZERO_MAX_RANKS 1024

/* The most elements one call processes (n, or a unit's slice): 2^34.  A
 * launch's size per dimension is a 32-bit count of work-items, and at 2^34
 * elements the largest grid here (the reduce, 256 threads per 2048 elements)
 * is 2^31 work-items.  Larger sizes are rejected with ZERO_EINVAL; callers
 * split them into several calls. */
#define ZERO_MAX_ELEMS (INT64_C(1) << 34)

/* Bits of the int32 step flag (device memory, OR-ed by the kernels). */
#define ZERO_FLAG_NONFINITE_GRAD 1 /* an input or reduced gradient is inf/NaN */
#define ZERO_FLAG_NONFINITE_NORM 2 /* the sum of squares is not finite */
#define ZERO_FLAG_NO_CONSTS 4      /* zero_adam_step_owners: no table entry for the step */

/* ---------------------------------------------------------------------- */
/* a0: partition (host only, integer arithmetic)                           */
/* ---------------------------------------------------------------------- */

/* Opaque plan; created and destroyed on the host. */
typedef struct zero_plan zero_plan;

/* A piece of a named tensor that a rank owns. */
typedef struct {
    int64_t tensor;     /* index into the tensor list */
    int64_t tensor_off; /* first element of the piece inside the tensor */
    int64_t shard_off;  /* where the piece starts in the rank's shard */
    int64_t len;        /* elements */
} zero_segment;

/* A run of a restored shard: `len` elements at `new_offset` of the new shard
 * come from old owner `old_rank`'s shard at `old_offset`. */
typedef struct {
    int64_t old_rank;
    int64_t old_offset;
    int64_t new_offset;
    int64_t len;
} zero_reshard_segment;

/*
 * zero_plan_create -- flat-bucket partition of `n_units` units over `nd` ranks.
 *
 * Adam is elementwise, so rank r only needs the state of its own piece of
 * the flat parameter vector (L18 notes §2.1); the parameters are flattened
 * into one vector and cut into nd equal pieces, a tensor may straddle two
 * ranks (L18 notes §3.2, exercise 6).  ZeRO-3 flattens and splits per module
 * (Illustrated ZeRO §8.4).
 *
 * stage 0: plain data parallelism, one owner holds everything.
 * stage 1, 2: the units are concatenated into ONE flat unit.
 * stage 3: each unit (e.g. a layer) is partitioned separately.
 * Each unit of U elements gets slice s = roundup(ceil(U / owners), align);
 * rank r owns unit-local padded positions [r*s, (r+1)*s); positions >= U
 * are padding.  Units are laid out back to back in the padded full buffer,
 * and their slices back to back in every rank's shard.
 *
 * unit_numels: host array of n_units sizes >= 0 (sum > 0, at most 2^50);
 * 1 <= nd <= 1024; 1 <= align_elems <= 2^30; the padded layout (full_numel)
 * must stay within 2^52 elements.  On success *out receives a plan the caller
 * frees with zero_plan_destroy.  Errors: ZERO_EINVAL, ZERO_ENOMEM.
 */
int zero_plan_create(const int64_t* unit_numels, int n_units, int nd, int stage,
                     int64_t align_elems, zero_plan** out);
void zero_plan_destroy(zero_plan* plan);

/* Number of units after merging (1 for stages 0-2) and number of owners. */
int zero_plan_info(const zero_plan* plan, int* n_units, int* owners, int* nd, int* stage);

/* Per-rank shard length (padded, the same for every rank) and the real
 * (non-padding) elements rank `rank` owns. */
int zero_plan_rank(const zero_plan* plan, int rank, int64_t* shard_numel, int64_t* real_numel);

/* Unit `unit`: real size, slice per owner, base in the padded full buffer,
 * base inside every shard. */
int zero_plan_unit(const zero_plan* plan, int unit, int64_t* numel, int64_t* slice_numel,
                   int64_t* full_base, int64_t* shard_base);

/* Padded length of the full gather buffer. */
int zero_plan_full_numel(const zero_plan* plan, int64_t* padded);

/*
 * zero_plan_segments -- the pieces of named tensors rank `rank` owns, in shard
 * order.  Tensors (host array of n_tensors sizes) fill the plan's units back to
 * back; for stage 3 a tensor may not cross a unit.  Writes at most `cap`
 * segments to `out` and the total number to *count (call with cap = 0 to
 * size the array).  Errors: ZERO_EINVAL (sizes do not fill the units).
 */
int zero_plan_segments(const zero_plan* plan, const int64_t* tensor_numels, int n_tensors,
                       int rank, zero_segment* out, int cap, int* count);

/* ---------------------------------------------------------------------- */
/* Accounting (host only)                                                  */
/* ---------------------------------------------------------------------- */

/*
 * Per-rank model-state bytes for psi parameters: stage 0 (4+K)psi, stage 1
 * 4psi + K psi/nd, stage 2 2psi + (2+K)psi/nd, stage 3 (4+K)psi/nd, with K
 * optimizer bytes per parameter (12 for fp32 master + m + v).  L18 notes
 * §1.2, §2.1; L3.2 §2.3.
 */
int zero_model_state_bytes(double psi, int nd, int stage, int k_bytes, double* out);

/* Elements one rank sends per step: 2psi (stages 0-2) or 3psi (stage 3), each
 * times (nd-1)/nd.  L18 notes §3.1; ZeRO paper notes 0x07. */
int zero_comm_volume(double psi, int nd, int stage, double* elems_sent);

/* ---------------------------------------------------------------------- */
/* Workspace                                                               */
/* ---------------------------------------------------------------------- */

/*
 * Bytes of device workspace for `n_sets` partial-sum sets over shards of n
 * elements.  The workspace holds a table of up to ZERO_MAX_RANKS device
 * pointers, 1024 second-level fp64 sums for the norm, and per set the fp64
 * sums of squares of one reduce (or partials) launch (one per 2048 elements).  The caller allocates it (any alignment >= 8) and passes it to
 * zero_reduce_shard / zero_grad_norm / zero_gather_params; its contents need no
 * initialisation.  Returns -1 on bad arguments.
 */
int64_t zero_workspace_bytes(int64_t n, int n_sets);

/* ---------------------------------------------------------------------- */
/* a1: local half of the reduce-scatter                                    */
/* ---------------------------------------------------------------------- */

/*
 * zero_reduce_shard -- the owner's averaged gradient slice.
 *
 * The owner receives the AVERAGE gradient of its slice (L18 notes §2.2 step 3;
 * ZeRO paper notes 0x05 §5.2), summed in a fixed rank order (L18 notes §2.5):
 *   acc = f32(c_0[i]); acc += f32(c_r[i]) for r = 1..nd-1   (fp32, no FMA)
 *   reduced_out[i] = round_to_nearest_even_16(acc / nd)
 * The loss scale stays in the stored value.  Fused into the same pass:
 *   - per-block fp64 sums of (f32(reduced_out[i]) * inv_loss_scale)^2 into
 *     workspace set `set` (consumed by zero_grad_norm);
 *   - *flag |= ZERO_FLAG_NONFINITE_GRAD if any c_r[i] or reduced_out[i] is
 *     inf/NaN.  The flag is OR-ed, never cleared: zero it once per step.
 *
 * contribs: HOST array of nd device pointers, each to n 16-bit values of
 *   `dtype` (rank 0 first).  1 <= nd <= 1024.
 * reduced_out: device, n values of `dtype`.  It may be exactly one of the
 *   contributions (the reduce in place, as a rank keeps the reduced slice in
 *   its own gradient buffer: each element is read from every rank before it
 *   is written); otherwise it may not overlap any contribution.
 * inv_loss_scale: a positive power of two (1 when no loss scaling).
 * workspace / workspace_bytes: >= zero_workspace_bytes(n, set + 1).
 * flag: device int32.
 */
int zero_reduce_shard(const void* const* contribs, int nd, int64_t n, int dtype,
                      float inv_loss_scale, void* reduced_out, void* workspace,
                      int64_t workspace_bytes, int set, int32_t* flag, void* stream);

/*
 * zero_reduce_owners -- zero_reduce_shard for `owners` emulated owners in one
 * launch, as when every rank of a data-parallel group is emulated on one GPU
 * (L18 notes §2.5, the 4-card simulation; the reduce-scatter's local half for
 * each owner, §2.2 step 3).  Owner o's contribution from rank r starts
 * o * contrib_stride elements past contribs[r]; its output starts
 * o * reduced_stride elements past reduced_out; its partial sums go to
 * workspace set o.  The result equals `owners` calls of zero_reduce_shard
 * with set = o, bit for bit.
 *
 * 1 <= owners <= 1024; with owners > 1, 0 <= contrib_stride <= 2^40 and
 * n <= reduced_stride <= 2^40 (owners' outputs do not overlap).  In place
 * as for zero_reduce_shard: reduced_out == contribs[k] with reduced_stride ==
 * contrib_stride.  Strides
 * that are multiples of 4 keep the vector path.  workspace_bytes >=
 * zero_workspace_bytes(n, owners).  Other arguments and errors as
 * zero_reduce_shard.
 */
int zero_reduce_owners(const void* const* contribs, int nd, int64_t n, int owners,
                       int64_t contrib_stride, int dtype, float inv_loss_scale, void* reduced_out,
                       int64_t reduced_stride, void* workspace, int64_t workspace_bytes,
                       int32_t* flag, void* stream);

/* ---------------------------------------------------------------------- */
/* a2: global gradient norm and clip coefficient                           */
/* ---------------------------------------------------------------------- */

/*
 * zero_grad_norm -- L2 norm over the flat gradient and the clip multiplier
 * (L18 notes §1.4; L3.2 §4.2 gradient_clipping).
 *
 * If `grad` is not NULL, first a partials pass over grad[0..n) (16-bit,
 * `dtype`) writes set 0 of the workspace (as zero_reduce_shard would) and ORs
 * ZERO_FLAG_NONFINITE_GRAD into *flag for inf/NaN -- this is the path for an
 * already-reduced gradient.  Then one block sums, in fp64 and in a fixed order,
 * sets 0..n_sets-1 of the workspace (set-major, the order the ranks were
 * reduced in) followed by extra_sumsq[0..n_extra) (device fp64, e.g. other
 * ranks' sums; may be NULL when n_extra = 0):
 *   norm = sqrt(sumsq)
 *   coef = (float)min(1, max_norm / (norm + 1e-6))   (fp64; max_norm <= 0: 1)
 * If the sum is not finite, *flag |= ZERO_FLAG_NONFINITE_NORM.  norm_out
 * (device fp64) and coef_out (device fp32) are always written.  The result is
 * bitwise repeatable: the summation tree depends only on n and n_sets.
 *
 * n is the per-set shard length used by the producing launches; 1 <= n_sets.
 * With n = 0 no partial sum is read (they are all zero) and grad may be NULL
 * or not: norm = sqrt(sum of extra_sumsq).
 */
int zero_grad_norm(const void* grad, int64_t n, int dtype, float inv_loss_scale,
                   void* workspace, int64_t workspace_bytes, int n_sets,
                   const double* extra_sumsq, int n_extra, float max_norm, int32_t* flag,
                   double* norm_out, float* coef_out, void* stream);

/* Largest n of zero_grad_norm_noalloc, and the size of its static scratch. */
#define ZERO_NOALLOC_MAX_ELEMS (INT64_C(1) << 34)
#define ZERO_NOALLOC_SCRATCH_BYTES (16384 + 8 * (ZERO_NOALLOC_MAX_ELEMS / 2048))

/*
 * zero_grad_norm_noalloc -- zero_grad_norm on an already-reduced gradient
 * (grad not NULL, one set), for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Instead of a caller's workspace it uses a static device array
 * of ZERO_NOALLOC_SCRATCH_BYTES (about 64 MiB) that each GPU the library runs
 * on holds until the process ends; the call itself allocates nothing.  Same
 * kernels, same summation tree, so norm_out, coef_out and the flag are
 * bitwise those of zero_grad_norm with n_sets = 1.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * partial sums (nothing in it needs clearing: each call writes every partial
 * it reads).  Calls that overlap on one GPU -- on different streams, or from
 * different threads -- race; order them on one stream.  The first call on a
 * device resolves the array's address on that device (hipGetSymbolAddress,
 * with that device current); make it outside graph capture.
 *
 * grad: device 16-bit (`dtype`), n; 0 <= n <= ZERO_NOALLOC_MAX_ELEMS.  Other
 * arguments and errors as zero_grad_norm (ZERO_EINVAL for a NULL grad or a
 * larger n, before anything is enqueued).
 */
int zero_grad_norm_noalloc(const void* grad, int64_t n, int dtype, float inv_loss_scale,
                           const double* extra_sumsq, int n_extra, float max_norm, int32_t* flag,
                           double* norm_out, float* coef_out, void* stream);

/* ---------------------------------------------------------------------- */
/* a3: fused Adam(W) on the owned fp32 state, writing the 16-bit parameter */
/* ---------------------------------------------------------------------- */

typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;   /* decoupled (AdamW); 0 = plain Adam */
    float inv_loss_scale; /* positive power of two */
    int64_t step;         /* t >= 1; bias corrections f32(1 - beta^t) from fp64 */
} zero_adam_hparams;

/*
 * zero_adam_step -- the owner updates its fp32 variance, momentum and master,
 * then copies the master to the 16-bit parameter (L18 notes §2.2 step 4;
 * Adam is elementwise, §2.1).  Per element, in fp64 from the fp32 state, the
 * 16-bit gradient and the fp32 scalars of zero_adam_consts_fill, one IEEE
 * fp64 rounding per operation in this order, no fused multiply-add,
 * correctly rounded division and square root:
 *   g  = f64(grad[i]) * (inv_loss_scale * (*coef_dev))   (the product is exact)
 *   m' = beta1*m + (1 - beta1)*g
 *   v' = beta2*v + (1 - beta2)*(g*g)
 *   p' = p - lr * ((m' / bc1) / (sqrt(v' / bc2) + eps) + weight_decay*p)
 *   m, v, p = f32(m'), f32(v'), f32(p')                  (one rounding each)
 *   param_out[i] = round_to_nearest_even_16(p)
 * This is the unsharded data-parallel update itself (L18 notes §2.5: the
 * sharded run computes what data parallelism computes), so the results do
 * not depend on how the vector is sharded.  zero_cpu_adam_step evaluates the
 * same sequence, so the two give identical bits.  master, m and v are each
 * read once and written once.  If *flag != 0 the kernel writes nothing (the
 * step is skipped).
 *
 * master, m, v: device fp32, n each, distinct.  grad: device 16-bit
 * (`grad_dtype`), n.  coef_dev: device fp32 (from zero_grad_norm).  flag:
 * device int32.  param_out: device 16-bit (`param_dtype`), n -- typically the
 * full gather buffer plus this rank's offset, so the cast lands in place.
 */
int zero_adam_step(float* master, float* m, float* v, const void* grad, int grad_dtype,
                   int64_t n, const zero_adam_hparams* hp, const float* coef_dev,
                   const int32_t* flag, void* param_out, int param_dtype, void* stream);

/* The fp32 scalars of one AdamW step, as zero_adam_step derives them from
 * zero_adam_hparams: 1 - beta and the bias corrections bc = 1 - beta^t, each
 * formed in fp64 and rounded to fp32. */
typedef struct {
    float lr, beta1, beta2, one_minus_beta1, one_minus_beta2, eps, weight_decay, inv_loss_scale;
    float bias_corr1, bias_corr2;
} zero_adam_consts;

/* Fills *out (host) from hp, with zero_adam_step's checks.  Errors: ZERO_EINVAL. */
int zero_adam_consts_fill(const zero_adam_hparams* hp, zero_adam_consts* out);

/*
 * zero_adam_step_consts -- zero_adam_step with its scalars read from device
 * memory (consts_dev: a zero_adam_consts filled by zero_adam_consts_fill and
 * copied to the device, 4-byte aligned), so a launch captured in a HIP graph
 * replays with the step count, learning rate and bias corrections the caller
 * writes there before each replay.  The same kernel and the same bits as
 * zero_adam_step for the same scalars.  The values in consts_dev are not
 * validated at launch.  Other arguments and errors as zero_adam_step.
 */
int zero_adam_step_consts(float* master, float* m, float* v, const void* grad, int grad_dtype,
                          int64_t n, const zero_adam_consts* consts_dev, const float* coef_dev,
                          const int32_t* flag, void* param_out, int param_dtype, void* stream);

/*
 * The device side of a step sequence: the step count t of the next update,
 * kept in device memory so that steps (and captured graph replays) need no
 * host round trip, and advanced only by applied steps -- a step skipped for
 * a non-finite gradient leaves t, and so the bias corrections, unchanged.
 * Initialise it on the device as {step = first t (>= 1), 0, 0, table_t0, 0, 0}.
 */
typedef struct {
    int64_t step;       /* t of the next update, >= 1 */
    int64_t applied;    /* steps applied */
    int64_t skipped;    /* steps skipped (a set flag) */
    int64_t table_t0;   /* the step of entry 0 of the scalars table */
    int32_t last_flag;  /* the flag of the last step that ended */
    int32_t reserved;
} zero_step_state;

/*
 * zero_adam_step_owners -- zero_adam_step for `owners` emulated owners in one
 * launch (L18 notes §2.5; each owner updates its own slice, §2.2 step 4),
 * with the step's scalars chosen on the device: entry
 * state_dev->step - state_dev->table_t0 of table_dev, a device array of
 * table_len zero_adam_consts (from zero_adam_consts_fill for consecutive
 * steps).  If that index is outside the table, or *flag != 0, nothing is
 * written; the former also sets ZERO_FLAG_NO_CONSTS in *flag.  Owner o's
 * master, m and v start o * state_stride elements past master, m and v, its
 * gradient o * grad_stride past grad, its 16-bit output o * param_stride
 * past param_out.  The same kernel and bits as zero_adam_step.
 *
 * 1 <= owners <= 1024; with owners > 1, n <= state_stride, param_stride <=
 * 2^40 and 0 <= grad_stride <= 2^40.  1 <= table_len <= 2^31.  state_dev:
 * device, 8-byte aligned.  flag: device int32 (written only as above).
 * Other arguments and errors as zero_adam_step.
 */
int zero_adam_step_owners(float* master, float* m, float* v, int64_t state_stride,
                          const void* grad, int grad_dtype, int64_t grad_stride, int64_t n,
                          int owners, const zero_adam_consts* table_dev, int64_t table_len,
                          const zero_step_state* state_dev, const float* coef_dev, int32_t* flag,
                          void* param_out, int64_t param_stride, int param_dtype, void* stream);

/*
 * zero_step_end -- closes a step on the device (one thread): records *flag in
 * state_dev->last_flag; if it is 0 the step was applied and step and applied
 * advance by one, otherwise skipped does; then *flag is cleared for the next
 * step.  Enqueue it after the step's last AdamW call.  Errors: ZERO_EINVAL
 * (NULL or misaligned), ZERO_EALIAS, ZERO_EHIP.
 */
int zero_step_end(int32_t* flag, zero_step_state* state_dev, void* stream);

/* ---------------------------------------------------------------------- */
/* a4: gather of 16-bit shards into the full parameter buffer              */
/* ---------------------------------------------------------------------- */

/*
 * zero_gather_params -- all-gather of the updated 16-bit slices (L18 notes
 * §2.2 step 5), unit by unit: ZeRO-3 gathers one module's parameters into a
 * contiguous buffer (Illustrated ZeRO §8.4).  A pure copy, for every unit u in
 * [unit_begin, unit_end) and owner r:
 *   full[full_base_u + r*s_u + j] = shards[r][shard_base_u + j],  j < s_u
 * shards: HOST array of `owners` device pointers (plan's owner count), each
 * to shard_numel 16-bit values.  full: device, plan's padded full length.
 * workspace: >= zero_workspace_bytes(0, 0) bytes (holds the pointer table
 * when there are more than 64 owners; may be NULL otherwise).
 */
int zero_gather_params(const zero_plan* plan, const void* const* shards, int unit_begin,
                       int unit_end, int dtype, void* full, void* workspace,
                       int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Block-quantised parameter gather (ZeRO++ quantised weights)             */
/* ---------------------------------------------------------------------- */

/*
 * ZeRO++ sends the ZeRO-3 parameter all-gather in low precision, with one
 * scale per block of values because one scale per tensor lets a few large
 * values stretch it (L18 notes §4.5: INT8 11.25% vs 0.89% error, INT4 98.69%
 * vs 14.53%, for one scale per tensor vs per 256 values).
 *
 * Format: blocks of ZERO_QBLOCK consecutive elements (the last may be short).
 * scale = max|x| / qmax in fp32 (qmax 127 for 8 bits, 7 for 4 bits; a block of
 * zeros has scale 0); code = clamp(round_half_even(x / scale), -qmax, qmax)
 * with x the fp32 value of the 16-bit input and IEEE fp32 division.  8-bit
 * codes are int8, one byte per element; 4-bit codes are two's complement
 * nibbles, two per byte, the even element in the low nibble (the high nibble
 * of a final odd byte is 0).  Dequantised value = round-to-nearest-even into
 * 16 bits of fp32(code * scale).  Inputs must be finite: a non-finite value
 * gives its block unspecified codes.
 */
#define ZERO_QBLOCK 256

/* Code bytes for n elements (n for 8 bits, ceil(n / 2) for 4 bits) and the
 * number of fp32 scales (ceil(n / ZERO_QBLOCK)); -1 on bad arguments. */
int64_t zero_quant_code_bytes(int64_t n, int bits);
int64_t zero_quant_scale_count(int64_t n);

/*
 * zero_quantize_blocks -- x[0..n) (16-bit, `dtype`, device, 8-byte aligned)
 * -> codes (device, zero_quant_code_bytes(n, bits) bytes, 4-byte aligned) and
 * scales (device fp32, zero_quant_scale_count(n), 4-byte aligned).  bits is 8
 * or 4.  Outputs may not overlap the input or each other.
 */
int zero_quantize_blocks(const void* x, int dtype, int64_t n, int bits, void* codes, float* scales,
                         void* stream);

/*
 * zero_dequantize_blocks -- codes and scales as written by
 * zero_quantize_blocks -> y[0..n) (16-bit, `dtype`, device, 8-byte aligned).
 */
int zero_dequantize_blocks(const void* codes, const float* scales, int64_t n, int bits, void* y,
                           int dtype, void* stream);

/*
 * zero_gather_dequant -- the receiving side of a quantised all-gather, fused
 * with dequantisation: for every unit u in [unit_begin, unit_end), owner r and
 * j < s_u,
 *   full[full_base_u + r*s_u + j] = dequant(code_shards[r], scale_shards[r],
 *                                           shard_base_u + j)
 * where code_shards[r] / scale_shards[r] hold owner r's whole shard quantised
 * with zero_quantize_blocks.  The plan's align must be a multiple of
 * ZERO_QBLOCK so blocks never straddle units or owners.  code_shards and
 * scale_shards are HOST arrays of `owners` device pointers (codes 16-byte
 * aligned, scales 4-byte aligned); full is the padded full 16-bit buffer,
 * 16-byte aligned (device allocations are).  workspace: >= zero_workspace_bytes(0, 0) bytes when there
 * are more than 64 owners (pointer tables), else may be NULL.
 */
int zero_gather_dequant(const zero_plan* plan, const void* const* code_shards,
                        const float* const* scale_shards, int unit_begin, int unit_end, int bits,
                        int dtype, void* full, void* workspace, int64_t workspace_bytes,
                        void* stream);

/* ---------------------------------------------------------------------- */
/* Sharded checkpoints and restoring under another partition               */
/* ---------------------------------------------------------------------- */

/* Where the arrays of a checkpoint call live. */
#define ZERO_LOC_DEVICE 0
#define ZERO_LOC_HOST 1 /* e.g. ZeRO-Offload's host-resident state */

/* Elements per checksummed block of a checkpoint array (1 MiB of fp32), and
 * the smallest staging buffer the checkpoint calls accept (two blocks). */
#define ZERO_CKPT_BLOCK 262144
#define ZERO_CKPT_MIN_STAGING (2 * 4 * ZERO_CKPT_BLOCK)

/*
 * zero_plan_reshard -- restoring sharded state under another partition has to
 * re-own it while keeping the parameter order and which moment belongs to
 * which parameter (026 notes §五).  The flat parameter order (units
 * concatenated) identifies a parameter, so rank `new_rank`'s shard under
 * `new_plan` is filled by maximal runs copied from the shards of `old_plan`,
 * in new-shard order; positions in no run are padding (zero).  The plans may
 * differ in Nd, stage, units and align but must partition the same number of
 * parameters.  Writes at most `cap` runs and the total to *count (cap = 0 to
 * size the array).  Errors: ZERO_EINVAL (NULL, rank, parameter counts).
 */
int zero_plan_reshard(const zero_plan* old_plan, const zero_plan* new_plan, int new_rank,
                      zero_reshard_segment* out, int cap, int* count);

/*
 * zero_ckpt_save -- writes rank `rank`'s optimizer state (master, m, v: fp32,
 * the plan's shard_numel each, padding included) and the plan to one file per
 * rank, so a restore can rebuild the old partition (026 notes §五; L3.2 §4.3:
 * a resumable checkpoint holds the sharded optimizer state, not only the
 * weights).  Layout: a 4 KiB-aligned header (magic, version, Nd, stage,
 * align, rank, step, the unit sizes, one 64-bit checksum per 1 MiB block of
 * each array), then the three arrays.  The file is written under a
 * temporary name unique to the process and call (`path`.tmp.<pid>.<n>),
 * flushed to stable storage and renamed (and the directory flushed), so
 * `path` never names a partial file; of two saves to one path, the later
 * rename wins.  `location`: ZERO_LOC_DEVICE
 * (arrays in device memory, copied out through `staging` on `stream`) or
 * ZERO_LOC_HOST.  staging: pinned host memory, >= ZERO_CKPT_MIN_STAGING
 * bytes, 64-byte aligned.  Blocks until the file is complete.  Errors:
 * ZERO_EINVAL, ZERO_EIO (with the path and the system's reason), ZERO_EHIP.
 */
int zero_ckpt_save(const char* path, const zero_plan* plan, int rank, int64_t step,
                   const float* master, const float* m, const float* v, int location,
                   void* staging, int64_t staging_bytes, void* stream);

/*
 * zero_ckpt_load -- restores rank `rank`'s shard under `plan` from the files
 * of ALL ranks of a saved run (paths[i] is old rank i's file, n_paths the old
 * owner count).  Every file must exist and agree (the same run, step, plan
 * and parameter count as `plan`), whether or not this rank reads from it, so a
 * missing or foreign file fails explicitly instead of yielding an incomplete
 * model.  The runs of zero_plan_reshard are read block by block; every block
 * read is checked against its stored checksum; positions in no run are set to
 * zero.  master, m, v: the plan's shard_numel fp32 each, in `location`.
 * *step_out: the saved step count.  staging as for zero_ckpt_save.  Blocks
 * until the state is in place.  Errors: ZERO_EIO (missing, short or corrupt
 * file, naming its rank and path), ZERO_EINVAL (mismatched files or plans,
 * arguments), ZERO_EHIP.  Missing, foreign, truncated and mismatched files
 * are found before any output is written; a corrupt block or a failed read
 * or copy is found while copying, and master, m and v are then partly
 * written and must not be used.
 */
int zero_ckpt_load(const char* const* paths, int n_paths, const zero_plan* plan, int rank,
                   float* master, float* m, float* v, int location, int64_t* step_out,
                   void* staging, int64_t staging_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* CPU-offloaded optimizer (ZeRO-Offload)                                  */
/* ---------------------------------------------------------------------- */

/* Instruction sets of the host AdamW (zero_cpu_isa / zero_cpu_set_isa). */
#define ZERO_CPU_SCALAR 0
#define ZERO_CPU_AVX2 1   /* AVX2 + F16C, 4 fp64 lanes per instruction */
#define ZERO_CPU_AVX512 2 /* AVX-512 F/BW/VL + F16C, 8 fp64 lanes per instruction */

/* Minimum size of the pinned staging buffer of zero_offload_adam_step. */
#define ZERO_OFFLOAD_MIN_STAGING 576

/*
 * zero_cpu_adam_step -- the AdamW update of zero_adam_step on HOST memory, for
 * ZeRO-Offload, which keeps the fp32 master, m and v (12 bytes per parameter)
 * in host memory and updates them with a multi-threaded, vectorised CPU Adam
 * (L18 notes §4.4).  The fp64 evaluation of zero_adam_step, operation for
 * operation, with coef in place of *coef_dev, so it gives the GPU kernel's
 * bits; the result does not depend on n_threads or on the instruction set.
 * The threads persist across calls (one pool for the process).
 *
 * master, m, v: host fp32, n each, distinct, 4-byte aligned.  grad: host
 * 16-bit (`grad_dtype`), n.  param_out: host 16-bit (`param_dtype`), n.  coef:
 * the clip multiplier (finite, > 0).  skip != 0 writes nothing (a non-finite
 * gradient).  n_threads in [1, 256]: the range is cut into that many
 * contiguous parts (fewer for small n); the call returns when all are done.
 */
int zero_cpu_adam_step(float* master, float* m, float* v, const void* grad, int grad_dtype,
                       int64_t n, const zero_adam_hparams* hp, float coef, int skip,
                       void* param_out, int param_dtype, int n_threads);

/*
 * zero_offload_adam_step -- one ZeRO-Offload update of an owned slice: the
 * reduced 16-bit gradient goes from the GPU to the host, the host AdamW
 * updates the host fp32 state, and the 16-bit parameters go back (2 bytes
 * each way per parameter; L18 notes §4.4).  The work is cut into chunks that
 * fit the staging buffer; the copy of the next chunk's gradient overlaps the
 * update of the current one, and its parameters are copied back while the
 * next chunk is updated.  The clip multiplier and the skip flag are read
 * from the device first (zero_grad_norm's outputs); a set flag moves nothing.
 *
 * master, m, v: host fp32, n each.  grad_dev: device 16-bit, n.  coef_dev,
 * flag_dev: device fp32 / int32.  param_dev: device 16-bit, n.  staging:
 * host memory allocated pinned (hipHostMalloc), 64-byte aligned, at least
 * ZERO_OFFLOAD_MIN_STAGING bytes; (staging_bytes - 64) / 8 values per chunk.
 * Blocks the calling thread until the last parameters have reached the
 * device (the stream is synchronised).  Errors: ZERO_EINVAL (arguments, or a
 * non-positive clip multiplier on the device), ZERO_EALIAS, ZERO_EHIP.  The
 * clip multiplier is checked before any state changes; a copy refused by the
 * runtime part-way leaves master, m, v and the parameters partly updated.
 */
int zero_offload_adam_step(float* master, float* m, float* v, const void* grad_dev,
                           int grad_dtype, int64_t n, const zero_adam_hparams* hp,
                           const float* coef_dev, const int32_t* flag_dev, void* param_dev,
                           int param_dtype, void* staging, int64_t staging_bytes, int n_threads,
                           void* stream);

/*
 * The one-step-delayed update of ZeRO-Offload (L18 notes §4.4: the CPU's
 * update of step t runs while the GPU already works on step t+1, so step
 * t+1's forward and backward see the parameters of step t-1).  A
 * zero_offload handle owns persistent host worker threads for the host
 * AdamW.  Per step t, after its reduce and norm are enqueued:
 *   zero_offload_end(step t-1)   -- waits for the update of step t-1 and
 *                                   enqueues the copy of its 16-bit
 *                                   parameters into param_dev;
 *   zero_offload_begin(step t)   -- brings step t's clip multiplier and flag
 *                                   to the host, copies its reduced gradient
 *                                   aside on the device and returns; a thread
 *                                   of the handle then streams that copy
 *                                   through the host AdamW chunk by chunk (as
 *                                   zero_offload_adam_step does), on a stream
 *                                   of its own;
 * so the GPU runs step t+1's reduce and norm while the host updates.  The
 * updates are those of zero_cpu_adam_step, in the same order, so the state
 * after any step equals the undelayed sequence bit for bit; only the
 * parameters the device holds lag by one step.
 *
 * zero_offload_create: n_threads in [1, 256] workers.  Errors: ZERO_EINVAL,
 * ZERO_ENOMEM.  zero_offload_destroy waits for an update in flight, then
 * frees the handle (the parameters of that update are dropped).
 */
typedef struct zero_offload zero_offload;

int zero_offload_create(int n_threads, zero_offload** out);
void zero_offload_destroy(zero_offload* h);

/*
 * zero_offload_begin -- starts the update of one step.  On `stream` it copies
 * *coef_dev and *flag_dev to the host and waits for them; a set flag (or
 * n = 0) starts nothing.  Otherwise it enqueues a device copy of
 * grad_dev[0..n) into the first 2n bytes of device_buffer (so the caller
 * may overwrite grad_dev in later stream work) and returns; the update
 * collects its 16-bit parameters in the next 2n bytes.
 *
 * master, m, v: host fp32, n each, distinct, updated in place.  staging:
 * pinned host memory as for zero_offload_adam_step.  device_buffer:
 * caller-owned device memory, >= 4n bytes, not overlapping grad_dev.  Until
 * the matching zero_offload_end returns, the caller must not touch master,
 * m, v, staging or device_buffer.  hp: as zero_cpu_adam_step.
 * 0 <= n <= 2^34.  Errors (nothing started): ZERO_EINVAL (arguments; an
 * update begun and not ended; a clip multiplier that is not finite and
 * positive), ZERO_EALIAS, ZERO_EHIP.
 */
int zero_offload_begin(zero_offload* h, float* master, float* m, float* v, const void* grad_dev,
                       int grad_dtype, int64_t n, const zero_adam_hparams* hp,
                       const float* coef_dev, const int32_t* flag_dev, int param_dtype,
                       void* device_buffer, int64_t device_bytes, void* staging,
                       int64_t staging_bytes, void* stream);

/*
 * zero_offload_end -- finishes the update begun last: waits for its host
 * AdamW and copies, then enqueues on `stream` the device copy of its 16-bit
 * parameters (param_dtype of the begin call, n values) into param_dev.
 * *applied (if not NULL) is 1 if the step was applied, 0 if it was skipped
 * (nothing moves).  Errors: ZERO_EINVAL (no update begun; param_dev NULL or
 * misaligned when the step was applied), ZERO_EALIAS (param_dev overlaps the
 * begin call's device_buffer), ZERO_EHIP (including a copy or launch refused
 * while the update was in flight: master, m and v are then partly updated).
 * After ZERO_EINVAL or ZERO_EALIAS the update is still in flight: call again.
 */
int zero_offload_end(zero_offload* h, void* param_dev, int* applied, void* stream);

/* The host AdamW's instruction set in use (ZERO_CPU_*). */
int zero_cpu_isa(void);

/* Use a lower instruction set than detected (for tests); EINVAL if the CPU
 * lacks it. */
int zero_cpu_set_isa(int isa);

/* ---------------------------------------------------------------------- */
/* Misc                                                                    */
/* ---------------------------------------------------------------------- */

/* Message for the last error on the calling thread ("" if none). */
const char* zero_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int zero_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_FLAT_H */
