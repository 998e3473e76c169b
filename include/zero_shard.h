/*
 * zero_shard.h -- C ABI of one ZeRO data-parallel rank's partitioned
 * mixed-precision Adam step (P_os+g), for AMD Instinct MI355X (gfx950).
 *
 * Sources for what is computed:
 *  - ZeRO method entry (Sharded Data Parallel Methods catalogue),
 *    description: model states are partitioned across the data-parallel
 *    processes instead of replicated.
 *  - Explainer "Data Parallelism Without the Copies" of the paper "ZeRO:
 *    Memory Optimizations Toward Training Trillion Parameter Models":
 *    section "The 16 Bytes per Parameter Audit" (fp16 weight, fp32 master,
 *    two fp32 Adam moments per parameter); Ch.02 "The Three Stages" (what
 *    P_os, P_os+g and P_os+g+p shard); Ch.05 "Super-Linear Scaling" (stage
 *    table).
 *  The pages give no update formula.  The steps implemented are dynamic loss
 *  scaling with inf/NaN skip (Micikevicius et al. 2018), global max-norm
 *  clipping (Pascanu et al. 2013; coefficient min(1, max/(norm + 1e-6))),
 *  bias-corrected Adam (Kingma & Ba 2015, eps outside the square root) with
 *  decoupled weight decay scaled by the learning rate (Loshchilov & Hutter
 *  2019), and round-to-nearest-even writeback of the 16-bit parameter copy.
 *
 * The step's contract is eight calls: zero_partition_plan and
 * zero_rank_fragments (the plan), zero_norm_workspace_bytes and
 * zero_shard_unscale_norm_overflow (steps 1-2), zero_shard_adam_step (steps
 * 3-4), zero_loss_scaler_update (the scalar decision), zero_status_string and
 * zero_last_error.  They allocate nothing and keep no state besides the
 * thread-local error string.  Every other call is an extra on the same
 * kernels, marked where it is declared:
 *  - the same step with its coefficients or its scaler state in caller-owned
 *    device memory (zero_adam_prepare, *_coef, *_dev, zero_step_decide_dev,
 *    zero_shard_norm_decide_dev) and the norm pass without a workspace
 *    (zero_shard_unscale_norm_overflow_noalloc, which uses a fixed array the
 *    library keeps on each GPU);
 *  - recorded step graphs (zero_step_graph_*), which ALLOCATE at create;
 *  - the rows around the step: fp32 gradient accumulation, the reduction of
 *    the ranks' gradient slices, the copy-and-norm pass, the combine of the
 *    ranks' scalars, and the step on host cores (whose worker threads start
 *    on first use and live until the process ends);
 *  - physically contiguous memory (zero_device_alloc_contiguous, zero_pool_*),
 *    whose purpose is to allocate, and the measurement copies
 *    (zero_copy_reference, zero_copy_widen_reference on the device,
 *    zero_cpu_copy_reference on the host).
 *
 * Conventions for every function:
 *  - Returns an int status: ZERO_OK (0) or a negative zero_status (the
 *    pool allocator pair excepted, whose signatures torch fixes).  Nothing
 *    throws.  On error a detail string is available from zero_last_error()
 *    (thread-local, valid until the next call on the same thread).
 *  - An invalid argument is detected on the host before anything is
 *    enqueued: on error no device work has been queued.
 *  - Device functions only enqueue work on `hip_stream` (a hipStream_t; NULL
 *    is the default stream) and return; results are valid once the stream
 *    has reached that point.  They never synchronize and never allocate,
 *    except the step-graph calls, which say where they do, and the memory
 *    calls near the end of this header, whose purpose is to allocate.
 *  - The caller owns every host array and device buffer.  Device pointers
 *    must point to device memory of the current HIP device and be 16-byte
 *    aligned (ZERO_EALIGN otherwise).
 *  - Sizes are element counts in int64; n = 0 is a valid no-op.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_SHARD_ABI_VERSION 1

typedef enum {
    ZERO_OK = 0,
    ZERO_EINVAL = -1,   /* bad argument (null pointer, n < 0, unknown dtype, ...) */
    ZERO_EALIGN = -2,   /* device pointer not 16-byte aligned */
    ZERO_ERANGE = -3,   /* a size overflows int64 or a kernel limit */
    ZERO_ENOSPC = -4,   /* caller's output array or workspace too small */
    ZERO_EHIP = -5      /* HIP runtime reported an error at launch */
} zero_status;

/* Floating-point formats.  ZERO_F16 / ZERO_BF16: 16-bit gradient or
 * parameter copy.  ZERO_F32: an fp32 gradient (the accumulation buffer of
 * zero_shard_grad_accumulate), accepted as grad_dtype by
 * zero_shard_unscale_norm_overflow and zero_shard_adam_step. */
enum { ZERO_F16 = 1, ZERO_BF16 = 2, ZERO_F32 = 3 };

/* Returns ZERO_SHARD_ABI_VERSION of the built library. */
int zero_abi_version(void);

/* ---------------------------------------------------------------------------
 * Partition plan (host only, integer arithmetic).
 *
 * ZeRO method entry, description; explainer, History ("ZeRO":
 * partition-and-all-gather) and "The 16 Bytes per Parameter Audit": every
 * rank owns one partition of the flattened model state.  Layout: tensors end
 * to end in list order with no gaps, the flat buffer padded at its end to
 * padded_total = n_d * S where S = align * ceil(T / (n_d * align)) and T is
 * the total element count; rank r owns flat range [r*S, (r+1)*S).
 *
 *  dims      all tensors' dimensions concatenated (int64, each >= 0);
 *            may be NULL if the sum of ndims is 0
 *  ndims     ndims[i] = number of dimensions of tensor i (0 = scalar, one
 *            element); NULL allowed only if n_tensors == 0
 *  n_tensors >= 0
 *  n_d       data-parallel degree, >= 1
 *  align     partition size granularity in elements, >= 1
 *  tensor_offsets  out, [n_tensors] flat start of each tensor (may be NULL
 *            if n_tensors == 0)
 *  partition_numel out, S;  padded_total  out, n_d * S
 * Errors: ZERO_EINVAL (null/negative), ZERO_ERANGE (int64 overflow).
 * ------------------------------------------------------------------------- */
int zero_partition_plan(const int64_t* dims, const int32_t* ndims, int32_t n_tensors,
                        int32_t n_d, int64_t align, int64_t* tensor_offsets,
                        int64_t* partition_numel, int64_t* padded_total);

/* One nonempty intersection of a tensor with a rank's partition: elements
 * [tensor_begin, tensor_begin + numel) of tensor `tensor` (row-major flat
 * index) sit at [shard_begin, shard_begin + numel) of the rank's shard. */
typedef struct {
    int32_t tensor;
    int32_t reserved;       /* 0 */
    int64_t tensor_begin;
    int64_t shard_begin;
    int64_t numel;
} zero_fragment;

/* Fragments of rank `rank` in list order.  Writes min(count, capacity)
 * entries to `out` (may be NULL when capacity == 0) and the required count
 * to *count; returns ZERO_ENOSPC if capacity < required (then *count still
 * holds the required count).  Other arguments as zero_partition_plan. */
int zero_rank_fragments(const int64_t* dims, const int32_t* ndims, int32_t n_tensors,
                        int32_t n_d, int64_t align, int32_t rank, zero_fragment* out,
                        int32_t capacity, int32_t* count);

/* ---------------------------------------------------------------------------
 * Step 1+2: unscale, inf/NaN detection, squared L2 norm of one gradient shard.
 * Contract call.
 *
 * Passages: the gradient shard is the 2-byte gradient of mixed-precision
 * Adam's per-parameter state (explainer, "The 16 Bytes per Parameter Audit";
 * Ch.02 "The Three Stages", memory per parameter), and under P_os+g each rank
 * holds only its partition of it (Ch.02, what each stage shards).  The pages
 * name mixed precision but not loss scaling or clipping: unscaling by the
 * loss scale with an inf/NaN skip follows Micikevicius et al. 2018, the
 * squared norm feeds max-norm clipping (Pascanu et al. 2013).
 *
 *  grad        device, [n] values of format grad_dtype: 16-bit raw bits
 *              (ZERO_F16, ZERO_BF16) or fp32 (ZERO_F32)
 *  inv_loss_scale  1 / loss scale (> 0, finite)
 *  d_sqnorm    device, out: one double = sum_i (grad_i * inv_loss_scale)^2
 *              (+inf if the shard holds an inf and no NaN, NaN if it holds
 *              a NaN).  Each square is exact in float64; the sum is taken
 *              in float64 in a fixed order that depends only on n, so the
 *              result is bit-identical from run to run.
 *  d_overflow  device, out: one int32, 1 if any element is +-inf or NaN
 *              (tested on the exponent bits, never inferred from the norm),
 *              else 0
 *  d_workspace device scratch of at least zero_norm_workspace_bytes(n)
 *              bytes (no initial contents needed; clobbered)
 * The grad shard is only read.  Two kernels are enqueued (block partials,
 * then a one-block fixed-order combine).  For n == 0 the outputs are
 * written as 0 by one small kernel.  The workspace, d_sqnorm and d_overflow
 * must not overlap one another, and the workspace must not overlap grad
 * (ZERO_EINVAL).
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ENOSPC (workspace), ZERO_ERANGE,
 * ZERO_EHIP.
 * ------------------------------------------------------------------------- */
size_t zero_norm_workspace_bytes(int64_t n);

int zero_shard_unscale_norm_overflow(const void* grad, int32_t grad_dtype, int64_t n,
                                     double inv_loss_scale, double* d_sqnorm,
                                     int32_t* d_overflow, void* d_workspace,
                                     size_t workspace_bytes, void* hip_stream);

/* zero_shard_unscale_norm_overflow without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The norm pass's block
 * partials live in a fixed 8 KiB array in device memory that the library
 * holds on each GPU until the process ends; the pass needs at most 6 KiB of
 * it for any n (ZERO_ENOSPC otherwise).  Same kernels, grid and results as
 * zero_shard_unscale_norm_overflow, bit for bit.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race and may return
 * wrong results.  Nothing needs clearing between calls.  The first call on a
 * device, with that device current, looks up the array's address there
 * (no allocation).  Arguments and errors as zero_shard_unscale_norm_overflow,
 * all checked before the device is touched. */
int zero_shard_unscale_norm_overflow_noalloc(const void* grad, int32_t grad_dtype, int64_t n,
                                             double inv_loss_scale, double* d_sqnorm,
                                             int32_t* d_overflow, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Steps 3+4: fused Adam/AdamW update of one shard and 16-bit writeback.
 * Contract call.
 *
 * Passages: each rank updates the fp32 master, momentum and variance of its
 * own partition only and writes the 2-byte weight copy of it (ZeRO method
 * entry, description; explainer, "The 16 Bytes per Parameter Audit" and
 * Ch.02 "The Three Stages", memory per parameter and what each stage shards;
 * History, "The mixed-precision era").  The update rule, which the pages do
 * not print, is bias-corrected Adam (Kingma & Ba 2015) with decoupled weight
 * decay (Loshchilov & Hutter 2019).
 *
 * Hyperparameters are double; the host derives the per-step float32
 * coefficients from them in double and rounds each once.  `step` is the
 * 1-based index t of the step being applied (bias corrections 1 - beta^t).
 * max_grad_norm <= 0 disables clipping.
 * ------------------------------------------------------------------------- */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;
    double inv_loss_scale, max_grad_norm;
} zero_adam_params;

/*  master, exp_avg, exp_avg_sq  device, [n] float32, updated in place
 *  grad        device, [n] gradient of format grad_dtype (16-bit, or fp32
 *              for an accumulated gradient, which is passed already unscaled
 *              with inv_loss_scale = 1), read only
 *  param_out   device, [n] 16-bit parameter copy (param_dtype) written as
 *              round-to-nearest-even of the new float32 master; NULL skips
 *              the writeback.  For the ZeRO-2 layout pass the rank's slice
 *              (offset r*S) of the full flat parameter buffer; for ZeRO-3 a
 *              shard-local buffer.
 *  d_global_sqnorm  device double: the data-parallel sum of every rank's
 *              d_sqnorm; read by the kernel to form the clip coefficient
 *              min(1, max/(sqrt(sq) + 1e-6)) in double.  May be NULL only
 *              when clipping is disabled.
 *  d_global_overflow  device int32: the OR of every rank's d_overflow.  If
 *              nonzero when the kernel runs, the kernel writes nothing at all
 *              (skipped step).  NULL: never skip.
 * Per element (float32): g = grad * gscale with gscale = float(inv_scale *
 * coef); m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*g^2;
 * p = p*(1 - lr*wd) - (lr/(1-b1^t)) * m / (sqrt(v)/sqrt(1-b2^t) + eps).
 * Exactly, with every operation rounded once to float32 (IEEE, nearest
 * even; fma(a, b, c) = a*b + c with one rounding; sqrt and / correctly
 * rounded) and the coefficients B1 = float(b1), O1 = float(1 - b1),
 * B2 = float(b2), O2 = float(1 - b2), SS = float(lr / (1 - b1^t)),
 * RB = float(1 / sqrt(1 - b2^t)), E = float(eps), D = float(1 - lr*wd)
 * formed in double (b^t by binary exponentiation: r = 1; while t: if t odd,
 * r = r*b; b = b*b; t = t/2):
 *     g = raw * gscale;  m = fma(B1, m, O1*g);  v = fma(B2, v, (O2*g)*g);
 *     d = fma(sqrt(v), RB, E);  p = fma(p, D, -((SS*m) / d)),
 * where coef = max_grad_norm / (sqrt(global sum of squares) + 1e-6) in
 * double, taken as 1 unless it is below 1 (clipping off: coef = 1).  The
 * results are reproducible bit for bit from this description.
 * Streams 28 bytes per element (2 grad + 3x4 read, 3x4 write + 2 param;
 * 30 with an fp32 gradient).
 * grad must not alias master, exp_avg, exp_avg_sq or param_out, and
 * d_global_sqnorm / d_global_overflow must not lie in any of those four
 * (every workgroup reads them while others write the shard): ZERO_EINVAL.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
int zero_shard_adam_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                         int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                         const zero_adam_params* hp, const double* d_global_sqnorm,
                         const int32_t* d_global_overflow, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Coefficients in device memory, and recorded step graphs.  Extras: the
 * coefficient block in device memory, and graphs that allocate at create.
 *
 * zero_adam_prepare writes the per-step coefficient block that
 * zero_shard_adam_step derives from hp (zero_adam_coef_bytes() bytes of
 * plain data; the same validation and errors) into host memory at coef_out.
 * zero_shard_adam_step_coef is zero_shard_adam_step with that block read
 * from device memory d_coef (8-byte aligned) when the kernel runs, so a
 * recorded launch can be replayed with new coefficients; d_global_sqnorm is
 * required.  Every workgroup reads d_coef while others write the shard, so
 * it must not lie in master, exp_avg, exp_avg_sq or param_out (the caller's
 * responsibility: unlike the norm and flag, it is not checked).
 *
 * A step graph records, once, on its own stream: the copy of the coefficient
 * block from pinned host memory, the norm pass (as
 * zero_shard_unscale_norm_overflow with the given inv_loss_scale, outputs
 * d_sqnorm / d_overflow, workspace d_workspace), the fused update (as
 * zero_shard_adam_step_coef, skip and clip from d_overflow / d_sqnorm) and
 * the copy of the overflow flag back to pinned host memory.  Launching
 * replays it on hip_stream: one graph launch and one event record per step
 * instead of four separate calls.  Meant for small shards, where launch
 * overhead dominates.  The step computed is the one defined above for
 * zero_shard_unscale_norm_overflow and zero_shard_adam_step (same passages).
 *  create   records the graph for these buffers and this loss scale.  It
 *           ALLOCATES (pinned host blocks, a device coefficient block, an
 *           event, the graph); destroy frees them.  Buffers must outlive it.
 *  launch   waits for the previous replay, writes hp's coefficients into the
 *           pinned block, replays.  hp->inv_loss_scale must equal the
 *           recorded one (ZERO_EINVAL otherwise: record a new graph when the
 *           loss scale changes).
 *  overflow waits for the last replay and returns its overflow flag.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ENOSPC, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
size_t zero_adam_coef_bytes(void);
int zero_adam_prepare(const zero_adam_params* hp, void* coef_out);
int zero_shard_adam_step_coef(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                              int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                              const void* d_coef, const double* d_global_sqnorm,
                              const int32_t* d_global_overflow, void* hip_stream);

typedef struct zero_step_graph zero_step_graph;
int zero_step_graph_create(zero_step_graph** out, float* master, float* exp_avg, float* exp_avg_sq,
                           const void* grad, int32_t grad_dtype, void* param_out, int32_t param_dtype,
                           int64_t n, double inv_loss_scale, double* d_sqnorm, int32_t* d_overflow,
                           void* d_workspace, size_t workspace_bytes);
int zero_step_graph_launch(zero_step_graph* g, const zero_adam_params* hp, void* hip_stream);
int zero_step_graph_overflow(zero_step_graph* g, int32_t* overflow);
int zero_step_graph_destroy(zero_step_graph* g);

/* ---------------------------------------------------------------------------
 * Gradient accumulation into an fp32 copy (explainer, Ch.02 "The Three
 * Stages", memory per parameter: an fp16 gradient plus its fp32 copy).
 * Extra: the fp32-accumulation row around the step.
 * For each micro-batch:  acc = (first ? 0 : acc) + grad * inv_loss_scale,
 * in fp32 with one rounding per element (fused multiply-add).
 *
 *  acc         device, [n] float32, updated in place (not read when first)
 *  grad        device, [n] 16-bit micro-batch gradient (ZERO_F16/ZERO_BF16)
 *  inv_loss_scale  1 / loss scale of this micro-batch (> 0, finite)
 *  first       nonzero for the first micro-batch of a step
 *  d_overflow  device int32 or NULL: set to 1 if this micro-batch holds an
 *              inf/NaN; never cleared by the library (the caller zeroes it
 *              when it wants a per-step flag).  Not needed for skipping: an
 *              inf/NaN propagates into acc, and the norm pass over acc
 *              (grad_dtype ZERO_F32) reports it.  Must not lie in acc.
 * Streams 10 bytes per element (6 for the first micro-batch).
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
int zero_shard_grad_accumulate(float* acc, const void* grad, int32_t grad_dtype, int64_t n,
                               double inv_loss_scale, int32_t first, int32_t* d_overflow,
                               void* hip_stream);

/* ---------------------------------------------------------------------------
 * Reduction of this partition's gradient over the data-parallel ranks: the
 * local half of a gradient reduce-scatter (extra: a row around the step).
 * Plain data parallelism sums the ranks' gradients (explainer, History,
 * "Data parallelism's reign"); once
 * gradients are partitioned each rank keeps the reduced gradient of its own
 * partition only (explainer, Ch.02 "The Three Stages", what each stage shards,
 * and the stage table: reduce-scatter).  A direct reduce-scatter delivers the
 * K ranks' 16-bit gradients of this partition into K buffers on this GPU;
 * this call sums them, in slice order, into the fp32 gradient copy:
 *     acc = g_0 * inv,   then  acc = acc + g_k * inv  for k = 1 .. K-1,
 * in fp32 with one rounding per addition (fused multiply-add): bit-identical
 * to zero_shard_grad_accumulate over the slices in order.  A mean instead of
 * a sum is inv_loss_scale / K.  The step then runs on acc (grad_dtype
 * ZERO_F32), as after accumulation.
 *
 *  acc        device, [n] float32, written (not read); must not overlap a slice
 *  slices     host array of n_slices device pointers, each [n] 16-bit
 *             gradient of grad_dtype (ZERO_F16/ZERO_BF16), 16-byte aligned;
 *             slices may alias one another
 *  n_slices   K, 1 <= K <= ZERO_MAX_SLICES
 *  inv_loss_scale  1 / loss scale (> 0, finite)
 *  d_overflow device int32 or NULL: set to 1 if any slice holds an inf/NaN;
 *             never cleared by the library; must not lie in acc
 * Streams 2K + 4 bytes per element.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
#define ZERO_MAX_SLICES 16
int zero_shard_grad_reduce(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                           int64_t n, double inv_loss_scale, int32_t* d_overflow, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Extra: the same step on host cores, for optimizer states kept in host
 * memory (the CPU-offload lineage: explainer, Legacy, "The trillion-parameter
 * claim";
 * glossary description, CPU offloading).  All pointers are HOST pointers
 * (pinned or pageable); the calls are synchronous and return when done.
 * They compute what the device entry points compute, from the same per-step
 * coefficients: the AdamW update in the float32 operation order documented
 * for zero_shard_adam_step (fused multiply-adds included), so a host step
 * and a device step from the same state, gradient and global norm agree bit
 * for bit; the norm with float64 partials:
 *
 * zero_cpu_shard_unscale_norm_overflow: *sqnorm = sum (grad * inv)^2 over
 *   [0, n), summed in float64 per 65536-element chunk and then in chunk
 *   order, so the result is identical for any thread count; *overflow = 1 if
 *   any element is inf/NaN.  grad_dtype ZERO_F16, ZERO_BF16 or ZERO_F32.
 * zero_cpu_shard_adam_step: the fused AdamW update of master/exp_avg/
 *   exp_avg_sq in place and the 16-bit parameter writeback (param_out may be
 *   NULL, any 2-byte alignment), with the data-parallel-reduced norm and flag
 *   passed by value; global_overflow != 0 leaves every buffer untouched.  The
 *   parameter copy is written with streaming (non-temporal) stores, so its
 *   lines are not read first, and the stores are fenced before the call
 *   returns.
 * nthreads <= 0 uses every hardware thread.  Buffers must not overlap.
 * Errors: ZERO_EINVAL, ZERO_ERANGE.
 * ------------------------------------------------------------------------- */
int zero_cpu_shard_unscale_norm_overflow(const void* grad, int32_t grad_dtype, int64_t n,
                                         double inv_loss_scale, double* sqnorm, int32_t* overflow,
                                         int32_t nthreads);

int zero_cpu_shard_adam_step(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                             int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                             const zero_adam_params* hp, double global_sqnorm,
                             int32_t global_overflow, int32_t nthreads);

/* Extra, a measurement aid for the host step: a plain copy of `bytes` (a
 * multiple of 4) from src to dst in host memory, cut into the same chunks and
 * run on the same worker threads, with the same vectorized (ordinary) stores
 * as the host AdamW loop's fp32 streams: the achievable rate of one read and
 * one write stream on the host cores.  Synchronous; host pointers, not overlapping; nthreads as
 * above.  Errors: ZERO_EINVAL. */
int zero_cpu_copy_reference(void* dst, const void* src, int64_t bytes, int32_t nthreads);

/* ---------------------------------------------------------------------------
 * Step 2 (scalar, host): dynamic loss scale update after a step.  Contract
 * call.  Passage: the pages name mixed-precision (fp16) training
 * (explainer, History, "The mixed-precision era") but not its loss scaling;
 * the dynamic scale with back-off on overflow and growth after a run of clean
 * steps follows Micikevicius et al. 2018.
 * On overflow: *skip_out = 1, scale = max(scale*backoff, min_scale),
 * good_steps = 0.  Otherwise *skip_out = 0, good_steps += 1 and, when it
 * reaches growth_interval, scale *= growth and good_steps = 0.
 * backoff = growth = 1 gives a static scale.  The caller advances its step
 * counter t only when *skip_out == 0.
 * Errors: ZERO_EINVAL (null, scale <= 0, min_scale <= 0, backoff or growth
 * <= 0, growth_interval < 1).
 * ------------------------------------------------------------------------- */
typedef struct {
    double scale, min_scale, backoff, growth;
    int64_t growth_interval, good_steps;
} zero_loss_scaler;

int zero_loss_scaler_update(zero_loss_scaler* s, int32_t overflow, int32_t* skip_out);

/* ---------------------------------------------------------------------------
 * The step with its scalar state in device memory: no host round trip.
 * Extras: the contract's steps with the scaler state in caller-owned device
 * memory.
 *
 * The loss scaler and the step counts live in a zero_step_state in device
 * memory.  The norm pass reads the loss scale from it; a one-thread kernel,
 * enqueued by zero_shard_adam_step_dev after the global overflow flag is
 * known, forms the coefficient block of step t = applied + 1 at that scale
 * (the same routine as zero_adam_prepare, bit for bit) and then advances the
 * state exactly as zero_loss_scaler_update does (skip: scale backed off,
 * skipped + 1; otherwise applied + 1 and growth after growth_interval clean
 * steps).  A whole step is therefore enqueued without waiting for the
 * device; the host reads the state back only when it wants to.  Same
 * passages as the norm pass, the update and the loss scaler above.
 *
 * zero_step_state: 72 bytes, device memory, 8-byte aligned, initialised by
 * the caller (a valid scaler as for zero_loss_scaler_update; applied = the
 * steps already applied; skipped, last_overflow, reserved = 0).
 *
 * zero_shard_unscale_norm_overflow_dev: zero_shard_unscale_norm_overflow
 *   with inv_loss_scale = 1/scale read from d_state when the kernel runs
 *   (1 for a ZERO_F32 gradient, which is already unscaled).
 * zero_shard_norm_decide_dev: the norm pass of a single rank, whose flag is
 *   the global one (no data-parallel reduction in between): its final
 *   one-block kernel also makes the decision (as zero_step_decide_dev,
 *   writing d_coef and advancing d_state); zero_shard_adam_step_coef with
 *   d_coef follows.  Saves the decision kernel's launch.
 * zero_step_decide_dev: the decision kernel alone: writes the coefficient
 *   block to d_coef (device scratch of zero_adam_coef_bytes() bytes, 8-byte
 *   aligned, owned by the caller) and advances d_state from
 *   d_global_overflow.  grad_dtype ZERO_F32 (an already unscaled copy)
 *   forms the block with inv_loss_scale 1.
 * zero_shard_adam_step_dev: zero_step_decide_dev, then the fused update
 *   (zero_shard_adam_step_coef with d_coef).  d_global_overflow is required;
 *   d_global_sqnorm when clipping.  With n = 0 the state still advances.
 * zero_shard_grad_accumulate_dev / zero_shard_grad_reduce_dev: the
 *   accumulation and reduction with inv_loss_scale = 1/scale from d_state.
 * In a data-parallel job every rank holds its own copy of the state; since
 * all ranks see the same global overflow flag, the copies stay identical.
 * Calls on one state must be ordered on one stream.  The state and d_coef
 * must not lie in any buffer the same call writes (not checked).
 * Errors: as the host-scaled calls, plus ZERO_EINVAL / ZERO_EALIGN for the
 * state pointer.
 * ------------------------------------------------------------------------- */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    double max_grad_norm;          /* <= 0 disables clipping */
} zero_adam_hyper;

typedef struct {
    zero_loss_scaler scaler;
    int64_t applied;               /* steps applied so far; the next step has t = applied + 1 */
    int64_t skipped;               /* steps skipped on overflow so far */
    int32_t last_overflow;         /* the last step's global overflow flag */
    int32_t reserved;
} zero_step_state;

int zero_shard_unscale_norm_overflow_dev(const void* grad, int32_t grad_dtype, int64_t n,
                                         const zero_step_state* d_state, double* d_sqnorm, int32_t* d_overflow,
                                         void* d_workspace, size_t workspace_bytes, void* hip_stream);
int zero_shard_norm_decide_dev(const void* grad, int32_t grad_dtype, int64_t n, const zero_adam_hyper* hp,
                               zero_step_state* d_state, double* d_sqnorm, int32_t* d_overflow, void* d_coef,
                               void* d_workspace, size_t workspace_bytes, void* hip_stream);
int zero_step_decide_dev(const zero_adam_hyper* hp, int32_t grad_dtype, zero_step_state* d_state,
                         const int32_t* d_global_overflow, void* d_coef, void* hip_stream);
int zero_shard_adam_step_dev(float* master, float* exp_avg, float* exp_avg_sq, const void* grad,
                             int32_t grad_dtype, void* param_out, int32_t param_dtype, int64_t n,
                             const zero_adam_hyper* hp, zero_step_state* d_state,
                             const double* d_global_sqnorm, const int32_t* d_global_overflow, void* d_coef,
                             void* hip_stream);
int zero_shard_grad_accumulate_dev(float* acc, const void* grad, int32_t grad_dtype, int64_t n,
                                   const zero_step_state* d_state, int32_t first, int32_t* d_overflow,
                                   void* hip_stream);
int zero_shard_grad_reduce_dev(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                               int64_t n, const zero_step_state* d_state, int32_t* d_overflow, void* hip_stream);

/* A recorded step with device state: zero_shard_norm_decide_dev then
 * zero_shard_adam_step_coef on these buffers, captured once as a HIP graph
 * (kernels only: no host blocks, no copies).  Each launch replays one whole
 * step of one rank; the loss scale, t and the skip come from d_state, so
 * nothing changes between replays and no launch waits.  The hyperparameters
 * are recorded with the graph (record a new one when they change).
 * create ALLOCATES (the graph and an event); destroy frees them and waits for
 * the last replay.  zero_step_graph_launch / _overflow reject such a graph,
 * and zero_step_graph_launch_dev rejects the host-coefficient kind.
 * Errors: as zero_shard_norm_decide_dev and zero_shard_adam_step_coef, plus
 * ZERO_EHIP from capture or launch. */
int zero_step_graph_create_dev(zero_step_graph** out, float* master, float* exp_avg, float* exp_avg_sq,
                               const void* grad, int32_t grad_dtype, void* param_out, int32_t param_dtype,
                               int64_t n, const zero_adam_hyper* hp, zero_step_state* d_state, double* d_sqnorm,
                               int32_t* d_overflow, void* d_coef, void* d_workspace, size_t workspace_bytes);
int zero_step_graph_launch_dev(zero_step_graph* g, void* hip_stream);

/* ---------------------------------------------------------------------------
 * The fp32 gradient copy and its norm in one pass (fp32 accumulation and the
 * local half of the reduce-scatter above, fused with the norm pass).  Extra.
 *
 * zero_shard_grad_sum_norm writes
 *     acc = (add_to_acc ? acc : 0) + sum_k slices[k] * inv_loss_scale,
 * slice by slice with one fp32 rounding per addition (bit-identical to
 * zero_shard_grad_reduce, or to zero_shard_grad_accumulate for one slice),
 * and in the same pass the squared L2 norm and the inf/NaN flag of the
 * result: *d_sqnorm = sum acc^2 (the copy is already unscaled), *d_overflow
 * = 1 if any element of acc is inf or NaN (it then equals +inf or NaN, as
 * the norm pass reports).  This replaces the norm pass over the copy (4
 * bytes per element).  Use it for the reduction of K ranks' slices
 * (add_to_acc = 0) or for the last micro-batch of an accumulation
 * (add_to_acc = 1 after the first, one slice).
 * The norm is summed in fp64, per one-wave task of 256 elements, then over
 * tasks and blocks in a fixed order: deterministic, but summed in another
 * order than the norm pass, so its last bits may differ from it.
 *  d_workspace  device scratch of zero_sum_norm_workspace_bytes(n) bytes,
 *               16-byte aligned (about n/32 bytes), overlapping neither acc,
 *               a slice, d_sqnorm nor d_overflow; d_sqnorm and d_overflow
 *               must not overlap each other or lie in acc
 * zero_shard_grad_sum_norm_dev: the same with inv_loss_scale = 1/scale
 *   read from d_state; with hp given (one rank, whose flag is the global
 *   one) its final kernel also makes the step's decision into d_coef, as
 *   zero_shard_norm_decide_dev does; with hp NULL the caller runs
 *   zero_step_decide_dev after the data-parallel reduction.
 * Streams 2K + 4 bytes per element (2K + 8 with add_to_acc).
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_ENOSPC, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
size_t zero_sum_norm_workspace_bytes(int64_t n);
int zero_shard_grad_sum_norm(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                             int64_t n, int32_t add_to_acc, double inv_loss_scale, double* d_sqnorm,
                             int32_t* d_overflow, void* d_workspace, size_t workspace_bytes, void* hip_stream);
int zero_shard_grad_sum_norm_dev(float* acc, const void* const* slices, int32_t n_slices, int32_t grad_dtype,
                                 int64_t n, int32_t add_to_acc, const zero_adam_hyper* hp,
                                 zero_step_state* d_state, double* d_sqnorm, int32_t* d_overflow, void* d_coef,
                                 void* d_workspace, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Extra, a measurement aid (not a step of the method): a plain device copy, one
 * 16-byte vector per lane, in the same streaming style as the step's kernels.
 * Its rate is the achievable rate of one read plus one write stream, which
 * the step's kernels are reported against beside the nominal HBM peak.
 * Async on hip_stream.  dst, src: device, 16-byte aligned, not overlapping;
 * bytes: a multiple of 16 (0 is a no-op), any size (one launch; past 64 GiB
 * its lanes loop).
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
int zero_copy_reference(void* dst, const void* src, int64_t bytes, void* hip_stream);

/* Extra, a measurement aid: the widening copy.  Reads src_bytes (a multiple
 * of 8) and writes 2 * src_bytes: each 8-byte word of src lands twice, as one
 * 16-byte vector of dst.  8 bytes read and 16 written per lane, the access
 * pattern of the first micro-batch's accumulation (2 bytes read, 4 written
 * per element), whose achievable rate it measures.  dst, src: device,
 * 16-byte aligned, not overlapping; async on hip_stream.
 * Errors: ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_EHIP. */
int zero_copy_widen_reference(void* dst, const void* src, int64_t src_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * The local half of the all-reduce of the norm pass's two scalars: the one
 * exchange inside the step (extra: a row around the step).  Each rank
 * updates only its own partition (ZeRO method entry, description;
 * explainer, Ch.02 "The Three Stages", what each
 * stage shards), while the clip coefficient and the skip depend on the whole
 * gradient: the data-parallel sum of the ranks' sums of squares and the OR of
 * their inf/NaN flags.  With a direct exchange every rank writes its
 * (d_sqnorm, d_overflow) into slot r of two arrays on every peer; once the
 * slots have landed, each rank runs this call:
 *     *d_global_sqnorm   = ((slot_sqnorm[0] + slot_sqnorm[1]) + ...) + slot_sqnorm[n_ranks-1]
 *     *d_global_overflow = 1 if any slot_overflow[r] != 0, else 0
 * The sum is taken in rank order in fp64, so every rank obtains the same bits
 * whatever order the slots arrived in.  Its outputs then feed
 * zero_shard_adam_step (or zero_step_decide_dev and the update).
 *  slot_sqnorm    device, [n_ranks] double, 8-byte aligned
 *  slot_overflow  device, [n_ranks] int32, 4-byte aligned
 *  n_ranks        1 <= n_ranks <= ZERO_MAX_RANKS
 *  d_global_sqnorm, d_global_overflow  device outputs; nothing may overlap
 * One one-workgroup kernel is enqueued.
 * Errors: ZERO_EINVAL (bad n_ranks, NULL, overlap), ZERO_EALIGN, ZERO_EHIP.
 * ------------------------------------------------------------------------- */
#define ZERO_MAX_RANKS 65536
int zero_norm_combine_ranks(const double* slot_sqnorm, const int32_t* slot_overflow, int32_t n_ranks,
                            double* d_global_sqnorm, int32_t* d_global_overflow, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Extras: physically contiguous device memory for a shard's streams (a
 * layout choice for HBM, not a step of the method).  The fused AdamW pass streams four
 * buffers in and four out at once, and its rate depends on where their pages
 * land.  On one MI355X, over 16 processes each, buffers from the default
 * allocator ran at 75-82% of the 8 TB/s peak (mean 79.5%).  Physically
 * contiguous buffers ran at 79-83.5% (mean 81.6%).
 *
 * zero_device_alloc_contiguous: *ptr = `bytes` of contiguous device memory on
 *   the current device (NULL for 0 bytes).  The caller owns it and releases
 *   it with zero_device_free.  No stream is involved and nothing is enqueued.
 *   Errors: ZERO_EINVAL (ptr NULL), ZERO_EHIP (no contiguous range of that
 *   size, or a runtime error; *ptr is NULL).
 * zero_device_free: releases memory from zero_device_alloc_contiguous (NULL:
 *   no-op).  It synchronises the device, as hipFree does.
 * zero_pool_alloc / zero_pool_free: the same memory behind the signatures of
 *   a PyTorch pluggable allocator (size, device, stream), for a torch memory
 *   pool that serves the shard's tensors.  zero_pool_alloc falls back to
 *   ordinary device memory when no contiguous range is left and returns NULL
 *   only when that fails too.  The stream argument is unused.
 * zero_pool_counts: how many segments zero_pool_alloc has handed out since
 *   the library was loaded, physically contiguous (*contiguous) and fallen
 *   back to ordinary device memory (*fallback), over all devices: two
 *   process-wide counters, the allocator's only state.  Errors: ZERO_EINVAL
 *   (NULL output).
 * These calls and the step graphs are the only ones that allocate device or
 * pinned memory.  (The other state the library keeps is listed at the head
 * of this header: the host step's worker threads and, per GPU, the fixed
 * array of the allocation-free norm pass and its looked-up address.)
 * ------------------------------------------------------------------------- */
int zero_device_alloc_contiguous(void** ptr, size_t bytes);
int zero_device_free(void* ptr);
void* zero_pool_alloc(size_t bytes, int device, void* stream);
void zero_pool_free(void* ptr, size_t bytes, int device, void* stream);
int zero_pool_counts(int64_t* contiguous, int64_t* fallback);

/* Static description of a status code, and the thread-local detail of the
 * last failing call (empty string if none). */
const char* zero_status_string(int status);
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZERO_SHARD_H */
