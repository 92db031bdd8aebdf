/*
 * zero_mi355x.h - C ABI of the per-rank partitioned mixed-precision optimizer
 * step (ZeRO / FSDP data parallelism) on AMD MI355X (gfx950).
 *
 * Cited page: "Zero Redundancy Optimizer (ZeRO) and Fully Sharded Data
 * Parallelism (FSDP): Mathematical Foundations of Memory Partitioning,
 * Communication Complexity, and Overlapped Execution" (llms.blog), written
 * [ZF] below with the section name.
 *
 * One rank's step, as [ZF] "Execution Flow for ZeRO-1" (steps 2-4) and
 * "ZeRO-Stage 2" lay it out, maps onto these calls:
 *   zero_partition_plan     flat padded buffer cut into N_d equal shards
 *   zero_grad_reduce_shard  the rank's averaged gradient slice (reduce-scatter,
 *                           seen from the receiving rank)
 *   zero_grad_sqnorm        squared-norm partial of a gradient shard
 *   zero_clip_scale         global-norm clip coefficient from all partials
 *   zero_shard_adamw_step   fp32 master/m/v update and bf16 parameter emit
 *   zero_multi_tensor_adamw_step  the same over a ragged list of tensors
 *                           (FSDP-2's per-parameter shards)
 *   zero_mt_table_*         the same list described once in device memory,
 *                           stepped in one launch
 *   zero_reduce_adamw_step  the reduce and the update in one pass, for a step
 *                           with no global norm between them
 *   zero_gather_params      bf16 shards back to per-tensor parameters
 *                           (all-gather output layout, then un-flatten)
 *   zero_flatten_params     per-tensor bf16 buffers into the padded flat buffer
 *                           (the step before the reduce; inverse of the gather)
 *   zero_*_table_create, zero_copy_table_run  the gather or flatten of fixed
 *                           buffers, described once in device memory
 *   zero_reduce_table_*     the reduce straight from per-tensor replicas of
 *                           fixed buffers (no flatten of each replica first)
 *   zero_offload_adamw_step ZeRO-Offload: the update on the host CPU, with the
 *                           gradient and parameter transfers overlapped
 *   zero_adamw_schedule_*, zero_*_scheduled  AdamW with the step number counted
 *                           on the device, so a step captured in a HIP graph
 *                           replays successive steps
 *
 * Conventions, for every function below:
 *   - bf16 values travel as raw uint16_t bit patterns; fp32 as float.
 *   - "device" pointers address GPU memory of the current HIP device; the
 *     caller allocates and owns them. The library never frees them and keeps
 *     no reference to them after the call returns.
 *   - "host" pointers are read during the call only.
 *   - Device work is enqueued on `stream` (0 = the legacy default stream) and
 *     runs asynchronously; the function returns once the work is enqueued.
 *     Results are visible to later work on the same stream.
 *   - Every function returns a zero_status; nothing aborts or throws across
 *     the ABI. On failure nothing has been enqueued, unless the status is
 *     ZERO_EHIP from a failed launch. zero_last_error() gives a readable
 *     detail for the last failure on the calling thread.
 *   - Element counts and offsets are int64_t; buffers beyond 2^32 elements
 *     are supported everywhere.
 *   - Any device pointer that is not 16-byte aligned is accepted; such calls
 *     run a slower scalar path with identical results.
 */
#ifndef ZERO_MI355X_H
#define ZERO_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum zero_status {
    ZERO_OK = 0,
    ZERO_EINVAL = 1,    /* an argument is invalid (null, negative, out of range) */
    ZERO_ERANGE = 2,    /* a size overflows int64 or exceeds a documented maximum */
    ZERO_ENOMEM = 3,    /* host memory allocation failed */
    ZERO_EHIP = 4,      /* a HIP runtime call or kernel launch failed */
    ZERO_ENOSPACE = 5   /* the caller's workspace is smaller than required */
} zero_status;

/* Largest number of gradient replicas one zero_grad_reduce_shard call reduces. */
#define ZERO_MAX_REPLICAS 64

/* Opaque partition plan: host memory owned by the library, immutable after
 * zero_partition_plan returns, safe to read from several threads. */
typedef struct zero_plan zero_plan;

/* The part of tensor `tensor` that lies in rank `rank`'s shard:
 * tensor elements [tensor_offset, tensor_offset + length) are shard elements
 * [shard_offset, shard_offset + length). */
typedef struct zero_segment {
    int32_t tensor;
    int32_t rank;
    int64_t tensor_offset;
    int64_t shard_offset;
    int64_t length;
} zero_segment;

/* ------------------------------------------------------------------ plan (host only)
 *
 * [ZF] "FSDP-1: FlatParameter and Module-Level Wrapping": a unit's tensors are
 * flattened into one contiguous 1-D buffer, padded to a length divisible by
 * the world size, and cut into N_d equal chunks; [ZF] "ZeRO-Stage 1" gives
 * each rank a Phi/N_d slice of the optimizer state.
 *
 * numels       host [n_tensors]: element count of each tensor, in flat order
 *              (each >= 0; zero-sized tensors are allowed and own no elements).
 * n_tensors    >= 0.
 * n_ranks      N_d >= 1.
 * align_elems  A >= 1: every shard length is a multiple of A, so the padded
 *              length P = ceil(Phi / (N_d*A)) * N_d*A and the shard length
 *              S = P / N_d. Tensor t starts at flat element sum(numels[<t]);
 *              elements [Phi, P) are padding. Rank r owns [r*S, (r+1)*S).
 * out          receives the new plan; free it with zero_plan_free.
 * Errors: ZERO_EINVAL for a null pointer, a negative count, n_ranks < 1 or
 * align_elems < 1; ZERO_ERANGE if P would overflow int64; ZERO_ENOMEM. */
zero_status zero_partition_plan(const int64_t* numels, int32_t n_tensors, int32_t n_ranks,
                                int32_t align_elems, zero_plan** out);
void zero_plan_free(zero_plan* plan);                       /* accepts NULL */

/* FSDP-2 per-parameter layout. [ZF] "FSDP-2: Per-Parameter Sharding via
 * DTensor (fully_shard)": each tensor is sharded on its own along its leading
 * dimension (a Shard(0) placement) instead of being flattened with the others,
 * and the shards of one unit travel in a coalesced communication buffer.
 *
 * Tensor t (numels[t] elements, dim0[t] >= 1 rows of inner_t = numels[t]/dim0[t]
 * elements; dim0[t] must divide numels[t]; a zero-sized tensor may give 0)
 * is cut into N_d chunks of c_t = ceil(dim0[t] / N_d) rows, as torch.chunk
 * cuts it: rank r holds rows [r*c_t, min((r+1)*c_t, dim0[t])), possibly none.
 * A rank's coalesced buffer holds its chunk of every tensor in order, each
 * padded to c_t*inner_t elements, the whole padded to a multiple of
 * align_elems: S = that length. The N_d coalesced buffers side by side form
 * the plan's flat buffer of P = N_d*S elements, so zero_grad_reduce_shard,
 * zero_shard_adamw_step, zero_gather_params and zero_flatten_params apply
 * unchanged; padding positions hold zeros. zero_plan_tensor_offset(t) gives
 * the start of tensor t's chunk inside every rank's buffer.
 * Errors as zero_partition_plan, plus ZERO_EINVAL when dim0 does not divide
 * a numel. */
zero_status zero_partition_plan_shard0(const int64_t* numels, const int64_t* dim0,
                                       int32_t n_tensors, int32_t n_ranks, int32_t align_elems,
                                       zero_plan** out);

/* 0 for a flat (FSDP-1 / ZeRO) plan, 1 for a Shard(0) plan, -1 for NULL. */
int32_t zero_plan_kind(const zero_plan* plan);

int64_t zero_plan_numel(const zero_plan* plan);             /* Phi, or -1 if plan is NULL */
int64_t zero_plan_padded_numel(const zero_plan* plan);      /* P,   or -1 */
int64_t zero_plan_shard_numel(const zero_plan* plan);       /* S,   or -1 */
int32_t zero_plan_num_tensors(const zero_plan* plan);       /* T,   or -1 */
int32_t zero_plan_num_ranks(const zero_plan* plan);         /* N_d, or -1 */
int64_t zero_plan_tensor_offset(const zero_plan* plan, int32_t tensor);  /* -1 if out of range;
                                                                           flat plans: the tensor's
                                                                           flat start */
int64_t zero_plan_tensor_numel(const zero_plan* plan, int32_t tensor);   /* -1 if out of range */
int32_t zero_plan_num_segments(const zero_plan* plan, int32_t rank);     /* -1 if out of range */

/* Copies rank's segments, in flat order, into host array out[capacity].
 * *count receives the number of segments; ZERO_ENOSPACE (with *count set) if
 * capacity is too small. */
zero_status zero_plan_segments(const zero_plan* plan, int32_t rank, zero_segment* out,
                               int32_t capacity, int32_t* count);

/* Static training-state bytes per GPU. [ZF] "Static Memory Allocation"
 * (16 bytes per parameter: 2 bf16 param, 2 bf16 grad, 12 fp32 master/m/v)
 * and the stage formulas of [ZF] "ZeRO-Stage 1" (4 Phi + 12 Phi/N_d),
 * "ZeRO-Stage 2" (2 Phi + 14 Phi/N_d) and "ZeRO-Stage 3 and Fully Sharded Data
 * Parallelism" (16 Phi/N_d). stage: 0 = DDP, 1, 2, 3. padded != 0 counts the
 * flat buffers at P and the shards at S (stage 0 stays 16 Phi). */
zero_status zero_plan_memory_bytes(const zero_plan* plan, int32_t stage, int32_t padded,
                                   double* bytes);

/* ------------------------------------------------------------------ gradient reduction
 *
 * [ZF] "Execution Flow for ZeRO-1", step 2: rank i receives the gradient of
 * its own partition averaged over the data-parallel ranks; [ZF] "ZeRO-Stage 2":
 * gradients are reduced into their owners' slices bucket by bucket as backward
 * produces them. On one GPU the R replicas sit in one HBM; this call is the
 * receiving rank's arithmetic of that reduce-scatter.
 *
 * replicas     host [n_replicas] of device pointers; replicas[k] points at
 *              replica k's bf16 gradient for global flat elements
 *              [begin, begin + count) (a whole flat buffer, or one bucket).
 * n_replicas   R, 1 <= R <= ZERO_MAX_REPLICAS.
 * begin,count  the global flat window the replica buffers cover (count >= 0,
 *              begin >= 0, begin + count <= P).
 * shard_grad   device [S]: element i is global element rank*S + i. Only the
 *              window's intersection with rank's shard is written; that slice
 *              must not overlap the replicas' slices the call reads, or the
 *              workspace:
 *              out = bf16_rne( (sum over k = 0..R-1, in order, of fp32(rep_k)) / R ),
 *              the sum and the division in IEEE fp32.
 * sqnorm_out   device, nullable: receives the fp64 sum of squares of the bf16
 *              values this call wrote (0 if it wrote nothing). Deterministic for a
 *              given window and workspace size.
 * workspace    device, required when sqnorm_out is non-null; at least
 *              zero_sqnorm_workspace_bytes() bytes, 8-byte aligned, owned by
 *              the caller. It holds the per-workgroup partials between the
 *              call's kernels; it needs no initialisation and its contents
 *              on return are unspecified. Calls that may run
 *              at the same time (on different streams) need separate
 *              workspaces; calls on one stream may share one.
 *              With zero_reduce_workspace_bytes(n) bytes or more, where n is
 *              the number of elements written (at most count), a window of
 *              2^24 elements or more, of at most 8 replicas, whose slices are
 *              4-byte aligned takes the one-pass kernel: one workgroup per 512 elements, a partial per
 *              workgroup and a two-level final sum. It is faster on windows too
 *              large for the caches. The bf16 output is the same either way.
 *              The fp64 sum is grouped differently, so its last bits may
 *              differ. Without a norm the one-pass kernel needs no workspace.
 * Errors: ZERO_EINVAL (null plan/replicas/shard_grad, a null replica pointer,
 * R out of range, rank out of range, bad window, workspace not 8-byte
 * aligned, the written slice overlapping a replica's slice or the workspace,
 * named in zero_last_error()); ZERO_ENOSPACE; ZERO_EHIP. */
zero_status zero_grad_reduce_shard(const zero_plan* plan, int32_t rank,
                                   const uint16_t* const* replicas, int32_t n_replicas,
                                   int64_t begin, int64_t count, uint16_t* shard_grad,
                                   double* sqnorm_out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): zero_grad_reduce_shard
 * with the same arguments except the workspace, which is a device array the
 * library owns, ZERO_NOALLOC_SCRATCH_BYTES bytes on each device, kept from the
 * library's load until the process ends. The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine. The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress) with
 * the device current; a caller that captures graphs makes that first call
 * before capturing. The bf16 output is zero_grad_reduce_shard's. The norm
 * equals zero_grad_reduce_shard's with a workspace of
 * ZERO_NOALLOC_SCRATCH_BYTES bytes: windows of 2^24 elements or more whose
 * one-pass partials fit the array (up to about 2.7e8 elements) take the
 * one-pass kernel, larger windows the grid-stride kernel and its fixed 2,048
 * partials, so no window size is refused. Every call on one device shares
 * that device's array: calls that may overlap on one device (other streams,
 * other host threads) race on it and must be ordered by the caller; calls in
 * order on one stream are safe. Errors: as zero_grad_reduce_shard (no
 * workspace errors); ZERO_ERANGE for a device index above 63; ZERO_EHIP. */
#define ZERO_NOALLOC_SCRATCH_BYTES (4u << 20)
zero_status zero_grad_reduce_shard_noalloc(const zero_plan* plan, int32_t rank,
                                           const uint16_t* const* replicas, int32_t n_replicas,
                                           int64_t begin, int64_t count, uint16_t* shard_grad,
                                           double* sqnorm_out, hipStream_t stream);

/* ------------------------------------------------------------------ squared norm
 *
 * Sum of squares of n bf16 values (device [n]), accumulated in fp64 (each
 * square is exact), written to device sqnorm_out[0]. Two fixed-order
 * reduction levels, no floating-point atomics: the result is reproducible on
 * a given device. The norm clip is not on the cited pages; the global norm it
 * needs is the sum of these partials over every rank. workspace as for
 * zero_grad_reduce_shard; with zero_reduce_workspace_bytes(n) bytes or more, a
 * 16-byte-aligned input of 2^24 elements or more takes a one-pass kernel (a
 * partial per 16,384 elements, two-level final sum; the fp64 grouping differs,
 * so the last bits may too).
 * Errors: ZERO_EINVAL (null pointers with n > 0, n < 0, workspace not 8-byte
 * aligned); ZERO_ENOSPACE; ZERO_EHIP. */
zero_status zero_grad_sqnorm(const uint16_t* grad, int64_t n, double* sqnorm_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes that zero_grad_sqnorm and zero_grad_reduce_shard need: a
 * fixed bound, independent of n and of the device. */
size_t zero_sqnorm_workspace_bytes(void);

/* Workspace bytes with which zero_grad_reduce_shard (with the norm) and
 * zero_grad_sqnorm can take their one-pass kernels on up to count elements:
 * about 8 bytes per 512 elements, never less than zero_sqnorm_workspace_bytes().
 * Host only. */
size_t zero_reduce_workspace_bytes(int64_t count);

/* ------------------------------------------------------------------ clip coefficient
 *
 * partials     device [n_partials] fp64 squared-norm partials (one per rank, or
 *              per bucket), summed in index order in fp64.
 * max_norm     clip threshold; <= 0 disables clipping (coefficient 1).
 * scale_out    device float: min(1, max_norm / (sqrt(total) + 1e-6)) rounded
 *              once to fp32; NaN when the total is not finite, which makes
 *              zero_shard_adamw_step skip its update.
 * Errors: ZERO_EINVAL (null pointers, n_partials < 1 or > 65536); ZERO_EHIP. */
zero_status zero_clip_scale(const double* partials, int32_t n_partials, double max_norm,
                            float* scale_out, hipStream_t stream);

/* ------------------------------------------------------------------ AdamW shard update
 *
 * [ZF] "Static Memory Allocation": fp32 master weights, fp32 first moment m_t
 * and fp32 second moment v_t, 16-bit parameters; [ZF] "Execution Flow for
 * ZeRO-1", steps 3-4: the rank updates its own slice and emits 16-bit
 * parameters for the all-gather; [ZF] "ZeRO-Offload Mechanics": O(1) work per
 * parameter, so the update is bound by memory traffic (28 bytes per element).
 *
 * Per element, each operation one IEEE fp32 operation (no fused multiply-add),
 * in this order, with the scalars computed in fp64 on the host and rounded
 * once to fp32 (t = step):
 *   g = fp32(grad) * clip
 *   m = beta1*m + (1-beta1)*g
 *   v = beta2*v + (1-beta2)*(g*g)
 *   p = p * (1 - lr*weight_decay)
 *   p = p - (lr/(1-beta1^t)) * (m / (sqrt(v)/sqrt(1-beta2^t) + eps))
 *   param_out = bf16_rne(p)
 * master, exp_avg, exp_avg_sq  device [n] fp32, updated in place.
 * grad         device [n] bf16, read only.
 * param_out    device [n] bf16, written.
 *              The four written arrays must not overlap one another or grad
 *              (each element is read and written by one lane; arrays shifted
 *              against each other would race).
 * step         t >= 1 (1-based bias-correction step).
 * clip_scale   device float, nullable (NULL means 1). A non-finite value skips
 *              the update: nothing is read or written.
 * Errors: ZERO_EINVAL (null pointers with n > 0, n < 0, step < 1, beta1 or
 * beta2 outside [0, 1), eps <= 0, lr < 0, non-finite scalars, overlapping
 * arrays, named in zero_last_error()); ZERO_EHIP. */
zero_status zero_shard_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                  const uint16_t* grad, uint16_t* param_out, int64_t n,
                                  int64_t step, double lr, double beta1, double beta2, double eps,
                                  double weight_decay, const float* clip_scale,
                                  hipStream_t stream);

/* Step counted on the device, for a step captured in a HIP graph. [ZF] "Execution
 * Flow for ZeRO-1", step 3, repeated every iteration: zero_shard_adamw_step
 * takes t from the host and computes the step's scalars there, so a captured
 * launch would replay one step forever. A schedule holds, in device memory,
 * the number of updates applied and the scalars of the next step, and a table
 * of the scalars of steps 1..L (each as zero_shard_adamw_step computes them
 * on the host, so the results are the same bits). L is the step from which
 * both bias corrections are exactly 1 in fp64 (beta^t < 2^-56), or the length
 * of the learning-rate list if longer: every later step has step L's scalars.
 * For beta2 = 0.999, L = 38,797 (1.2 MB).
 *
 * zero_adamw_schedule_create: lr is a host array of n_lr >= 1 learning rates,
 * step t using lr[min(t, n_lr) - 1] (one value: a constant rate); betas, eps
 * and weight_decay as zero_shard_adamw_step; the first update applied is step
 * first_step >= 1 (a resumed run passes its next step). Allocates on the
 * current device. Errors: ZERO_EINVAL (bad hyperparameters, NULL lr or out,
 * n_lr < 1, first_step < 1); ZERO_ERANGE when L would pass 2^24 (a beta within
 * about 2.3e-6 of 1, or a longer list); ZERO_ENOMEM; ZERO_EHIP.
 * zero_shard_adamw_step_scheduled: zero_shard_adamw_step's update and
 * arguments, with the step's scalars read on the device from the schedule;
 * it does not move the schedule on, so a step may update any number of
 * arrays with it (buckets, tensors, ranks).
 * zero_adamw_schedule_advance: once per step, after the step's updates on the
 * same stream: counts the step as applied and loads the next step's scalars.
 * A non-finite clip coefficient (the updates skipped) leaves the schedule as it
 * is, so a skipped step is not counted. One lane; allocates nothing.
 * zero_adamw_schedule_applied: the number of updates applied, read back
 * synchronously (hipMemcpy; the caller first waits for the streams that
 * advanced the schedule). zero_adamw_schedule_length: L (-1 for NULL).
 * Calls that move one schedule on must be ordered by the caller (one stream).
 * Errors of the step and advance: ZERO_EINVAL (NULL schedule, the schedule on
 * another device, as zero_shard_adamw_step otherwise); ZERO_EHIP.
 *
 * zero_adamw_step_scalars: host only; the eight fp32 scalars every AdamW entry
 * point computes for step t, in order beta1, 1-beta1, beta2, 1-beta2, eps,
 * lr/(1-beta1^t), sqrt(1-beta2^t), 1-lr*weight_decay. Errors: as
 * zero_shard_adamw_step's hyperparameter checks; ZERO_EINVAL for a NULL out. */
typedef struct zero_adamw_schedule zero_adamw_schedule;
zero_status zero_adamw_schedule_create(const double* lr, int64_t n_lr, double beta1, double beta2,
                                       double eps, double weight_decay, int64_t first_step,
                                       zero_adamw_schedule** out);
void zero_adamw_schedule_free(zero_adamw_schedule* schedule);
int64_t zero_adamw_schedule_length(const zero_adamw_schedule* schedule);
zero_status zero_adamw_schedule_applied(const zero_adamw_schedule* schedule, int64_t* applied);
zero_status zero_adamw_schedule_advance(zero_adamw_schedule* schedule, const float* clip_scale,
                                        hipStream_t stream);
zero_status zero_shard_adamw_step_scheduled(float* master, float* exp_avg, float* exp_avg_sq,
                                            const uint16_t* grad, uint16_t* param_out, int64_t n,
                                            const zero_adamw_schedule* schedule,
                                            const float* clip_scale, hipStream_t stream);
zero_status zero_adamw_step_scalars(int64_t step, double lr, double beta1, double beta2, double eps,
                                    double weight_decay, float* out);
/* The scheduled forms of the multi-tensor table step and of the one-pass
 * reduce and update (declared with their plain forms below): the same
 * arguments and results, with the step's scalars read on the device from the
 * schedule, which they do not move on. Errors: as their plain forms (without
 * the hyperparameter checks); ZERO_EINVAL for a NULL schedule or one that
 * lives on another device than the current one (or, for the table, than the
 * table). */

/* Reduce and update in one pass. [ZF] "Execution Flow for ZeRO-1", steps 2-3:
 * the rank receives the averaged gradient of its slice and updates its master
 * weights and optimizer state from it. When the step needs no global norm
 * between the two (no clipping, or a clip coefficient the caller already
 * holds), they run as one pass over the rank's window: for every element of
 * [begin, begin + count) within the rank's shard, the averaged gradient is
 * zero_grad_reduce_shard's (fp32 sum in replica order, one fp32 division by
 * R, bf16 round-to-nearest-even) and the update zero_shard_adamw_step's on
 * it, bit for bit the two calls in sequence, without the gradient's round trip
 * through HBM (2R + 26 bytes per element instead of 2R + 30).
 * plan, rank, replicas, n_replicas, begin, count: as zero_grad_reduce_shard.
 * master, exp_avg, exp_avg_sq  device [S] fp32, the rank's shard state, in place.
 * param_out    device [S] bf16, the rank's parameter shard. Element i of
 *              these arrays is global element rank*S + i; only the window's
 *              part of the shard is read and written.
 * shard_grad   device [S] bf16, nullable: when given, also receives the
 *              averaged gradient, as zero_grad_reduce_shard writes it.
 *              Within the window, the written arrays (the three fp32 arrays,
 *              param_out, shard_grad) must not overlap one another or the
 *              replicas' slices the call reads.
 * step, lr, beta1, beta2, eps, weight_decay, clip_scale: as
 *              zero_shard_adamw_step; a non-finite coefficient skips the
 *              update (shard_grad, when given, is still written).
 * Errors: ZERO_EINVAL (null plan or replicas, a null replica or state array
 * for a non-empty window, R or rank out of range, bad window, bad
 * hyperparameters, overlapping arrays, named in zero_last_error());
 * ZERO_EHIP. */
zero_status zero_reduce_adamw_step(const zero_plan* plan, int32_t rank,
                                   const uint16_t* const* replicas, int32_t n_replicas,
                                   int64_t begin, int64_t count, float* master, float* exp_avg,
                                   float* exp_avg_sq, uint16_t* param_out, uint16_t* shard_grad,
                                   int64_t step, double lr, double beta1, double beta2, double eps,
                                   double weight_decay, const float* clip_scale,
                                   hipStream_t stream);
zero_status zero_reduce_adamw_step_scheduled(const zero_plan* plan, int32_t rank,
                                             const uint16_t* const* replicas, int32_t n_replicas,
                                             int64_t begin, int64_t count, float* master,
                                             float* exp_avg, float* exp_avg_sq, uint16_t* param_out,
                                             uint16_t* shard_grad, const zero_adamw_schedule* schedule,
                                             const float* clip_scale, hipStream_t stream);

/* Multi-tensor form. [ZF] "FSDP-2: Per-Parameter Sharding via DTensor
 * (fully_shard)": each parameter keeps its own local shard, so the rank's
 * optimizer step runs over a ragged list of per-parameter tensors rather than
 * one flat buffer. Tensor t has its own arrays masters[t], exp_avgs[t],
 * exp_avg_sqs[t] (device [numels[t]] fp32, in place), grads[t] (device bf16,
 * read only) and params_out[t] (device bf16, written); tensor t's four
 * written arrays must not overlap one another or grads[t], and different
 * tensors' written arrays must not overlap (that is the caller's to keep: the
 * call checks each tensor's arrays against each other only); the pointer arrays and numels are host arrays of
 * n_tensors entries. Every element gets zero_shard_adamw_step's arithmetic
 * (identical bits), with one step, one set of hyperparameters and one clip
 * coefficient for the whole list. Zero-sized tensors are skipped (their
 * pointers may be NULL). Any pointer alignment. The tensors are batched
 * largest first, 78 per launch (the order changes no result).
 * Errors: as zero_shard_adamw_step, per tensor (ZERO_EINVAL names it);
 * ZERO_ERANGE for a tensor of 2^39 elements or more; ZERO_ENOMEM; ZERO_EHIP. */
zero_status zero_multi_tensor_adamw_step(float* const* masters, float* const* exp_avgs,
                                         float* const* exp_avg_sqs, const uint16_t* const* grads,
                                         uint16_t* const* params_out, const int64_t* numels,
                                         int32_t n_tensors, int64_t step, double lr, double beta1,
                                         double beta2, double eps, double weight_decay,
                                         const float* clip_scale, hipStream_t stream);

/* The multi-tensor form for a fixed list, with its table in device memory.
 * [ZF] "FSDP-2: Per-Parameter Sharding via DTensor (fully_shard)": the same
 * per-parameter list is stepped every iteration, so its description can be
 * built once. zero_mt_table_create checks the list exactly as
 * zero_multi_tensor_adamw_step does and copies, to device memory that the
 * table owns, one 64-byte descriptor per non-empty tensor (its five device
 * pointers and its size) and one 4-byte tensor index per workgroup of 512
 * elements (about 0.8 bytes per 100 elements). zero_mt_table_adamw_step then
 * updates every tensor of the list in one launch (a list of 2^24 workgroups or
 * more, above 8.6e9 elements, in several), with zero_shard_adamw_step's
 * arithmetic: identical bits to both other AdamW entry points.
 * Create: the arguments as zero_multi_tensor_adamw_step's list; out receives
 * the table. It calls hipMalloc and a synchronous hipMemcpy on the current
 * device, once. The table keeps the device pointers (not the data): the
 * caller keeps those buffers alive and in place for the table's lifetime.
 * Errors: as zero_multi_tensor_adamw_step's list checks; ZERO_EINVAL for a
 * NULL out; ZERO_ERANGE for 2^31 workgroups or more; ZERO_ENOMEM; ZERO_EHIP
 * (allocation or copy failed).
 * Step: step, hyperparameters and clip_scale as zero_shard_adamw_step. It must
 * run with the table's device current (ZERO_EINVAL otherwise). An empty list
 * enqueues nothing.
 * Free: releases the device memory (hipFree, which waits for the device);
 * no step using the table may still be running. Accepts NULL.
 * Blocks: the workgroups of one step, or -1 for NULL. */
typedef struct zero_mt_table zero_mt_table;
zero_status zero_mt_table_create(float* const* masters, float* const* exp_avgs,
                                 float* const* exp_avg_sqs, const uint16_t* const* grads,
                                 uint16_t* const* params_out, const int64_t* numels,
                                 int32_t n_tensors, zero_mt_table** out);
void zero_mt_table_free(zero_mt_table* table);
int64_t zero_mt_table_blocks(const zero_mt_table* table);
zero_status zero_mt_table_adamw_step(const zero_mt_table* table, int64_t step, double lr,
                                     double beta1, double beta2, double eps, double weight_decay,
                                     const float* clip_scale, hipStream_t stream);
zero_status zero_mt_table_adamw_step_scheduled(const zero_mt_table* table,
                                               const zero_adamw_schedule* schedule,
                                               const float* clip_scale, hipStream_t stream);

/* ------------------------------------------------------------------ gather
 *
 * [ZF] "Execution Flow for ZeRO-1", step 4 and "FSDP-1": the N_d bf16 shards,
 * concatenated in rank order, are the flat parameter buffer; tensor t is its
 * slice [offset_t, offset_t + numel_t). This copies every plan segment from
 * its shard into its tensor (padding is not copied). For a Shard(0) plan
 * ([ZF] "FSDP-2: Per-Parameter Sharding via DTensor"), tensor t is its ranks'
 * dim-0 chunks stacked in rank order, each read from its chunk's place in
 * that rank's coalesced buffer.
 * shards       host [N_d] of device pointers, each to S bf16 values. A NULL
 *              entry skips that rank's segments (their tensor elements are
 *              left as they are): ranks can be gathered in separate calls, for
 *              example the other ranks' while the own shard is being updated.
 * tensors      host [T] of device pointers, tensor t to numel_t bf16 values
 *              (may be NULL only for zero-sized tensors). Outputs must not
 *              overlap the shards or each other.
 * Errors: ZERO_EINVAL (null plan/arrays or a needed null pointer, a tensor
 * overlapping another tensor or a shard, named in zero_last_error());
 * ZERO_ENOMEM; ZERO_EHIP. */
zero_status zero_gather_params(const zero_plan* plan, const uint16_t* const* shards,
                               uint16_t* const* tensors, hipStream_t stream);

/* ------------------------------------------------------------------ flatten
 *
 * [ZF] "FSDP-1: FlatParameter and Module-Level Wrapping": a unit's tensors are
 * flattened into one contiguous 1-D buffer, padded to a length divisible by
 * the world size. This builds that buffer from per-tensor bf16 buffers: every
 * plan segment is copied from its tensor to its place in the flat buffer
 * (flat plans: tensor t at [offset_t, offset_t + numel_t); Shard(0) plans:
 * each rank's chunk into that rank's coalesced buffer) and every other
 * position is set to +0. It is the inverse of zero_gather_params and the step
 * before zero_grad_reduce_shard: each data-parallel replica flattens its
 * per-tensor gradients into the flat buffer that the reduce-scatter cuts into
 * N_d shards.
 * tensors      host [T] of device pointers, tensor t to numel_t bf16 values
 *              (may be NULL only for zero-sized tensors).
 * flat         device [P] bf16, written entirely; must not overlap the tensors.
 * Errors: ZERO_EINVAL (null plan/arrays or a needed null pointer, flat
 * overlapping a tensor, named in zero_last_error()); ZERO_ENOMEM; ZERO_EHIP. */
zero_status zero_flatten_params(const zero_plan* plan, const uint16_t* const* tensors,
                                uint16_t* flat, hipStream_t stream);

/* Gather and flatten for fixed buffers, with their tables in device memory.
 * A training loop gathers the same shards into the same tensors every step
 * (and flattens the same per-tensor gradients into the same flat buffer), so
 * the copy can be described once. zero_gather_table_create takes the
 * arguments of zero_gather_params, zero_flatten_table_create those of
 * zero_flatten_params, with the same checks. Each lists every plan segment
 * (for the flatten also every zero-filled gap) as a piece, and copies to
 * device memory that the table owns one 32-byte descriptor per piece (source,
 * destination, length) and one 4-byte piece index per workgroup of 2,048
 * elements (0.1% of the bytes copied). zero_copy_table_run then performs the
 * whole copy in one launch (several only past 2^24 workgroups, above 3.4e10
 * elements), for flat and Shard(0) plans alike, with the same result as the
 * call the table was made from: the same bits are copied, and the same
 * positions zero-filled.
 * Create: hipMalloc and a synchronous hipMemcpy on the current device, once.
 * The table keeps the device pointers, not the data: the caller keeps those
 * buffers alive and in place for the table's lifetime. A NULL shard skips its
 * rank, as in zero_gather_params. out receives the table.
 * Errors: as the call it mirrors; ZERO_EINVAL for a NULL out; ZERO_ERANGE for
 * 2^31 workgroups or more; ZERO_ENOMEM; ZERO_EHIP (allocation or copy).
 * Run: enqueued on stream; it must run with the table's device current
 * (ZERO_EINVAL otherwise). An empty table enqueues nothing.
 * Free: releases the device memory (hipFree, which waits for the device);
 * no run using the table may still be in flight. Accepts NULL.
 * Blocks: the workgroups of one run, or -1 for NULL. */
typedef struct zero_copy_table zero_copy_table;
zero_status zero_gather_table_create(const zero_plan* plan, const uint16_t* const* shards,
                                     uint16_t* const* tensors, zero_copy_table** out);
zero_status zero_flatten_table_create(const zero_plan* plan, const uint16_t* const* tensors,
                                      uint16_t* flat, zero_copy_table** out);
zero_status zero_copy_table_run(const zero_copy_table* table, hipStream_t stream);
int64_t zero_copy_table_blocks(const zero_copy_table* table);
void zero_copy_table_free(zero_copy_table* table);

/* Reduce from per-tensor replicas, for fixed buffers. [ZF] "FSDP-1:
 * FlatParameter and Module-Level Wrapping" (every tensor's place in the flat
 * padded buffer) with "Execution Flow for ZeRO-1", step 2 (the rank's slice
 * of the gradient averaged over the replicas). When the R replicas are still
 * per-tensor buffers, the rank's averaged gradient is reduced from them
 * directly, without first flattening each replica (zero_flatten_params): for
 * every segment of the rank's shard, tensor elements [tensor_offset,
 * tensor_offset + length) of each replica are reduced into shard elements
 * [shard_offset, shard_offset + length), and every other shard position
 * (padding) is set to +0. The bits are those of zero_flatten_params on each
 * replica followed by zero_grad_reduce_shard over the whole shard (fp32 sum in
 * replica order, one fp32 division by R, bf16 round-to-nearest-even); the
 * squared-norm partial, when asked for, is the same fp64 sum to within
 * rounding. Per shard element (2R + 2) bytes move, against 6R + 2 with the
 * flattens. Flat and Shard(0) plans alike.
 * plan, rank      the plan and this rank.
 * replica_tensors host [R * T] of device pointers: entry k * T + t is replica
 *                 k's tensor t, numel_t bf16 values; may be NULL only for
 *                 tensors with no segment in this rank's shard.
 * n_replicas      R, 1..ZERO_MAX_REPLICAS.
 * shard_grad      device [S] bf16, written entirely by each run; must not
 *                 overlap the replicas.
 * Create: lists the rank's segments and padding gaps as pieces and copies to
 * device memory that the table owns one 64-byte descriptor per piece, one
 * 4-byte piece index per workgroup of 2,048 shard elements, the R * T replica
 * pointers and room for one fp64 partial per workgroup (hipMalloc and a
 * synchronous hipMemcpy on the current device, once). The table keeps the
 * pointers, not the data: the caller keeps the buffers alive and in place.
 * Errors: ZERO_EINVAL (NULL out, plan, replica_tensors or shard_grad; rank or
 * R out of range; a NULL replica tensor the shard needs, or one that overlaps
 * shard_grad); ZERO_ERANGE (2^31
 * workgroups or more); ZERO_ENOMEM; ZERO_EHIP.
 * Run: enqueued on stream, with the table's device current (ZERO_EINVAL
 * otherwise); sqnorm_out (device double, nullable) receives the squared
 * norm of the written gradient. Runs of one table must not overlap (they
 * share its partials). Free: hipFree; accepts NULL. Blocks: the workgroups of
 * one run, or -1 for NULL. */
typedef struct zero_reduce_table zero_reduce_table;
zero_status zero_reduce_table_create(const zero_plan* plan, int32_t rank,
                                     const uint16_t* const* replica_tensors, int32_t n_replicas,
                                     uint16_t* shard_grad, zero_reduce_table** out);
zero_status zero_reduce_table_run(const zero_reduce_table* table, double* sqnorm_out,
                                  hipStream_t stream);
int64_t zero_reduce_table_blocks(const zero_reduce_table* table);
void zero_reduce_table_free(zero_reduce_table* table);

/* ------------------------------------------------------------------ ZeRO-Offload
 *
 * [ZF] "ZeRO-Offload Mechanics": the fp32 optimizer state lives in host DRAM;
 * the GPU's bf16 gradients travel to the host over PCIe / CXL, the host CPU
 * runs the fp32 Adam step and updates the fp32 weights, and the bf16
 * parameters travel back, the transfers overlapping the host work.
 *
 * zero_host_adamw_step: the host CPU update alone, on host arrays [n], with
 * zero_shard_adamw_step's exact per-element arithmetic (identical bits).
 * clip_scale is a host float (a non-finite value skips the step). The work is
 * split over a persistent pool of host threads: n_threads tasks, or one per
 * CPU in the calling process's affinity mask when n_threads <= 0. Calls from
 * several threads are safe; their parallel parts run one after another.
 * Errors: as zero_shard_adamw_step. */
zero_status zero_host_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                 const uint16_t* grad, uint16_t* param_out, int64_t n,
                                 int64_t step, double lr, double beta1, double beta2, double eps,
                                 double weight_decay, float clip_scale, int32_t n_threads);

/* zero_offload_adamw_step: one offloaded step. The bf16 gradient (device
 * d_grad [n]) is copied to the host chunk by chunk while the host updates the
 * previous chunk (h_master, h_exp_avg, h_exp_avg_sq: host [n] fp32, in place)
 * and the bf16 parameters of the chunk before go back to device
 * d_param_out [n]. h_staging: pinned host memory (hipHostMalloc or a pinned
 * torch tensor) of staging_elems bf16 values, split into two gradient and two
 * parameter buffers of staging_elems/4 elements each (the chunk size).
 * d_clip_scale: device float, nullable (1); a non-finite value skips the step
 * (nothing is written). n_threads: as zero_host_adamw_step. Work already
 * enqueued on `stream` happens before the gradient copies; work enqueued on
 * `stream` afterwards sees the new parameters. The copies run on two internal
 * streams of the current device (default priority). The call returns when the
 * host update is done and the staging buffers are free again, on errors too.
 * Calls from several host threads are safe: they share the worker pool and the
 * copy streams and so run one after another. The written ranges (the three
 * host state arrays, the staging in use, d_param_out) must not overlap one
 * another or d_grad.
 * Errors: as zero_host_adamw_step; ZERO_ENOSPACE if staging_elems < 4; ZERO_EHIP. */
zero_status zero_offload_adamw_step(float* h_master, float* h_exp_avg, float* h_exp_avg_sq,
                                    const uint16_t* d_grad, uint16_t* d_param_out,
                                    uint16_t* h_staging, int64_t staging_elems, int64_t n,
                                    int64_t step, double lr, double beta1, double beta2,
                                    double eps, double weight_decay, const float* d_clip_scale,
                                    int32_t n_threads, hipStream_t stream);

/* ------------------------------------------------------------------ diagnostics */
const char* zero_status_string(zero_status status);   /* static string */
const char* zero_last_error(void);                    /* thread-local; "" if none */

#ifdef __cplusplus
}
#endif

#endif /* ZERO_MI355X_H */
