"""Per-rank partitioned mixed-precision optimizer step (ZeRO / FSDP) on MI355X.

The entry points mirror the C ABI in include/zero_mi355x.h one for one:

    zero_partition_plan     flat padded buffer -> N_d equal shards (host)
    zero_partition_plan_shard0  FSDP-2 per-parameter Shard(0) layout (host)
    zero_grad_reduce_shard  a rank's averaged gradient slice from R replicas
    zero_grad_sqnorm        fp64 squared-norm partial of a bf16 gradient
    zero_clip_scale         global-norm clip coefficient (device scalar)
    zero_shard_adamw_step   fused fp32 AdamW update with bf16 parameter emit
    zero_multi_tensor_adamw_step  the same over a ragged list of tensors
    zero_gather_params      bf16 shards -> per-tensor parameters
    zero_flatten_params     per-tensor buffers -> padded flat buffer
    zero_host_adamw_step    the same update on the host CPU (ZeRO-Offload)
    zero_offload_adamw_step host update with overlapped grad/param transfers

All arithmetic runs in the HIP kernels of libzero_mi355x.so (gfx950); this
package only marshals torch tensors (device memory and streams) into the C
calls. Importing it without the built library raises ImportError.

step.RankStep holds one rank's device state and issues its step (reduce,
clip, AdamW, gather) on one stream, e.g. for GPT-2 small over 8 ranks:

    plan = zero_partition_plan(numels, n_ranks=8, align_elems=128)
    rs = RankStep(plan, rank=7, n_windows=1, hyper=Hyper(), max_norm=1.0,
                  device=torch.device("cuda:0"))
    rs.set_remote_partials(other_ranks_sqnorms)       # from the scalar all-reduce
    rs.step([(0, plan.padded_numel, replica_buffers)]) # rs.tensors: new parameters

RankStep(..., offload=True) keeps the fp32 state in host memory (ZeRO-Offload).
"""
from ._binding import (LIB_PATH, ZERO_MAX_REPLICAS, AdamWSchedule, CopyTable,  # noqa: F401
                       MultiTensorTable, Plan, ReduceTable,
                       zero_adamw_step_scalars, zero_shard_adamw_step_scheduled,
                       zero_reduce_adamw_step_scheduled,
                       ZeroError, reduce_workspace, zero_reduce_workspace_bytes,
                       sqnorm_workspace, zero_clip_scale, zero_flatten_params, zero_gather_params,
                       zero_grad_reduce_shard, zero_grad_reduce_shard_noalloc,
                       zero_reduce_adamw_step,
                       ZERO_NOALLOC_SCRATCH_BYTES,
                       zero_grad_sqnorm, zero_last_error, zero_partition_plan,
                       zero_partition_plan_shard0, zero_host_adamw_step, zero_offload_adamw_step,
                       zero_multi_tensor_adamw_step,
                       zero_shard_adamw_step, zero_sqnorm_workspace_bytes, zero_status_string)
