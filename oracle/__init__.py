"""CPU oracle for FSDP/HSDP flat-buffer sharding.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__ and by the CPU-baseline leg of bench.py.  The product
package never imports it, and it imports nothing from the product package.
"""

from .fsdp_oracle import (  # noqa: F401
    AVG,
    FUSED_ALIGN_BYTES,
    SUM,
    BucketLayout,
    ag_copy_in,
    ag_copy_out,
    bf16_to_f32,
    f32_to_bf16,
    all_gather,
    bucket_layout,
    dim0_chunk,
    fused_ar,
    fused_layout,
    grad_sync_plan,
    group_sizes,
    reduce_grads_fused,
    reduce_grads_nonfused,
    replicate_groups,
    rs_copy_in,
    rs_copy_reduce,
    rs_reduce,
    shard_groups,
    shard_params,
    sharded_grad,
)
