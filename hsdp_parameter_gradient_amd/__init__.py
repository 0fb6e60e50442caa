"""MI355X-native FSDP/HSDP flat-buffer hot path.

A thin ctypes binding over libfsdpflat.so (the C ABI of include/fsdp_flat.h).
The functions have the C entry points' names and only marshal arguments:
every step of the path runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the
library has not been built, the first call raises.
"""

from ._binding import (  # noqa: F401
    AVG,
    SUM,
    FSDPError,
    Layout,
    fsdp_ag_copy_in,
    fsdp_ag_copy_out,
    fsdp_bucket_layout,
    fsdp_cache_info,
    fsdp_fused_ar,
    fsdp_fused_layout,
    fsdp_group_ranks,
    fsdp_last_error,
    fsdp_release_cache,
    fsdp_rs_copy_in,
    fsdp_rs_copy_reduce,
    fsdp_rs_copy_reduce_noalloc,
    fsdp_rs_reduce,
    fsdp_time_next_launch,
    lib,
    lib_path,
    prepare,
)
from .flat_bucket import FlatBucket, FusedGroup  # noqa: F401
from .pipeline import BackwardPipeline  # noqa: F401

__all__ = [
    "FlatBucket", "FusedGroup", "BackwardPipeline",
    "AVG", "SUM", "FSDPError", "Layout", "fsdp_ag_copy_in", "fsdp_ag_copy_out",
    "fsdp_bucket_layout", "fsdp_cache_info", "fsdp_fused_ar", "fsdp_fused_layout", "fsdp_group_ranks",
    "fsdp_last_error", "fsdp_release_cache", "fsdp_rs_copy_in", "fsdp_rs_copy_reduce",
    "fsdp_rs_copy_reduce_noalloc", "fsdp_rs_reduce",
    "fsdp_time_next_launch",
    "lib", "lib_path", "prepare",
]
