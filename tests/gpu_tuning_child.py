"""Child process of test_gpu_tuning.py (not collected by pytest).

The library reads its launch tuning (FSDP_MAX_GRID, FSDP_COPY_CHUNK_SHIFT,
FSDP_REDUCE_CHUNK_SHIFT) once per process, so each tuning runs in a fresh
process: this script runs a set of the parity cases of test_gpu_parity.py
(every device entry point, against the oracle, bit for bit) under the tuning
its environment holds.  A capped grid makes every workgroup walk several
chunks (the grid-stride loop and its XCD-aware chunk order); the extreme
chunk sizes move the strided-block and the chunk-edge cases.  It prints
each case before it runs and "ok" at the end; a failure raises.
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import torch  # noqa: E402

import oracle as O  # noqa: E402
import test_gpu_parity as T  # noqa: E402
from gpu_util import require_gpu  # noqa: E402

CASES = [
    ("tiny", T.test_tiny_fsdp_workload, ()),
    ("tiny misaligned", T.test_tiny_fsdp_misaligned, (3,)),
    ("ragged heavy scaled", T.test_ragged_heavy_scaled, ()),
    ("bf16 ragged all alignments", T.test_bf16_ragged_all_alignments, ()),
    ("many parameters", T.test_many_parameters_deep_chunk_search, ()),
    ("strided blocks fp32", T.test_strided_blocks_all_steps, (4, 8, torch.float32)),
    ("strided blocks bf16", T.test_strided_blocks_all_steps, (8, 8, torch.bfloat16)),
    ("non-zero dims misaligned", T.test_nonzero_shard_dims_all_steps, (4, 8, torch.float32)),
    ("short odd-pitch rows (fold items)", T.test_odd_pitch_blocks_all_steps, (4, 8, torch.bfloat16, False)),
    ("short odd-pitch rows, aligned", T.test_odd_pitch_blocks_all_steps, (2, 4, torch.bfloat16, True)),
    ("narrow fold pieces, 4-byte units", T.test_narrow_fold_paths_all_steps, (4, 8, torch.float32, True)),
    ("narrow fold pieces, runtime group size", T.test_narrow_fold_paths_all_steps, (3, 6, torch.bfloat16, True)),
    ("narrow fold pieces, operands at other offsets", T.test_narrow_fold_paths_all_steps, (8, 16, torch.bfloat16, False)),
    ("rs copy-reduce ragged", T.test_rs_copy_reduce_ragged_heavy_scaled, ()),
    ("hsdp end to end 16 = 2 x 8", T.test_hsdp_end_to_end_multi_bucket, (16, 8, O.AVG)),
    ("16-bit rs copy-in and reduce", T.test_16bit_rs_copy_in_and_reduce, (8, 4, torch.float16)),
    ("16-bit fused AR pure TP", T.test_16bit_fused_ar_pure_tp, (O.AVG, torch.bfloat16)),
    ("special values", T.test_special_values_rs_and_fused_ar, (torch.float32, 8, 4)),
]


def main():
    require_gpu()
    T.hp.lib()
    tuning = {k: v for k, v in os.environ.items() if k.startswith("FSDP_")}
    for name, fn, args in CASES:
        print(f"[tuning {tuning}] {name}", flush=True)
        fn(*args)
    T.hp.fsdp_release_cache()
    print("ok", flush=True)


if __name__ == "__main__":
    main()
