"""GPU parity under other launch tunings, one child process each.

The default launch (one workgroup per chunk, 16 KiB copy and 8 KiB reduce
chunks) never makes a workgroup take a second chunk below 2^22 chunks.
These runs cap the grid (so every workgroup walks the grid-stride loop, on
a grid that is or is not a multiple of the 8 XCDs) and move both chunk
sizes to the extremes the tuning accepts, and check the same parity cases
bit for bit against the oracle (tests/gpu_tuning_child.py).
"""

import os
import subprocess
import sys

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

TUNINGS = {
    "grid_8": {"FSDP_MAX_GRID": "8"},
    "grid_5": {"FSDP_MAX_GRID": "5"},
    "grid_1000": {"FSDP_MAX_GRID": "1000"},
    "chunks_512B": {"FSDP_COPY_CHUNK_SHIFT": "9", "FSDP_REDUCE_CHUNK_SHIFT": "9"},
    "chunks_1MiB_grid_64": {"FSDP_COPY_CHUNK_SHIFT": "20", "FSDP_REDUCE_CHUNK_SHIFT": "20", "FSDP_MAX_GRID": "64"},
}


@pytest.mark.parametrize("tuning", list(TUNINGS))
def test_parity_under_tuning(tuning):
    require_gpu()
    env = {k: v for k, v in os.environ.items() if not k.startswith("FSDP_")}
    env.update(TUNINGS[tuning])
    print(f"[gpu tuning] {tuning}: {TUNINGS[tuning]}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "gpu_tuning_child.py")], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.rstrip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
