"""The compiler's resource report of the built kernels (written by the build
as lib/kernel_resources.json): no kernel uses private scratch memory (a
register spill or a lane-indexed private array would add memory traffic to
HBM-bound streams), every kernel of the path keeps at least 4 waves per SIMD,
and the LDS a workgroup declares fits several workgroups per CU."""

import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RES = os.path.join(ROOT, "hsdp_parameter_gradient_amd", "lib", "kernel_resources.json")
KERNELS = ("seg_copy_kernel", "reduce_kernel", "fold_copy_kernel", "fold_reduce_kernel", "table_write_kernel")
LDS_PER_CU = 160 * 1024


@pytest.fixture(scope="module")
def res():
    if not os.path.exists(RES):
        pytest.skip("the library has not been built here (hsdp_parameter_gradient_amd.build writes the report)")
    with open(RES) as f:
        r = json.load(f)
    assert r, "empty resource report"
    return r


def test_every_kernel_is_reported(res):
    for k in KERNELS:
        assert any(k in name for name in res), f"{k} missing from the resource report"


def test_no_private_scratch(res):
    bad = {n: v for n, v in res.items() if v.get("scratch_bytes", 0) or v.get("vgpr_spill", 0)}
    assert not bad, f"kernels using private scratch: {bad}"


def test_occupancy_and_lds(res):
    for n, v in res.items():
        if not any(k in n for k in KERNELS):
            continue
        assert v["waves_per_simd"] >= 4, (n, v)
        assert v["lds_bytes"] * 4 <= LDS_PER_CU, (n, v)
