"""Build the gfx950 shared library libfsdpflat.so in-tree with hipcc.

    python -m hsdp_parameter_gradient_amd.build

Every call compiles from source (no up-to-date check); the library is
written to a temporary name and renamed into place, so a process that has
the old library loaded keeps a consistent file.  The compiler's resource
report of every kernel (registers, occupancy, LDS, private scratch) is
written beside it as kernel_resources.json.
"""

from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libfsdpflat.so"
RESOURCES = "kernel_resources.json"
_REMARK = "kernel-resource-usage"
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs", "ScratchSize [bytes/lane]": "scratch_bytes",
           "Occupancy [waves/SIMD]": "waves_per_simd", "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}
SOURCES = ("fsdp_flat.cpp", "kernels.hip")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # IEEE fp32 everywhere: keep denormals, correctly rounded division
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfsdpflat.so)")


def parse_resources(stderr: str) -> dict:
    """Per-kernel figures of hipcc's kernel-resource-usage remarks, keyed by
    the mangled kernel name."""
    out, cur = {}, None
    for line in stderr.splitlines():
        if _REMARK not in line:
            continue
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\w+) \[", line)
        if m and cur is not None and m.group(1) in _FIELDS:
            v = m.group(2)
            cur[_FIELDS[m.group(1)]] = int(v) if v.isdigit() else v
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    out = os.path.join(LIB_DIR, LIB_NAME)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp, "-Rpass-analysis=" + _REMARK]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "not a recognized feature for this target"
    warn = "\n".join(l for l in (r.stderr or "").splitlines()
                     if noise not in l and "ignoring feature" not in l and _REMARK not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.unlink(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (r.returncode, r.stdout, warn))
    if verbose and warn.strip():
        print(warn, file=sys.stderr)
    res = parse_resources(r.stderr or "")
    rtmp = os.path.join(LIB_DIR, RESOURCES + ".tmp%d" % os.getpid())
    with open(rtmp, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    os.replace(tmp, out)
    os.replace(rtmp, os.path.join(LIB_DIR, RESOURCES))
    return out


if __name__ == "__main__":
    print(build(verbose=True))
