"""Host-side logic of bench.py, without a GPU: the algorithmic byte model
against the sizes of the oracle's own arrays, the staleness hash of the
traffic summaries, the overlap summary of a backward-overlap kernel trace,
the CPU baseline's sample and the refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("wname", ["tiny_fsdp_r4_s4", "hsdp_block_h1024_r8_s4_d2", "ragged_heavy_r8_s8"])
def test_step_bytes_match_the_oracles_arrays(wname):
    """Every step's algorithmic bytes = the bytes its oracle reads plus the
    bytes it writes, counted from the arrays' own sizes (tiny inputs of the
    workload's layout stand in where the workload is large: the byte model
    depends only on the layout)."""
    w = W.WORKLOADS[wname]
    R, S = w.rank_size, w.shard_size
    lay = O.bucket_layout(w.param_shapes, S)
    _, F = O.fused_layout([lay.I])
    got = bench.step_bytes(w, lay, F)
    e = 2 if "bfloat16" in str(w.param_dtype) or "float16" in str(w.param_dtype) else 4
    g = 4
    N = sum(int(np.prod(s)) for s in w.param_shapes)
    shard_elems = sum(lay.row_len[i][s] * lay.inner[i] for i in range(len(w.param_shapes)) for s in range(S))
    assert shard_elems == N
    ag_elems = S * lay.I
    full_elems = N
    rs_in_elems = R * S * lay.I
    rs_out_elems = R * lay.I
    assert got["ag_copy_in"] == shard_elems * e + ag_elems * e
    # copy-out reads only the logical rows of the gathered buffer
    assert got["ag_copy_out"] == full_elems * e + full_elems * e
    assert got["rs_copy_in"] == R * N * g + rs_in_elems * g
    assert got["rs_reduce"] == rs_in_elems * g + rs_out_elems * g
    # the fused step never writes nor reads the RS input
    assert got["rs_copy_reduce"] == got["rs_copy_in"] + got["rs_reduce"] - 2 * rs_in_elems * g
    assert got["fused_ar"] == 2 * R * F * g


def test_kernel_source_sha_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", [str(src)])
    a = bench.kernel_source_sha()
    src.write_text("/* a block\n comment */ int f(int x)   {\n\n  return x + 1;  // another\n}\n")
    assert bench.kernel_source_sha() == a
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_sha() != a


def test_measured_traffic_is_null_once_the_sources_change(tmp_path, monkeypatch):
    t = tmp_path / "l2_fabric_traffic_{workload}.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    (tmp_path / "l2_fabric_traffic_x.json").write_text(json.dumps(
        {"kernel_source_sha": bench.kernel_source_sha(), "steps": {"rs_copy_in": {"bytes_per_launch": 123}}}))
    assert bench.measured_traffic("x", "rs_copy_in") == 123
    assert bench.measured_traffic("x", "rs_reduce") is None
    assert bench.measured_traffic("absent", "rs_copy_in") is None
    (tmp_path / "l2_fabric_traffic_x.json").write_text(json.dumps(
        {"kernel_source_sha": "0" * 16, "steps": {"rs_copy_in": {"bytes_per_launch": 123}}}))
    assert bench.measured_traffic("x", "rs_copy_in") is None


def _trace_csv(path, passes):
    """A kernel trace with the columns overlap_summary reads; passes is a
    list of lists of (kernel name, start us, end us), 1 ms apart."""
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for k, p in enumerate(passes):
            base = k * 1_000_000
            for name, a, b in p:
                f.write(f"\"{name}\",{base + int(a * 1e3)},{base + int(b * 1e3)}\n")


def test_overlap_summary_finds_passes_busy_times_and_overlap(tmp_path, capsys):
    RS, AR = "void reduce_kernel<0, 4, true>(...)", "void reduce_kernel<0, 2, true>(...)"
    reps = 1
    # per case 2 (reps + 3) = 8 replays: 4 serial then 4 two-stream; an
    # earlier eager pass of the same shape is ignored
    serial = [(RS, 0, 100), (AR, 100, 150), (RS, 150, 250), (AR, 250, 300)]
    piped = [(RS, 0, 100), (AR, 60, 140), (RS, 100, 200), (AR, 180, 230)]
    other = [(RS, 0, 40), (AR, 40, 60)]
    passes = [serial] + [serial] * 4 + [piped] * 4 + [other] * 8
    csv = tmp_path / "trace_kernel_trace.csv"
    _trace_csv(csv, passes)
    bench.overlap_summary(str(csv), reps)
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    cases = {c["kernels_per_pass"]: c for c in out["cases"]}
    four = cases[4]
    assert four["serial"] == {"pass_us": 300, "rs_busy_us": 200, "ar_busy_us": 100, "overlap_us": 0, "passes": 4}
    # RS busy [0, 200], AR busy [60, 140] and [180, 230]: overlap 80 + 20
    assert four["pipelined"] == {"pass_us": 230, "rs_busy_us": 200, "ar_busy_us": 130, "overlap_us": 100,
                                 "passes": 4}
    assert cases[2]["serial"]["pass_us"] == 60 and cases[2]["pipelined"]["overlap_us"] == 0


def test_cpu_baseline_sample():
    """The Llama-7B-shaped bucket's sample is exactly its first layer; small
    buckets are taken whole."""
    w = W.WORKLOADS["llama7b_4layer_r8_s8"]
    k = bench.sample_shapes(w)
    assert k == 9 and w.param_shapes[:9] == w.param_shapes[9:18]
    for name in ("tiny_fsdp_r4_s4", "hsdp_block_h1024_r8_s4_d2"):
        w = W.WORKLOADS[name]
        assert bench.sample_shapes(w) == len(w.param_shapes)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
