#!/usr/bin/env python3
"""Benchmark of the FSDP/HSDP flat-buffer hot path on one MI355X.

One step is one pass of the whole hot path over one bucket, inputs already
resident in HBM: AG copy-in (pack the shards of all S ranks into the padded
AG buffer), AG copy-out (unpack into the full parameters), RS copy-in (chunk
the R ranks' full gradients into their padded RS inputs), RS over every
shard group into views of the 512-byte-aligned fused buffers, and the fused
AR over every replicate group when dp_size > 1.  The headline workload is
the 4-layer Llama-7B-shaped bucket (hidden 4096, ffn 11008; rank_size 8 =
shard_size 8; bf16 parameters, fp32 gradients, AVG): 84 GB per step, far
beyond the 256 MB Infinity Cache, so HBM sets the rate.

value = algorithmic bytes of one step x steps / time (GB/s, whole job).
Algorithmic bytes count every required read and write once (padding is
written, never read as a copy source):
  AG copy-in   sum(N_i) e + S I e         AG copy-out  2 sum(N_i) e
  RS copy-in   4 R (sum(N_i) + S I)       RS reduce    4 R S I + 4 R I
  fused AR     8 R F
Timing: W untimed steps, then K steps between synchronisations (the value);
inside them the dominant kernel (found on a few untimed steps) records a pair
of HIP events in its own dispatch, at its start and its end
(fsdp_time_next_launch), which give its average launch time (the roofline); a
separate pass afterwards gives every step's time (the "ops" breakdown), and
medians of single launches with the Infinity Cache flushed first (cold) or
not (warm).  A 4 GiB device-to-device copy (hipMemcpyAsync, and the
library's copy kernel) gives the plain-copy ceiling.
The CPU oracle is timed on whole steps of a bounded sample of the same
workload (cpu_baseline: its first layer).  The other workloads (the HSDP
block, which alone runs all five steps and carries the variants; the
ragged-heavy set; the pure-TP AR; the tiny bucket) follow under
"other_workloads", each with its own pass, dominant kernel and breakdown.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (and % of peak) for AG copy-in/out + RS/AR reduce per bucket"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_OF_STEP = {"ag_copy_in": "seg_copy_kernel", "ag_copy_out": "seg_copy_kernel",
                  "rs_copy_in": "seg_copy_kernel", "rs_reduce": "reduce_kernel",
                  "rs_copy_reduce": "reduce_kernel", "fused_ar": "reduce_kernel"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "l2_fabric_traffic_{workload}.json")
# what fixes the kernels' memory traffic: their code, the descriptor formats,
# the launch tuning (chunk sizes, store policy) and the planner that builds
# the tables
KERNEL_SRC = [os.path.join(ROOT, "hsdp_parameter_gradient_amd", "csrc", f)
              for f in ("kernels.hip", "plan.hpp", "tuning.hpp", "fsdp_flat.cpp")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the code (comments and whitespace removed) of the sources that
    fix the kernels' traffic, so that editing a comment keeps the measured
    traffic valid."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SRC:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def step_bytes(w, lay, F: int, grad_bytes: int = 4):
    """Algorithmic bytes of every step (e = parameter element size, g =
    gradient element size)."""
    import torch
    e = 2 if w.param_dtype in (torch.bfloat16, torch.float16) else 4
    g = grad_bytes
    R, S, I = w.rank_size, w.shard_size, lay.I
    N = sum(_numel(s) for s in w.param_shapes)
    return {
        "ag_copy_in": N * e + S * I * e,
        "ag_copy_out": 2 * N * e,
        "rs_copy_in": g * R * (N + S * I),
        "rs_reduce": g * R * S * I + g * R * I,
        "rs_copy_reduce": g * R * N + g * R * I,
        "fused_ar": 2 * g * R * F,
    }


def _numel(shape):
    n = 1
    for d in shape:
        n *= d
    return n


def measured_traffic(workload: str, step: str):
    """Bytes per launch of the dominant kernel between L2 and the memory
    fabric (rocprofv3 FETCH_SIZE + WRITE_SIZE, each scaled by what it reads
    for a plain copy of known size) from the committed PMC summary, or None
    when absent or when the kernel source has changed since the counters
    were taken.  The counters see L2 misses, Infinity Cache hits included:
    no per-kernel DRAM byte counter exists on this ROCm."""
    try:
        with open(TRAFFIC_FILE.format(workload=workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    ent = t.get("steps", {}).get(step)
    if not ent:
        return None
    return ent.get("bytes_per_launch")


class PureTPRunner:
    """shard_size 1 (pure-TP compatible path): no AG and no RS; every
    gradient is one 512-byte-aligned segment of its rank's fused buffer and
    one fused AR over the replicate group (all R ranks) is the whole step."""

    def __init__(self, w, op):
        import torch

        import hsdp_parameter_gradient_amd as hp
        import workloads as W
        R = w.rank_size
        sizes = [_numel(s) for s in w.param_shapes]
        self.layout = hp.fsdp_bucket_layout(w.param_shapes, 1)
        offs, self.F = hp.fsdp_fused_layout(sizes, 4)
        grads = W.grads(w, "cuda")
        self.fused = []
        for g in range(R):
            buf = torch.zeros(self.F, dtype=torch.float32, device="cuda")
            for o, t in zip(offs, grads[g]):
                buf[o:o + t.numel()] = t.reshape(-1)
            self.fused.append(buf)
        del grads
        self.call = hp.prepare("fsdp_fused_ar", sizes, R, 1, R, op, self.fused)

    def steps(self):
        return ["fused_ar"]

    def run(self, name, stream=None):
        self.call(stream)

    def step(self, stream=None):
        self.call(stream)


def timing_events(n):
    """n pairs of timing events, created (recorded once) so that a kernel's
    dispatch can record them (fsdp_time_next_launch)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        b.record()
    return ev


def per_step_us(runner, steps, n):
    """Average duration (us) of every step's kernel over n passes, from the
    HIP events each kernel's own dispatch records at its start and end."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    flat = timing_events(n * len(steps))
    ev = [flat[k * len(steps):(k + 1) * len(steps)] for k in range(n)]
    torch.cuda.synchronize()
    for k in range(n):
        for j, name in enumerate(steps):
            hp.fsdp_time_next_launch(*ev[k][j])
            runner.run(name)
    torch.cuda.synchronize()
    return {name: sum(ev[k][j][0].elapsed_time(ev[k][j][1]) for k in range(n)) / n * 1e3
            for j, name in enumerate(steps)}


def op_medians(runner, steps, reps: int, flush):
    """Median single-launch duration (us) of every step, cold and warm: a
    cold launch follows a read of a scratch buffer four times the 256 MB
    Infinity Cache (so the caches hold clean, unrelated lines: neither the
    step's inputs nor its outputs), a warm one follows a launch of the same
    step."""
    import statistics

    import torch

    import hsdp_parameter_gradient_amd as hp
    out = {}
    a, b = timing_events(1)[0]
    for name in steps:
        res = {}
        for mode in ("cold", "warm"):
            t = []
            for _ in range(reps):
                if mode == "cold":
                    flush.sum()
                else:
                    runner.run(name)
                hp.fsdp_time_next_launch(a, b)
                runner.run(name)
                torch.cuda.synchronize()
                t.append(a.elapsed_time(b) * 1e3)
            res[mode] = statistics.median(t)
        out[name] = res
    return out


def copy_ceiling(mib: int, reps: int):
    """Device-to-device copy of mib MiB with hipMemcpyAsync (torch's copy_
    of a contiguous tensor) and with the library's copy kernel (one aligned
    segment): read + write GB/s, the achievable ceiling of a plain copy."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    call = hp.prepare("fsdp_ag_copy_out", [(n,)], 1, a, [b])
    out = {"bytes_each_way": 4 * n}
    for name, fn in (("hipMemcpyAsync_DtoD", lambda: b.copy_(a)), ("seg_copy_kernel", lambda: call())):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) / reps * 1e3
        out[name] = {"us": round(us, 1), "GB/s": round(2 * 4 * n / (us * 1e-6) / 1e9, 1)}
    del a, b
    torch.cuda.empty_cache()
    log(f"  copy ceiling ({mib} MiB): hipMemcpyAsync {out['hipMemcpyAsync_DtoD']['GB/s']} GB/s, "
        f"seg_copy_kernel {out['seg_copy_kernel']['GB/s']} GB/s")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bucket_variant(w, op, K: int, warmup: int, grad_dtype=None, shard_dims=None):
    """The whole pass of the workload with 16-bit gradients (reduce dtype
    bf16 or fp16), or with the 2-D parameters sharded on dim 1: time per
    pass, GB/s of its algorithmic bytes, and each step's time."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W
    R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
    gdt = grad_dtype or torch.float32
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=op, grad_dtype=gdt, shard_dims=shard_dims)
    params = W.params(w, "cuda")
    grads = W.grads(w, "cuda", dtype=gdt)
    fb.bind(fb.shard_views(params), [grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
    steps = fb.steps()
    nbytes = step_bytes(w, fb.layout, fb.F, gdt.itemsize)
    total = sum(nbytes[s] for s in steps)
    for _ in range(warmup):
        fb.step()
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    for _ in range(K):
        fb.step()
    e0.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / K
    per = per_step_us(fb, steps, K)
    out = {"grad_dtype": str(gdt).replace("torch.", ""), "shard_dims": shard_dims, "ms_per_step": round(ms, 4),
           "bytes_per_step": total, "GB/s": round(total / (ms * 1e-3) / 1e9, 1),
           "ops": {n: {"us": round(per[n], 2), "GB/s": round(nbytes[n] / (per[n] * 1e-6) / 1e9, 1)} for n in steps}}
    log(f"  variant grad_dtype={out['grad_dtype']} shard_dims={shard_dims}: step {ms * 1e3:.1f} us, "
        f"{out['GB/s']:.1f} GB/s")
    return out


def zero_copy_ag_variant(w, op, reps: int):
    """The forward AG of the workload with one bucket per parameter: AG
    copy-in + copy-out per bucket, against AG copy-in alone with each
    parameter used as the zero-copy prefix view of its gathered buffer."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W
    R, S = w.rank_size, w.shard_size
    params = W.params(w, "cuda")
    buckets = []
    for sh, p in zip(w.param_shapes, params):
        fb = hp.FlatBucket([sh], R, S, w.param_dtype, op=op)
        g0 = torch.zeros(p.numel(), device="cuda")  # the AG steps read no gradient
        fb.bind(fb.shard_views([p]), [g0] * R)
        fb.full_views()  # a one-parameter bucket: the view is valid
        buckets.append(fb)
    out = {"buckets": len(buckets)}
    passes = {"copy_in_and_out": ("ag_copy_in", "ag_copy_out"), "zero_copy_views": ("ag_copy_in",)}
    for name, steps in passes.items():
        def run():
            for fb in buckets:
                for st in steps:
                    fb.run(st)
        for _ in range(3):
            run()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            run()
        e0.record()
        torch.cuda.synchronize()
        out[name + "_us"] = round(s0.elapsed_time(e0) / reps * 1e3, 1)
    log(f"  zero-copy AG, one bucket per parameter: copy-in + copy-out {out['copy_in_and_out_us']:.1f} us, "
        f"copy-in with views {out['zero_copy_views_us']:.1f} us")
    return out


def fused_group_variant(w, op, reps: int, warmup: int):
    """The pass with one bucket per parameter whose RS outputs share one
    512-byte-aligned fused buffer and one fused AR (FusedGroup): time per
    pass and GB/s of its algorithmic bytes."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W
    R, S = w.rank_size, w.shard_size
    buckets = [[sh] for sh in w.param_shapes]
    grp = hp.FusedGroup(buckets, R, S, w.param_dtype, op=op)
    params = W.params(w, "cuda")
    grads = W.grads(w, "cuda")
    grp.bind([fb.shard_views([params[k]]) for k, fb in enumerate(grp.buckets)],
             [[grads[g][k].reshape(-1) for g in range(R)] for k in range(len(buckets))])
    total = 0
    for k, fb in enumerate(grp.buckets):
        wk = dataclasses_replace(w, param_shapes=(w.param_shapes[k],))
        nb = step_bytes(wk, fb.layout, 0)
        total += sum(nb[s] for s in ("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"))
    if grp.do_ar:
        total += 8 * R * grp.fused[0].numel()
    for _ in range(warmup):
        grp.step()
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    for _ in range(reps):
        grp.step()
    e0.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(e0) / reps
    graph = grp.graph(n_streams=3)
    for _ in range(warmup):
        graph.replay()
    s1, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s1.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = s1.elapsed_time(e1) / reps
    del graph
    out = {"buckets": len(buckets), "fused_numel": grp.fused[0].numel(), "ms_per_step": round(ms, 4),
           "bytes_per_step": total, "GB/s": round(total / (ms * 1e-3) / 1e9, 1),
           "graph_3_streams_ms_per_step": round(gms, 4),
           "graph_3_streams_GB/s": round(total / (gms * 1e-3) / 1e9, 1)}
    log(f"  one bucket per parameter, one fused AR: step {ms * 1e3:.1f} us, {out['GB/s']:.1f} GB/s; "
        f"replayed from a graph over 3 streams {gms * 1e3:.1f} us")
    return out


def dataclasses_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def pipeline_variant(w, op, layers: int, reps: int):
    """The backward of `layers` buckets of this workload (RS copy-reduce of
    each layer, fused AR of the previous layer): serial on one stream vs the
    4-step overlap on two streams (BackwardPipeline), issued eagerly and
    replayed from a captured HIP graph."""
    import dataclasses

    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W
    R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
    buckets = []
    for l in range(layers):
        wl = dataclasses.replace(w, number=w.number * 1000 + l)
        fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=op)
        params = [torch.zeros(sh, dtype=w.param_dtype, device="cuda") for sh in w.param_shapes]
        grads = W.grads(wl, "cuda")
        fb.bind(fb.shard_views(params), [grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
        buckets.append(fb)
    pipe = hp.BackwardPipeline(buckets, fused_rs=True)
    out = {"layers": layers}
    g_serial, g_pipe = pipe.graph(pipelined=False), pipe.graph(pipelined=True)
    for name, fn in (("serial_ms", pipe.run_serial), ("pipelined_ms", pipe.run_pipelined),
                     ("graph_serial_ms", g_serial.replay), ("graph_pipelined_ms", g_pipe.replay)):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        out[name] = round(s.elapsed_time(e) / reps, 4)
    del g_serial, g_pipe
    log(f"  backward pipeline, {layers} layers: serial {out['serial_ms']:.3f} ms, "
        f"two streams {out['pipelined_ms']:.3f} ms; replayed from a HIP graph: serial "
        f"{out['graph_serial_ms']:.3f} ms, two streams {out['graph_pipelined_ms']:.3f} ms")
    return out


def graph_variant(runner, reps: int, warmup: int):
    """The contract's pass captured once in a HIP graph (torch.cuda.graph)
    and replayed: the same kernels with the same arguments, launched by the
    graph instead of one host call each.  Plans are cached by the eager
    passes before, so the capture records kernel launches only."""
    import torch
    graph = torch.cuda.CUDAGraph()
    runner.step()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        runner.step()
    for _ in range(max(1, warmup)):
        graph.replay()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del graph
    log(f"  HIP graph variant: step {ms * 1e3:.1f} us")
    return {"ms_per_step": round(ms, 4), "note": "one graph replay per pass, same kernels and arguments"}


def calibration_copy(mib: int, reps: int) -> None:
    """A plain copy of known size for calibrating the HBM byte counters: the
    copy kernel on one aligned fp32 segment (AG copy-out with one shard), so
    each launch reads and writes exactly mib MiB."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    n = mib * (1 << 20) // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    call = hp.prepare("fsdp_ag_copy_out", [(n,)], 1, a, [b])
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    print(json.dumps({"calibration_copy": {"bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                                           "launches": reps, "grid": -(-4 * n // (1 << 14))}}), flush=True)


# Parameters sharded on dim 1 whose chunk rows are short or sit at per-row
# alignments (the fold kernels' cases, the last two with rows too long for
# one chunk: flat chunks), with a control of 16-byte-aligned rows:
# (shapes, S, R, dtype name).
FOLD_SHAPES = [
    ([(8000000, 6)], 2, 2, "float32"),
    ([(4000000, 12, 3)], 4, 4, "bfloat16"),
    ([(1000000, 32)], 4, 4, "float32"),
    ([(500000, 48)], 8, 16, "float16"),
    ([(30000, 2050, 1)], 2, 2, "bfloat16"),
    ([(20000, 1540)], 4, 4, "bfloat16"),
    ([(20000, 1030, 4)], 2, 2, "float16"),
    ([(20000, 1024)], 4, 4, "bfloat16"),
    ([(10000, 4098)], 2, 2, "float32"),
    ([(3000, 8248)], 8, 8, "bfloat16"),
]


def fold_shapes(reps: int) -> None:
    """AG copy-out, RS copy-in and RS copy-reduce of every FOLD_SHAPES case
    (one parameter sharded on dim 1, SUM): prepared calls issued back to
    back, events around `reps` calls of each step, one JSON line."""
    import torch

    import hsdp_parameter_gradient_amd as hp
    out = []
    for shapes, S, R, dt_name in FOLD_SHAPES:
        dt = getattr(torch, dt_name)
        n = _numel(shapes[0])
        dims = [1]
        I = hp.fsdp_bucket_layout(shapes, S, shard_dims=dims).I
        e = torch.empty(0, dtype=dt).element_size()
        ag = torch.randn(S * I, device="cuda").to(dt)
        full = [torch.empty(n, dtype=dt, device="cuda")]
        g = [torch.randn(n, device="cuda").to(dt) for _ in range(R)]
        rs_in = [torch.empty(S * I, dtype=dt, device="cuda") for _ in range(R)]
        rs_out = [torch.empty(I, dtype=dt, device="cuda") for _ in range(R)]
        calls = {"ag_copy_out": (hp.prepare("fsdp_ag_copy_out", shapes, S, ag, full, dims), 2 * n * e),
                 "rs_copy_in": (hp.prepare("fsdp_rs_copy_in", shapes, R, S, g, rs_in, dims), R * (n + S * I) * e),
                 "rs_copy_reduce": (hp.prepare("fsdp_rs_copy_reduce", shapes, R, S, R // S, "sum", g, rs_out, dims),
                                    R * (n + I) * e)}
        res = {}
        for step, (call, nbytes) in calls.items():
            for _ in range(3):
                call()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            for _ in range(reps):
                call()
            b.record()
            b.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            res[step] = {"us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log(f"  {shapes[0]} {dt_name} S={S} R={R}: " +
            ", ".join(f"{k} {v['us']:.1f} us ({v['GB/s']:.0f} GB/s)" for k, v in res.items()))
        out.append({"shape": list(shapes[0]), "shard_dim": 1, "S": S, "R": R, "dtype": dt_name, "ops": res})
        del ag, full, g, rs_in, rs_out, calls
    hp.fsdp_release_cache()
    print(json.dumps({"fold_shapes": out, "timing": f"events around {reps} back-to-back prepared calls"}), flush=True)


def pipeline_cases():
    """The backward-overlap cases: 8 layers of the HSDP block, and 2 layers
    shaped like one Llama-7B layer each (its q, k, v, o, gate, up, down and
    two norms) in the same HSDP configuration (rank_size 8 = 2 x 4), since
    the 4-layer bucket itself has no replicate group (dp_size 1)."""
    import dataclasses

    import workloads as W
    blk = W.HSDP_BLOCK
    llama_layer = dataclasses.replace(blk, name="llama7b_layer_r8_s4_d2", number=6,
                                      param_shapes=W.LLAMA7B_4L.param_shapes[:9],
                                      param_dtype=W.LLAMA7B_4L.param_dtype)
    return [(blk, 8), (llama_layer, 2)]


def pipeline_trace(reps: int) -> None:
    """Replays of the captured backward (RS copy-reduce of each layer, fused
    AR of the previous one; BackwardPipeline) for every pipeline case:
    first the serial graph, then the two-stream graph, `reps` timed replays
    each after 3 untimed ones, a synchronisation after every replay (so
    that a kernel trace of this command shows the passes apart).  Prints
    one JSON line with the median pass times."""
    import statistics

    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W
    out = []
    for w, layers in pipeline_cases():
        R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
        buckets = []
        for l in range(layers):
            wl = dataclasses_replace(w, number=w.number * 1000 + l)
            fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=bench_op(w))
            params = [torch.zeros(sh, dtype=w.param_dtype, device="cuda") for sh in w.param_shapes]
            grads = W.grads(wl, "cuda")
            fb.bind(fb.shard_views(params), [grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
            buckets.append(fb)
        pipe = hp.BackwardPipeline(buckets, fused_rs=True)
        res = {"case": w.name, "layers": layers, "rank_size": R, "shard_size": S, "dp_size": R // S}
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for name, pipelined in (("serial", False), ("pipelined", True)):
            g = pipe.graph(pipelined=pipelined)
            for _ in range(3):
                g.replay()
                torch.cuda.synchronize()
            t = []
            for _ in range(reps):
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                t.append(a.elapsed_time(b))
            res[name + "_ms_median"] = round(statistics.median(t), 4)
            del g
        log(f"  {w.name} x {layers} layers: graph replay serial {res['serial_ms_median']:.3f} ms, "
            f"two streams {res['pipelined_ms_median']:.3f} ms")
        out.append(res)
        del pipe, buckets
        hp.fsdp_release_cache()
        torch.cuda.empty_cache()
    print(json.dumps({"pipeline_trace": out, "replays_per_order": reps}), flush=True)


def overlap_summary(csv_path: str, reps: int, gap_us: float = 15.0) -> None:
    """Reads a rocprofv3 kernel trace (trace_kernel_trace.csv) of
    `bench.py --pipeline-trace --steps reps` and finds its passes (told apart
    by idle gaps of more than gap_us); per pass, the pass time, the busy
    time of the RS copy-reduce kernels (4 operands) and of the fused AR
    kernels (2 operands), and the time both run at once.  Per case (the
    passes with one kernel count), its last 2 (reps + 3) passes are the
    replays, the serial graph's then the two-stream graph's; prints their
    medians.  One JSON line."""
    import statistics
    import csv
    ev = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            kind = "rs" if "reduce_kernel<0, 4" in name else "ar" if "reduce_kernel<0, 2" in name else None
            if kind:
                ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind))
    ev.sort()
    passes, cur, end = [], [], 0
    for e in ev:
        if cur and e[0] - end > gap_us * 1e3:
            passes.append(cur)
            cur = []
        end = max(end, e[1]) if cur else e[1]
        cur.append(e)
    if cur:
        passes.append(cur)

    def union(iv):
        iv = sorted(iv)
        out = []
        for a, b in iv:
            if out and a <= out[-1][1]:
                out[-1][1] = max(out[-1][1], b)
            else:
                out.append([a, b])
        return out

    def inter(x, y):
        i = j = 0
        tot = 0
        while i < len(x) and j < len(y):
            lo, hi = max(x[i][0], y[j][0]), min(x[i][1], y[j][1])
            tot += max(0, hi - lo)
            if x[i][1] < y[j][1]:
                i += 1
            else:
                j += 1
        return tot

    rows = []
    for p in passes:
        rs = union([(a, b) for a, b, k in p if k == "rs"])
        ar = union([(a, b) for a, b, k in p if k == "ar"])
        rows.append({"kernels": len(p), "pass_us": (max(b for _, b, _ in p) - p[0][0]) / 1e3,
                     "rs_busy_us": sum(b - a for a, b in rs) / 1e3, "ar_busy_us": sum(b - a for a, b in ar) / 1e3,
                     "overlap_us": inter(rs, ar) / 1e3})
    cases = []
    for nk in dict.fromkeys(r["kernels"] for r in rows if r["kernels"] > 1):
        sel = [r for r in rows if r["kernels"] == nk][-2 * (reps + 3):]
        half = len(sel) // 2
        case = {"kernels_per_pass": nk}
        for order, part in (("serial", sel[:half]), ("pipelined", sel[half:])):
            case[order] = {k: round(statistics.median(r[k] for r in part), 2)
                           for k in ("pass_us", "rs_busy_us", "ar_busy_us", "overlap_us")}
            case[order]["passes"] = len(part)
        cases.append(case)
    print(json.dumps({"trace": csv_path, "cases": cases}), flush=True)


def sample_shapes(w):
    """The CPU baseline's sample of a workload: the whole bucket when it has
    at most 64 M elements, else its leading parameters up to a quarter of
    its elements (for the 4-layer Llama-7B-shaped bucket: exactly its first
    layer, 9 parameters)."""
    n_all = sum(_numel(s) for s in w.param_shapes)
    if n_all <= 64 << 20:
        return len(w.param_shapes)
    k, n = 0, 0
    while k < len(w.param_shapes) and (k == 0 or n + _numel(w.param_shapes[k]) <= n_all // 4):
        n += _numel(w.param_shapes[k])
        k += 1
    return k


def cpu_baseline(w, seconds: float, op: str, params, grads):
    """The oracle, as it stands, timed on whole steps of a bounded sample of
    the workload (sample_shapes: its leading parameters, the same ranks, the
    same values, copied from the device tensors the GPU pass used), and on
    each of the step's operations (perf_counter around each oracle call).
    Returns (parameters in the sample, steps run, seconds, bytes per sample
    step, seconds per operation)."""
    import dataclasses

    import numpy as np
    import torch

    import oracle as O

    R, S = w.rank_size, w.shard_size
    k = sample_shapes(w)
    ws = dataclasses.replace(w, param_shapes=tuple(w.param_shapes[:k]))
    lay = O.bucket_layout(ws.param_shapes, S)
    if w.param_dtype == torch.float32:
        xs = [p.cpu().numpy() for p in params[:k]]
        np_dt = np.float32
    else:
        xs = [p.view(torch.int16).cpu().numpy().view(np.uint16) for p in params[:k]]
        np_dt = np.uint16
    gnp = [[t.cpu().numpy() for t in grads[g][:k]] for g in range(R)]
    do_ar = bool([c for c in O.grad_sync_plan(R, S) if c[0] == "AR"])

    if S == 1:  # pure-TP compatible path: the fused AR is the whole step
        sizes = [_numel(s) for s in ws.param_shapes]
        offs, F = O.fused_layout(sizes)
        fused0 = []
        for g in range(R):
            buf = np.zeros(F, np.float32)
            for o, t in zip(offs, gnp[g]):
                buf[o:o + t.size] = t.reshape(-1)
            fused0.append(buf)
    else:
        offs, F = O.fused_layout([lay.I])
    nb = step_bytes(ws, lay, F)
    steps = ["fused_ar"] if S == 1 else (["ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"] +
                                        (["fused_ar"] if do_ar else []))
    per = {}

    def timed(name, fn, *a):
        t = time.perf_counter()
        r = fn(*a)
        per[name] = per.get(name, 0.0) + time.perf_counter() - t
        return r

    def pure_tp_step():
        timed("fused_ar", O.fused_ar, fused0, R, S, op)

    def hsdp_step():
        ag = timed("ag_copy_in", lambda: O.ag_copy_in(O.shard_params(xs, lay), lay, np_dt))
        timed("ag_copy_out", lambda: O.ag_copy_out(O.all_gather(ag), lay))
        rs_in = timed("rs_copy_in", lambda: [O.rs_copy_in(gnp[g], lay) for g in range(R)])
        out = timed("rs_reduce", O.rs_reduce, rs_in, lay.I, R, S, op)
        del rs_in
        if do_ar:
            fused = []
            for g in range(R):
                buf = np.zeros(F, np.float32)
                buf[offs[0]:offs[0] + lay.I] = out[g]
                fused.append(buf)
            timed("fused_ar", O.fused_ar, fused, R, S, op)

    one_step = pure_tp_step if S == 1 else hsdp_step
    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 200:
            break
    return k, n, el, sum(nb[s] for s in steps), {s: (per[s] / n, nb[s]) for s in steps}


def frac_vs(achieved: float, ceiling) -> dict:
    """A rate against the published peak and, when measured, against the
    same run's plain 4 GiB copy with the library's copy kernel."""
    out = {"frac_of_peak": round(achieved / HBM_PEAK_GBS, 4)}
    if ceiling:
        c = ceiling["seg_copy_kernel"]["GB/s"]
        out["frac_of_copy_ceiling"] = round(achieved / c, 4)
    return out


class Pass:
    """One workload's whole pass on the GPU: the runner, its inputs (kept
    for the CPU baseline's sample) and the byte model."""

    def __init__(self, w, op):
        import torch

        import hsdp_parameter_gradient_amd as hp
        import workloads as W
        self.w, self.op = w, op
        R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
        if S > 1:
            fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=op)
            self.params = W.params(w, "cuda")
            self.grads = W.grads(w, "cuda")
            fb.bind(fb.shard_views(self.params), [self.grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
            self.runner = fb
            self.lay, self.F = fb.layout, fb.F
        else:
            self.runner = PureTPRunner(w, op)
            self.lay, self.F = self.runner.layout, self.runner.F
            self.params = None
            self.grads = None
        self.steps = self.runner.steps()
        self.nbytes = step_bytes(w, self.lay, self.F)
        self.bytes_per_step = sum(self.nbytes[s] for s in self.steps)
        torch.cuda.synchronize()

    def measure(self, K: int, warmup: int, cold_warm_reps: int):
        """W untimed steps, then K timed steps between synchronisations, the
        dominant kernel's own dispatch recording its start and end in every
        timed step; then the per-step breakdown and, if asked, the cold and
        warm single-launch medians."""
        import torch

        import hsdp_parameter_gradient_amd as hp
        runner, steps, nbytes = self.runner, self.steps, self.nbytes
        for _ in range(warmup):
            runner.step()
        torch.cuda.synchronize()
        # a few untimed steps with events around every step find the dominant
        # kernel; the timed region then records events around that one only
        probe = per_step_us(runner, steps, max(3, warmup))
        dom = max(steps, key=probe.get)
        ev = timing_events(K)  # the dominant kernel's dispatch records these
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for k in range(K):
            for name in steps:
                if name == dom:
                    hp.fsdp_time_next_launch(ev[k][0], ev[k][1])
                runner.run(name)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start.elapsed_time(end)
        res = {"ms_per_step": total_ms / K, "wall_s": wall, "dominant": dom,
               "value": self.bytes_per_step * K / (total_ms * 1e-3) / 1e9,
               "dom_us": sum(a.elapsed_time(b) for a, b in ev) / K * 1e3}
        # per-step breakdown, measured after the timed region (events around
        # every step perturb the whole-step time, so they stay out of it)
        after = per_step_us(runner, steps, K)
        ops = {}
        for name in steps:
            us = after[name]
            gbs = nbytes[name] / (us * 1e-6) / 1e9
            ops[name] = {"kernel": KERNEL_OF_STEP[name], "bytes": nbytes[name], "us": round(us, 2),
                         "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
            log(f"  {name:12s} {nbytes[name] / 1e6:10.1f} MB  {us:9.1f} us  {gbs:8.1f} GB/s  "
                f"{100 * gbs / HBM_PEAK_GBS:5.1f}% of peak")
        res["ops"] = ops
        cw = {}
        if cold_warm_reps > 0:
            flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
            med = op_medians(runner, steps, cold_warm_reps, flush)
            del flush
            for name in steps:
                cw[name] = {m: {"us": round(med[name][m], 2),
                                "GB/s": round(nbytes[name] / (med[name][m] * 1e-6) / 1e9, 1)}
                            for m in ("cold", "warm")}
                log(f"  {name:12s} median of {cold_warm_reps}: cold {med[name]['cold']:8.1f} us "
                    f"({cw[name]['cold']['GB/s']:7.1f} GB/s), warm {med[name]['warm']:8.1f} us "
                    f"({cw[name]['warm']['GB/s']:7.1f} GB/s)")
        res["cold_warm"] = cw or None
        log(f"  step: {res['ms_per_step'] * 1e3:.1f} us, {res['value']:.1f} GB/s; wall {wall:.3f} s for {K} steps")
        return res

    def roofline(self, res, ceiling):
        dom = res["dominant"]
        achieved = self.nbytes[dom] / (res["dom_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": KERNEL_OF_STEP[dom], "step": dom,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(self.w.name, dom),
                "traffic_note": "L2-to-fabric bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a plain "
                                "copy); Infinity Cache hits are included, so not DRAM bytes",
                "algorithmic_bytes_per_launch": self.nbytes[dom], "avg_launch_us": round(res["dom_us"], 2),
                "timing": "HIP events recorded by the call's own kernel dispatch at its start and end, "
                          "every timed step"}
        if ceiling:
            roof["frac_of_copy_ceiling"] = round(achieved / ceiling["seg_copy_kernel"]["GB/s"], 4)
        return roof

    def fused_rs_variant(self, K: int, warmup: int):
        """The same pass with RS copy-in fused into the RS (the RS input is
        never materialised): reported beside the contract's step."""
        import torch
        runner = self.runner
        fsteps = runner.steps(fused_rs=True)
        for _ in range(warmup):
            runner.step(fused_rs=True)
        fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fs.record()
        for _ in range(K):
            runner.step(fused_rs=True)
        fe.record()
        torch.cuda.synchronize()
        f_ms = fs.elapsed_time(fe) / K
        f_us = per_step_us(runner, ["rs_copy_reduce"], K)["rs_copy_reduce"]
        b = self.nbytes["rs_copy_reduce"]
        pass_bytes = sum(self.nbytes[s] for s in fsteps)
        log(f"  fused RS variant: step {f_ms * 1e3:.1f} us; rs_copy_reduce {f_us:.1f} us, "
            f"{b / (f_us * 1e-6) / 1e9:.1f} GB/s")
        return {"steps_per_pass": fsteps, "ms_per_step": round(f_ms, 4), "bytes_per_step": pass_bytes,
                "GB/s": round(pass_bytes / (f_ms * 1e-3) / 1e9, 1),
                "rs_copy_reduce": {"bytes": b, "us": round(f_us, 2), "GB/s": round(b / (f_us * 1e-6) / 1e9, 1)},
                "note": "RS input never written; results identical to rs_copy_in + rs_reduce"}

    def release(self):
        import torch

        import hsdp_parameter_gradient_amd as hp
        self.runner = self.params = self.grads = None
        hp.fsdp_release_cache()
        torch.cuda.empty_cache()


def config_of(p: Pass):
    w = p.w
    return {"workload": w.name, "rank_size": w.rank_size, "shard_size": w.shard_size, "dp_size": w.dp_size,
            "param_dtype": str(w.param_dtype).replace("torch.", ""), "grad_dtype": "float32",
            "reduce_op": p.op, "params": len(w.param_shapes), "elements": sum(_numel(s) for s in w.param_shapes),
            "slice_numel": p.lay.I, "fused_numel": p.F, "bytes_per_step": p.bytes_per_step,
            "steps_per_pass": p.steps}


def bench_op(w) -> str:
    """The reduce op a workload is timed with: AVG (the pages' default for
    gradients not managed as DTensors) where the workload runs it."""
    return "avg" if "avg" in w.reduce_ops else w.reduce_ops[0]


HEADLINE = "llama7b_4layer_r8_s8"
OTHERS = ("hsdp_block_h1024_r8_s4_d2", "ragged_heavy_r8_s8", "pure_tp_2000grads_r8_s1_d8", "tiny_fsdp_r4_s4")
MALL_NOTE = ("working set ~1.3 GB per step against the 256 MB MALL: the RS input (403 MB) is written with "
             "cacheable stores and partly re-read from the MALL by the RS, so its fractions can exceed the "
             "HBM-only plain-copy ceiling (MALL-assisted)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="the headline workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the HSDP block's variants (16-bit gradients, shard dim 1, zero-copy AG, "
                         "per-parameter buckets, backward overlap) and the headline's HIP-graph pass")
    ap.add_argument("--pipeline-layers", type=int, default=8,
                    help="layers in the backward-overlap variant (0 = skip it)")
    ap.add_argument("--cold-warm-reps", type=int, default=20,
                    help="single launches per step for the cold/warm medians (0 = skip)")
    ap.add_argument("--ceiling-mib", type=int, default=4096,
                    help="size of the plain device-to-device copy ceiling (0 = skip)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--fold-shapes", action="store_true",
                    help="only time the dim-1 short-row and odd-pitch cases (fold kernels) and exit")
    ap.add_argument("--pipeline-trace", action="store_true",
                    help="only replay the captured backward overlap (serial, then two streams) and exit")
    ap.add_argument("--overlap-summary", metavar="CSV",
                    help="only summarise a rocprofv3 kernel trace of --pipeline-trace and exit (no GPU)")
    args = ap.parse_args()

    if args.overlap_summary:
        overlap_summary(args.overlap_summary, max(1, args.steps))
        return

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: the benchmark runs on one GPU only (the R ranks are "
              "simulated as HBM-resident slices of one GPU); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import hsdp_parameter_gradient_amd as hp
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibration_copy:
        calibration_copy(args.calibration_copy, max(1, args.steps))
        return
    if args.fold_shapes:
        fold_shapes(max(1, args.steps))
        return
    if args.pipeline_trace:
        pipeline_trace(max(1, args.steps))
        return
    torch.cuda.set_device(0)
    K = args.steps
    w = W.WORKLOADS[args.workload]
    op = bench_op(w)
    log(f"bench: workload {w.name} ({w.description}); R={w.rank_size} S={w.shard_size} D={w.dp_size} op={op}")
    head = Pass(w, op)
    res = head.measure(K, args.warmup, args.cold_warm_reps)
    ceiling = copy_ceiling(args.ceiling_mib, 10) if args.ceiling_mib > 0 else None
    roof = head.roofline(res, ceiling)
    variants = {}
    if isinstance(head.runner, hp.FlatBucket):
        variants["fused_rs_copy_reduce"] = head.fused_rs_variant(K, args.warmup)
        if not args.no_variants:
            variants["hip_graph"] = graph_variant(head.runner, K, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        k, n, el, sb, cpu_per = cpu_baseline(w, args.cpu_seconds, op, head.params or [], head.grads or [])
        what = "the whole bucket" if k == len(w.param_shapes) else \
            f"its first {k} of {len(w.param_shapes)} parameters ({sum(_numel(s) for s in w.param_shapes[:k])} " \
            f"of {sum(_numel(s) for s in w.param_shapes)} elements)"
        cpu = {"value": round(sb * n / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} whole steps of {w.name} restricted to {what}, same ranks and values, in "
                         f"{el:.1f} s; NumPy, single-threaded: 1 core of {os.cpu_count()} ({cpu_model()})",
               "ops": {s: {"ms": round(t * 1e3, 3), "GB/s": round(b / t / 1e9, 3)} for s, (t, b) in cpu_per.items()}}
        log(f"  cpu oracle: {cpu['value']} GB/s over {n} sample steps ({el:.1f} s)")
    out = {
        "metric": METRIC, "value": round(res["value"], 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16/f32", "data": "synthetic",
        "dtype_note": "copies move bf16 parameter bits and fp32 gradient bits; reductions compute in fp32",
        "config": config_of(head),
        "roofline": roof,
        "cpu_baseline": cpu,
        "ops": res["ops"],
        "ops_cold_warm": res["cold_warm"],
        "copy_ceiling": ceiling,
        "variants": variants,
    }
    head.release()
    del head

    # the other workloads: their own pass, dominant kernel and breakdown;
    # the HSDP block (the only one running all five steps) carries the
    # variants that need a replicate group
    others = {}
    if not args.no_other_workloads:
        for name in OTHERS:
            if name == w.name:
                continue
            wo = W.WORKLOADS[name]
            log(f"bench: other workload {wo.name} ({wo.description})")
            p = Pass(wo, bench_op(wo))
            r = p.measure(K, args.warmup, 0)
            ent = {"config": config_of(p), "value": round(r["value"], 1), "unit": "GB/s",
                   "ms_per_step": round(r["ms_per_step"], 4), "roofline": p.roofline(r, ceiling),
                   "ops": r["ops"]}
            ent["value_vs"] = frac_vs(r["value"], ceiling)
            if wo.name == "hsdp_block_h1024_r8_s4_d2":
                ent["note"] = MALL_NOTE
            if wo.name == "tiny_fsdp_r4_s4":
                ent["note"] = "under 4 KB per step: launch latency only"
            if isinstance(p.runner, hp.FlatBucket):
                v = {"fused_rs_copy_reduce": p.fused_rs_variant(K, args.warmup)}
                if not args.no_variants and wo.name == "hsdp_block_h1024_r8_s4_d2":
                    v["hip_graph"] = graph_variant(p.runner, K, args.warmup)
                    if args.pipeline_layers > 1 and p.runner.do_ar:
                        v["backward_pipeline"] = pipeline_variant(wo, p.op, args.pipeline_layers, K)
                    v["zero_copy_ag"] = zero_copy_ag_variant(wo, p.op, K)
                    v["per_parameter_buckets_one_ar"] = fused_group_variant(wo, p.op, K, args.warmup)
                    v["bf16_grads"] = bucket_variant(wo, p.op, K, args.warmup, grad_dtype=torch.bfloat16)
                    v["fp16_grads"] = bucket_variant(wo, p.op, K, args.warmup, grad_dtype=torch.float16)
                    dims = [1 if len(sh) > 1 and sh[1] % wo.shard_size == 0 else 0 for sh in wo.param_shapes]
                    if any(dims):
                        v["shard_dim_1"] = bucket_variant(wo, p.op, K, args.warmup, shard_dims=dims)
                ent["variants"] = v
            p.release()
            others[wo.name] = ent
    out["other_workloads"] = others or None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
