"""GPU parity on seeded random buckets, every entry point, bit for bit.

Forty buckets from tests/bucket_cases.py (the same cases whose planner
tables test_host_sanitizers.py runs through the CPU emulation of the
kernels): ragged and zero-length dims, parameters sharded on dims 1 and 2,
shard groups of 1-8 and replicate groups of 1-4 ranks, fp32 / bf16 / fp16
parameters and gradients chosen independently, and every buffer at its own
element offset.  Per bucket: AG copy-in and copy-out, RS copy-in, the RS
into a view of a 512-byte-aligned fused buffer that also holds other
segments, the fused AR over it, and the fused RS copy-reduce, each against
the oracle on guard-banded NaN-filled buffers.

FSDP_RANDOM_CASES=SEED:COUNT runs COUNT other buckets drawn with SEED
instead (a longer sweep; their tables are not the ones the CPU emulation
checks unless tests/bucket_cases.py's generator is run there with the same
seed).
"""

import os

import numpy as np
import pytest
import torch

import bucket_cases as BC
import oracle as O
import workloads as W
from gpu_util import Guarded, bits, first_mismatch, note, np_bits, require_gpu, to_oracle, to_oracle_values

hp = pytest.importorskip("hsdp_parameter_gradient_amd")

pytestmark = pytest.mark.gpu

SEED, COUNT = 20261202, 40  # the cases test_host_sanitizers.py emulates
if os.environ.get("FSDP_RANDOM_CASES"):
    SEED, COUNT = (int(x) for x in os.environ["FSDP_RANDOM_CASES"].split(":"))
CASES = BC.random_cases(SEED, COUNT)

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
NP_VALUES = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16}  # oracle forms of reduction operands
NP_BITS = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}  # oracle forms of copied data


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    hp.lib()
    yield
    hp.fsdp_release_cache()


def _check(buf, want, what):
    assert buf.guards_intact(), f"{what}: a write outside the buffer"
    m = first_mismatch(bits(buf.t), np_bits(want))
    assert m == "", f"{what}: {m}"


@pytest.mark.parametrize("case", CASES, ids=[f"case{c.index}" for c in CASES])
def test_random_bucket_every_step(case):
    c = case
    S, R, D = c.S, c.R, c.R // c.S
    shapes, dims = [tuple(s) for s in c.shapes], list(c.dims)
    pdt, gdt = TORCH[c.param_dtype], TORCH[c.grad_dtype]
    rng = np.random.default_rng(SEED + c.index)
    op = (O.SUM, O.AVG)[c.index % 2]
    note(f"[random] case {c.index}: S={S} R={R} {c.param_dtype}/{c.grad_dtype} {op} "
         f"misaligned={c.misaligned} shapes={shapes} dims={dims} extra={c.extra_segments}")

    def offset(es):  # an element offset: any, or a multiple of 16 bytes
        return int(rng.integers(0, 8)) * (1 if c.misaligned else 16 // es)

    w = W.Workload(f"random_case_{c.index}", 900 + c.index, R, S, tuple(shapes), pdt, ("normal", 1.0),
                   ("normal", 1.0), ("sum", "avg"), W.ALL_STEPS)
    lay = O.bucket_layout(shapes, S, shard_dims=dims)
    P, I = len(shapes), lay.I
    pes, ges = BC.ES[c.param_dtype], BC.ES[c.grad_dtype]

    # forward: AG copy-in, AG copy-out
    params = W.params(w)
    xs = [to_oracle(p) for p in params]
    ag_o = O.ag_copy_in(O.shard_params(xs, lay), lay, NP_BITS[c.param_dtype])
    dparams = [p.cuda() for p in params]
    keep, shards = [], []
    for s in range(S):
        for i in range(P):
            x = dparams[i].narrow(dims[i], lay.row_off[i][s], lay.row_len[i][s]).contiguous().reshape(-1)
            g = Guarded(x.numel(), pdt, offset(pes))
            g.t.copy_(x)
            keep.append(g)
            shards.append(g.t)
    ag = Guarded(S * I, pdt, offset(pes))
    hp.fsdp_ag_copy_in(shapes, S, shards, ag.t, shard_dims=dims)
    full = [Guarded(p.numel(), pdt, offset(pes)) for p in params]
    hp.fsdp_ag_copy_out(shapes, S, ag.t, [f.t for f in full], shard_dims=dims)
    torch.cuda.synchronize()
    _check(ag, ag_o, "ag_copy_in")
    for i in range(P):
        _check(full[i], xs[i], f"ag_copy_out param {i}")

    # backward: RS copy-in, RS into the fused buffers, fused AR
    grads = W.grads(w, dtype=gdt)
    gnp = [[to_oracle_values(g) for g in grads[r]] for r in range(R)]
    rs_o = [O.rs_copy_in(gnp[g], lay, NP_VALUES[c.grad_dtype]) for g in range(R)]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    rs_in = [Guarded(S * I, gdt, offset(ges)) for _ in range(R)]
    hp.fsdp_rs_copy_in(shapes, R, S, dgrads, [b.t for b in rs_in], shard_dims=dims)
    torch.cuda.synchronize()
    for g in range(R):
        _check(rs_in[g], rs_o[g], f"rs_copy_in rank {g}")

    segs = [I, *c.extra_segments]
    offs, F = hp.fsdp_fused_layout(segs, ges)
    assert (offs, F) == O.fused_layout(segs, ges)
    gen = torch.Generator().manual_seed(SEED * 7 + c.index)
    extra = [[torch.randn(n, generator=gen).to(gdt) for n in c.extra_segments] for _ in range(R)]
    fused, fused_np = [], []
    for g in range(R):
        f = Guarded(F, gdt, 0)
        assert f.t.data_ptr() % 512 == 0
        f.t.zero_()
        f.t[:I].view(torch.int16 if ges == 2 else torch.int32).fill_(0x7FA5 if ges == 2 else 0x7FA5A5A5)
        for o, t in zip(offs[1:], extra[g]):
            f.t[o:o + t.numel()] = t.cuda()
        fused.append(f)
    want_rs = O.rs_reduce(rs_o, I, R, S, op)
    hp.fsdp_rs_reduce(shapes, R, S, D, op, [b.t for b in rs_in], [f.t[:I] for f in fused], shard_dims=dims)
    torch.cuda.synchronize()
    for g in range(R):
        assert fused[g].guards_intact()
        m = first_mismatch(bits(fused[g].t[:I]), np_bits(want_rs[g]))
        assert m == "", f"rs_reduce {op} rank {g}: {m}"
        buf = np.zeros(F, NP_VALUES[c.grad_dtype])
        buf[:I] = want_rs[g]
        for o, t in zip(offs[1:], extra[g]):
            buf[o:o + t.numel()] = to_oracle_values(t)
        fused_np.append(buf)
    want_ar = O.fused_ar(fused_np, R, S, op)
    hp.fsdp_fused_ar(segs, R, S, D, op, [f.t for f in fused])
    torch.cuda.synchronize()
    for g in range(R):
        _check(fused[g], want_ar[g], f"fused_ar {op} rank {g}")

    # the fused RS copy-reduce gives the RS results without the RS input
    out = [Guarded(I, gdt, offset(ges)) for _ in range(R)]
    hp.fsdp_rs_copy_reduce(shapes, R, S, D, op, dgrads, [o.t for o in out], shard_dims=dims)
    torch.cuda.synchronize()
    for g in range(R):
        _check(out[g], want_rs[g], f"rs_copy_reduce {op} rank {g}")
