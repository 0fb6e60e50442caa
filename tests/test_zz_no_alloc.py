"""fsdp_rs_copy_reduce_noalloc (the entry point for callers that cannot
allocate device memory) against fsdp_rs_copy_reduce, bit for bit, through
the C ABI: several calls in a row on one GPU, each rewriting the scratch
array's tables, the second with a smaller input than the first; a dim-1
short-row parameter brings the fold-reduce launch (a second table in the
scratch array), an odd slice size the shifted reduction.  Outputs are
prefilled with a NaN pattern so that a skipped element cannot match."""

import pytest
import torch

import workloads as W
from gpu_util import bits, first_mismatch, note, require_gpu

hp = pytest.importorskip("hsdp_parameter_gradient_amd")

pytestmark = pytest.mark.gpu

# (name, shapes, shard dims, R, S)
CASES = [
    ("mixed_dim0_dim1", [(7, 8), (5, 3), (16,), (1000, 3), (64, 12), (3, 40, 8)], [0, 0, 0, 0, 1, 1], 8, 4),
    ("smaller", [(5, 3), (16,)], None, 8, 4),
    ("odd_offsets_s8", [(5, 3), (4097, 40), (1101, 4), (3,)], None, 8, 8),
]


def _poison(t):
    t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).fill_(0x7FA5 if t.dtype != torch.float32
                                                                            else 0x7FA5A5A5)


def _run(name, shapes, dims, R, S, op, dtype, seed):
    w = W.Workload(f"noalloc_{name}", seed, R, S, tuple(shapes), torch.float32, ("uniform", 1.0),
                   ("uniform", 1.0), ("sum", "avg"), W.ALL_STEPS)
    P = len(shapes)
    grads = W.grads(w, device="cuda", dtype=dtype)
    flat = [grads[g][i].reshape(-1) for g in range(R) for i in range(P)]
    I = hp.fsdp_bucket_layout(shapes, S, shard_dims=dims).I
    want = [torch.empty(I, dtype=dtype, device="cuda") for _ in range(R)]
    got = [torch.empty(I, dtype=dtype, device="cuda") for _ in range(R)]
    for t in want + got:
        _poison(t)
    hp.fsdp_rs_copy_reduce(shapes, R, S, R // S, op, flat, want, shard_dims=dims)
    before = hp.fsdp_cache_info()["plans"]
    hp.fsdp_rs_copy_reduce_noalloc(shapes, R, S, R // S, op, flat, got, shard_dims=dims)
    torch.cuda.synchronize()
    assert hp.fsdp_cache_info()["plans"] == before, "the call without allocation cached a plan"
    for g in range(R):
        m = first_mismatch(bits(got[g]), bits(want[g]))
        assert m == "", f"{name} {op} {dtype} rank {g}: {m}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_noalloc_matches_rs_copy_reduce_on_calls_in_a_row(op, dtype):
    require_gpu()
    hp.lib()
    # large, then smaller, then large again and the odd slice size: each
    # call rewrites the tables the previous one left in the scratch array
    for k, (name, shapes, dims, R, S) in enumerate(CASES + CASES[:1]):
        note(f"[no-alloc] call {k}: {name} R={R} S={S} {op} {dtype}")
        _run(name, shapes, dims, R, S, op, dtype, seed=900 + k)


def test_noalloc_refuses_oversized_tables_before_enqueueing():
    """Tables beyond the scratch array are refused (FSDP_EINVAL) and nothing
    runs: the outputs keep their contents."""
    require_gpu()
    hp.lib()
    note("[no-alloc] oversized tables are refused")
    P, R, S = 2000, 8, 8
    shapes = [(8,)] * P
    g = torch.ones(R * P * 8, device="cuda")
    flat = [g[k * 8:(k + 1) * 8] for k in range(R * P)]
    out = [torch.full((P,), 7.0, device="cuda") for _ in range(R)]
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_rs_copy_reduce_noalloc(shapes, R, S, 1, "sum", flat, out)
    assert e.value.code == 1 and "scratch" in e.value.message
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in out)


def test_noalloc_replayed_from_a_captured_graph():
    """The entry point inside a HIP graph capture: the captured table writes
    and kernels are replayed three times, each after new gradients were
    written and after an eager call of another shape rewrote the scratch
    array, and every replay equals the cached-plan rs_copy_reduce of the
    gradients it saw."""
    require_gpu()
    hp.lib()
    name, shapes, dims, R, S = CASES[0]
    other = CASES[2]
    P = len(shapes)
    note(f"[no-alloc] graph capture: {name} R={R} S={S}")
    w = W.Workload("noalloc_graph", 950, R, S, tuple(shapes), torch.float32, ("uniform", 1.0), ("uniform", 1.0),
                   ("sum", "avg"), W.ALL_STEPS)
    grads = W.grads(w, device="cuda")
    flat = [grads[g][i].reshape(-1) for g in range(R) for i in range(P)]
    I = hp.fsdp_bucket_layout(shapes, S, shard_dims=dims).I
    got = [torch.empty(I, device="cuda") for _ in range(R)]
    want = [torch.empty(I, device="cuda") for _ in range(R)]
    # eager first: the scratch array's address is looked up outside the capture
    hp.fsdp_rs_copy_reduce_noalloc(shapes, R, S, R // S, "avg", flat, got, shard_dims=dims)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hp.fsdp_rs_copy_reduce_noalloc(shapes, R, S, R // S, "avg", flat, got, shard_dims=dims)
    torch.cuda.synchronize()
    o_name, o_shapes, o_dims, o_R, o_S = other
    ow = W.Workload("noalloc_graph_other", 951, o_R, o_S, tuple(o_shapes), torch.float32, ("uniform", 1.0),
                    ("uniform", 1.0), ("sum", "avg"), W.ALL_STEPS)
    og = W.grads(ow, device="cuda")
    oflat = [og[g][i].reshape(-1) for g in range(o_R) for i in range(len(o_shapes))]
    oI = hp.fsdp_bucket_layout(o_shapes, o_S, shard_dims=o_dims).I
    oout = [torch.empty(oI, device="cuda") for _ in range(o_R)]
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        note(f"[no-alloc] graph replay {rep}")
        gen.manual_seed(960 + rep)
        for t in flat:
            t.copy_(2 * torch.rand(t.shape, device="cuda", generator=gen) - 1)
        for t in got + want:
            _poison(t)
        # another shape's tables overwrite the scratch array before the replay
        hp.fsdp_rs_copy_reduce_noalloc(o_shapes, o_R, o_S, o_R // o_S, "sum", oflat, oout, shard_dims=o_dims)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hp.fsdp_rs_copy_reduce(shapes, R, S, R // S, "avg", flat, want, shard_dims=dims)
        torch.cuda.synchronize()
        for g in range(R):
            m = first_mismatch(bits(got[g]), bits(want[g]))
            assert m == "", f"replay {rep} rank {g}: {m}"
    del graph
