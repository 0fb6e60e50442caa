"""GPU parity: every device entry point against the CPU oracle, bit for bit.

Sizes here are ones the oracle finishes in seconds while still spanning
many 16-32 KiB work chunks with ragged tails (and, for the HSDP block,
the full benchmark size).  Outputs live inside guard-banded, NaN-filled
buffers (tests/gpu_util.py), so writes outside a buffer and skipped
elements are both caught.  Copies are compared as bit patterns; the fp32
reductions too, because the kernels add in the same ascending rank order
as the oracle (max relative error 0, inside the 1e-6 bound).
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import Guarded, bits, first_mismatch, note, np_bits, require_gpu, to_oracle, to_oracle_values

hp = pytest.importorskip("hsdp_parameter_gradient_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    hp.lib()  # raises if the library is not built
    yield
    hp.fsdp_release_cache()


def _numel(shape):
    n = 1
    for d in shape:
        n *= d
    return n


def make_shards(dparams, lay, dtype, offsets=None):
    """Rank-major shards [s*P + i]: views of the full parameters, or (with
    offsets) copies in their own guard-banded buffers at those element
    offsets, to vary the source alignment."""
    S, P = lay.S, len(lay.shapes)
    out, keep = [], []
    for s in range(S):
        for i in range(P):
            a, n = lay.row_off[i][s], lay.row_len[i][s]
            v = dparams[i].reshape(lay.shapes[i])[a:a + n].reshape(-1)
            if offsets is not None:
                g = Guarded(v.numel(), dtype, offsets[(s * P + i) % len(offsets)])
                g.t.copy_(v)
                keep.append(g)
                v = g.t
            out.append(v)
    return out, keep


def run_copy_and_rs(name, shapes, R, S, params, grads, ops=(O.SUM, O.AVG),
                    shard_offsets=None, out_offset=0):
    note(f"[parity] {name}: R={R} S={S} P={len(shapes)} dtype={params[0].dtype if params else None} "
         f"shard_offsets={shard_offsets} out_offset={out_offset}")
    lay = O.bucket_layout(shapes, S)
    P, I, D = len(shapes), lay.I, R // S
    dtype = params[0].dtype if params else torch.float32
    xs = [to_oracle(p) for p in params]
    np_dtype = np.float32 if dtype == torch.float32 else np.uint16
    ag_o = O.ag_copy_in(O.shard_params(xs, lay), lay, np_dtype)
    full_o = O.ag_copy_out(O.all_gather(ag_o), lay)

    dparams = [p.cuda() for p in params]
    shards, _keep = make_shards(dparams, lay, dtype, shard_offsets)
    ag = Guarded(S * I, dtype, out_offset)
    hp.fsdp_ag_copy_in(shapes, S, shards, ag.t)
    full = [Guarded(_numel(sh), dtype, out_offset) for sh in shapes]
    hp.fsdp_ag_copy_out(shapes, S, ag.t, [f.t for f in full])
    torch.cuda.synchronize()
    assert ag.guards_intact(), "ag_copy_in wrote outside ag"
    assert first_mismatch(bits(ag.t), np_bits(ag_o)) == "", "ag_copy_in: " + first_mismatch(bits(ag.t), np_bits(ag_o))
    for i in range(P):
        assert full[i].guards_intact(), f"ag_copy_out wrote outside full[{i}]"
        m = first_mismatch(bits(full[i].t), np_bits(full_o[i].reshape(-1)))
        assert m == "", f"ag_copy_out param {i}: {m}"
        assert np.array_equal(bits(full[i].t), np_bits(xs[i].reshape(-1)))  # all_gather(shard(x)) == x

    if grads is None:
        return
    gnp = [[to_oracle(g) for g in grads[r]] for r in range(R)]
    rs_o = [O.rs_copy_in(gnp[g], lay, np.float32) for g in range(R)]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    rs_in = [Guarded(S * I, torch.float32, out_offset) for _ in range(R)]
    hp.fsdp_rs_copy_in(shapes, R, S, dgrads, [b.t for b in rs_in])
    torch.cuda.synchronize()
    for g in range(R):
        assert rs_in[g].guards_intact(), f"rs_copy_in wrote outside rs_in[{g}]"
        m = first_mismatch(bits(rs_in[g].t), np_bits(rs_o[g]))
        assert m == "", f"rs_copy_in rank {g}: {m}"
    for op in ops:
        out_o = O.rs_reduce(rs_o, I, R, S, op)
        out = [Guarded(I, torch.float32, out_offset + 1 + g % 3) for g in range(R)]
        hp.fsdp_rs_reduce(shapes, R, S, D, op, [b.t for b in rs_in], [o.t for o in out])
        torch.cuda.synchronize()
        for g in range(R):
            assert out[g].guards_intact(), f"rs_reduce wrote outside rs_out[{g}]"
            m = first_mismatch(bits(out[g].t), np_bits(out_o[g]))
            assert m == "", f"rs_reduce {op} rank {g}: {m}"


def test_tiny_fsdp_workload():
    w = W.TINY_FSDP
    run_copy_and_rs(w.name, w.param_shapes, w.rank_size, w.shard_size, W.params(w), W.grads(w))


@pytest.mark.parametrize("out_offset", [1, 2, 3])
def test_tiny_fsdp_misaligned(out_offset):
    w = W.TINY_FSDP
    run_copy_and_rs(w.name + "_misaligned", w.param_shapes, w.rank_size, w.shard_size, W.params(w), W.grads(w),
                    shard_offsets=[0, 1, 2, 3, 5, 7], out_offset=out_offset)


def test_ragged_heavy_scaled():
    """The ragged-heavy set with its second dim cut from 4096 to 8: same
    dim-0 sizes, an odd slice size I, zero-length shards, many chunks."""
    w = W.scaled(W.RAGGED_HEAVY, [(4097, 8), (11009, 8), (32001, 8), (5, 64), (3,)])
    run_copy_and_rs(w.name, w.param_shapes, w.rank_size, w.shard_size, W.params(w), W.grads(w))


def test_bf16_ragged_all_alignments():
    """bf16 with 1-D parameters whose shards start at odd elements: every
    2-byte source/destination misalignment, HSDP 16 = 2 x 8."""
    shapes = [(100003,), (7, 3), (13,), (0, 5), (1,), (257, 33), (40001, 3)]
    w = W.Workload("bf16_ragged", 11, 16, 8, tuple(shapes), torch.bfloat16, ("normal", 0.02),
                   ("normal", 1e-3), ("sum", "avg"), W.ALL_STEPS)
    run_copy_and_rs(w.name, shapes, 16, 8, W.params(w), W.grads(w),
                    shard_offsets=[0, 1, 2, 3, 4, 5, 6, 7, 9, 13], out_offset=5)


def test_fp16_copies_and_nonpow2_groups():
    shapes = [(1001, 7), (17,), (3, 3, 3), (0,)]
    w = W.Workload("fp16_r6_s3", 12, 6, 3, tuple(shapes), torch.float16, ("uniform", 1.0),
                   ("uniform", 1.0), ("sum", "avg"), W.ALL_STEPS)
    run_copy_and_rs(w.name, shapes, 6, 3, W.params(w), W.grads(w), shard_offsets=[0, 3, 1])


def test_fp32_nonpow2_shard_group():
    shapes = [(1001, 7), (17,), (3, 3, 3), (50000,)]
    w = W.Workload("fp32_r6_s3", 13, 6, 3, tuple(shapes), torch.float32, ("uniform", 1.0),
                   ("uniform", 1.0), ("sum", "avg"), W.ALL_STEPS)
    run_copy_and_rs(w.name, shapes, 6, 3, W.params(w), W.grads(w))


def test_many_parameters_deep_chunk_search():
    """700 small ragged parameters over 8 ranks: 5600 AG segments and 44800
    RS copy-in segments, most of them a part of one chunk, so the copy
    kernel's per-chunk item map holds thousands of items; the fused RS
    copy-reduce's 5600 jobs take the reduce kernel's 64-ary chunk search
    three levels deep."""
    rng = np.random.default_rng(77)
    shapes = [tuple([int(rng.integers(0, 40))] + ([int(rng.choice([1, 3, 8]))] if rng.random() < 0.5 else []))
              for _ in range(700)]
    w = W.Workload("many_params", 21, 8, 8, tuple(shapes), torch.float32, ("uniform", 1.0), ("normal", 1.0),
                   ("sum", "avg"), W.ALL_STEPS)
    grads = W.grads(w)
    run_copy_and_rs(w.name, shapes, 8, 8, W.params(w), grads, shard_offsets=[0, 1, 2, 3], out_offset=1)
    run_rs_copy_reduce(w.name, shapes, 8, 8, grads, out_offset=1)


def test_random_buckets():
    rng = np.random.default_rng(2024)
    for case in range(16):
        S = int(rng.choice([1, 2, 3, 4, 5, 8]))
        D = int(rng.choice([1, 2, 3]))
        P = int(rng.integers(1, 6))
        shapes = []
        for _ in range(P):
            n0 = int(rng.integers(0, 3 * S + 40))
            rest = [int(rng.choice([1, 2, 3, 7, 64, 129]))] if rng.random() < 0.6 else []
            shapes.append(tuple([n0] + rest))
        dtype = [torch.float32, torch.bfloat16, torch.float16][case % 3]
        w = W.Workload(f"random_{case}", 100 + case, S * D, S, tuple(shapes), dtype, ("uniform", 1.0),
                       ("normal", 1.0), ("sum", "avg"), W.ALL_STEPS)
        run_copy_and_rs(w.name, shapes, S * D, S, W.params(w), W.grads(w),
                        shard_offsets=[int(v) for v in rng.integers(0, 8, size=5)],
                        out_offset=int(rng.integers(0, 8)))


def test_hsdp_block_full_size_copies_and_rs():
    w = W.HSDP_BLOCK
    run_copy_and_rs(w.name, w.param_shapes, w.rank_size, w.shard_size, W.params(w), W.grads(w),
                    ops=(O.AVG, O.SUM))


def test_padding_rewritten_on_reuse_and_side_stream():
    """Padding is written as zero on every call (stale values in a reused
    buffer are overwritten), also when the call runs on a side stream."""
    shapes = [(7, 8), (5, 3), (16,), (3,)]
    S = 4
    lay = O.bucket_layout(shapes, S)
    xs = [torch.randn(sh) for sh in shapes]
    dparams = [x.cuda() for x in xs]
    shards, _ = make_shards(dparams, lay, torch.float32)
    ag = torch.full((S * lay.I,), float("nan"), device="cuda")
    st = torch.cuda.Stream()
    for rep in range(3):
        ag.fill_(float(rep + 1))
        with torch.cuda.stream(st):
            hp.fsdp_ag_copy_in(shapes, S, shards, ag)
        st.synchronize()
        want = O.ag_copy_in(O.shard_params([x.numpy() for x in xs], lay), lay, np.float32)
        assert np.array_equal(bits(ag), np_bits(want))


_POISON = {torch.float32: -1, torch.bfloat16: -1, torch.float16: -1}  # all-ones bits: a NaN


@pytest.mark.parametrize("case", [
    # ragged dim-0 shards, zero-length ranks, a zero-size parameter
    ("ragged_dim0", [(7, 8), (5, 3), (0, 4), (1,), (3,), (1000, 33), (4099,)], None, 8, torch.float32),
    ("ragged_dim0_bf16", [(7, 8), (5, 3), (0, 4), (1,), (3,), (1000, 33), (4099,)], None, 6, torch.bfloat16),
    # dim-1 shards (which have no padding: the dim divides S) between padded
    # dim-0 ones: short rows (one workgroup per whole full row), long rows,
    # pitches that are not multiples of 16 bytes
    ("dim1_fp32", [(64, 8), (33, 12, 3), (5,), (9, 20), (1000, 6), (3, 2048, 1), (300, 1024)],
     [1, 1, 0, 1, 1, 1, 1], 2,
     torch.float32),
    ("dim1_fp16", [(64, 8), (33, 12, 3), (9, 20), (5,), (1000, 12), (3, 2048, 1), (5, 8, 3)],
     [1, 1, 1, 0, 1, 1, 1], 4,
     torch.float16),
])
def test_ag_copy_out_never_reads_padding(case):
    """AG copy-out reads only the actual rows of every rank slice: with all
    padding of the gathered buffer overwritten by a NaN pattern, the full
    parameters still come out bit for bit (padding never enters the module,
    the ragged-sharding paper's section on padded shards)."""
    name, shapes, dims, S, dtype = case
    note(f"[parity] padding poison {name}: S={S} dtype={dtype}")
    dims = dims if dims is not None else [0] * len(shapes)
    lay = O.bucket_layout(shapes, S, shard_dims=dims)
    P, I = len(shapes), lay.I
    gen = torch.Generator().manual_seed(321)
    xs = [torch.randn(sh, generator=gen).to(dtype) for sh in shapes]
    np_dt = np.float32 if dtype == torch.float32 else np.uint16
    # where the data lands: AG copy-in of all-ones shards is nonzero exactly there
    ones = [np.ones(sh, np_dt) for sh in shapes]
    data_mask = O.ag_copy_in(O.shard_params(ones, lay), lay, np_dt) != 0
    n_pad = int((~data_mask).sum())
    assert n_pad > 0
    dparams = [x.cuda() for x in xs]
    shards = [dparams[i].narrow(dims[i], lay.row_off[i][s], lay.row_len[i][s]).contiguous().reshape(-1)
              for s in range(S) for i in range(P)]
    ag = Guarded(S * I, dtype, 3)
    hp.fsdp_ag_copy_in(shapes, S, shards, ag.t, shard_dims=dims)
    it = _INT_VIEW[dtype]
    pad_idx = torch.from_numpy(np.flatnonzero(~data_mask)).cuda()
    ag.t.view(it).index_fill_(0, pad_idx, _POISON[dtype])
    full = [Guarded(_numel(sh), dtype, 1) for sh in shapes]
    hp.fsdp_ag_copy_out(shapes, S, ag.t, [f.t for f in full], shard_dims=dims)
    torch.cuda.synchronize()
    assert int((bits(ag.t)[~data_mask.reshape(-1)] == -1).sum()) == n_pad
    for i in range(P):
        assert full[i].guards_intact(), f"ag_copy_out wrote outside full[{i}]"
        m = first_mismatch(bits(full[i].t), np_bits(to_oracle(xs[i]).reshape(-1)))
        assert m == "", f"{name} param {i} {shapes[i]}: {m}"


_INT_VIEW = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}


def test_empty_buckets():
    note("[parity] empty buckets")
    S, R = 4, 8
    for shapes in ([], [(0,), (0, 7)]):
        lay = O.bucket_layout(shapes, S)
        assert lay.I == 0
        ag = torch.empty(0, device="cuda")
        shards = [torch.empty(0, device="cuda") for _ in range(S * len(shapes))]
        hp.fsdp_ag_copy_in(shapes, S, shards, ag)
        hp.fsdp_ag_copy_out(shapes, S, ag, [torch.empty(sh, device="cuda").reshape(-1) for sh in shapes])
        grads = [torch.empty(0, device="cuda") for _ in range(R * len(shapes))]
        rs_in = [torch.empty(0, device="cuda") for _ in range(R)]
        hp.fsdp_rs_copy_in(shapes, R, S, grads, rs_in)
        hp.fsdp_rs_reduce(shapes, R, S, 2, O.AVG, rs_in, [torch.empty(0, device="cuda") for _ in range(R)])
        hp.fsdp_fused_ar([], R, S, 2, O.AVG, [torch.empty(0, device="cuda") for _ in range(R)])
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# fused AR and the end-to-end gradient path
# ---------------------------------------------------------------------------

def fill_fused(seg_grads, offs, F):
    """Fused buffers (gaps zero) holding rank g's segments at offs (on the GPU)."""
    out = []
    for segs in seg_grads:
        buf = torch.zeros(F, dtype=torch.float32, device="cuda")
        for o, t in zip(offs, segs):
            buf[o:o + t.numel()] = t.reshape(-1)
        out.append(buf)
    return out


@pytest.mark.parametrize("op", [O.AVG, O.SUM])
def test_pure_tp_fused_ar_full_size(op):
    """2000 gradients, log-uniform sizes, one 512-byte-aligned segment each,
    AR over all 8 ranks (shard_size 1, dp_size 8)."""
    w = W.PURE_TP
    R, S = w.rank_size, w.shard_size
    sizes = [s[0] for s in w.param_shapes]
    note(f"[parity] {w.name} fused_ar {op}: {len(sizes)} segments")
    g_cpu = W.grads(w)
    offs_o, F_o = O.fused_layout(sizes)
    fused_o = []
    for g in range(R):
        buf = np.zeros(F_o, np.float32)
        for o, t in zip(offs_o, g_cpu[g]):
            buf[o:o + t.numel()] = t.numpy()
        fused_o.append(buf)
    want = O.fused_ar(fused_o, R, S, op)
    offs, F = hp.fsdp_fused_layout(sizes, 4)
    assert (offs, F) == (offs_o, F_o)
    fused = fill_fused([[t.cuda() for t in g_cpu[g]] for g in range(R)], offs, F)
    hp.fsdp_fused_ar(sizes, R, S, R // S, op, fused)
    torch.cuda.synchronize()
    for g in range(R):
        m = first_mismatch(bits(fused[g]), np_bits(want[g]))
        assert m == "", f"fused_ar rank {g}: {m}"


def run_hsdp_end_to_end(name, buckets, R, S, op, dtype=torch.float32, seed=7):
    """Per bucket RS copy-in and RS into views of the fused buffers, then one
    fused AR; compared with the oracle's fused path (final sharded grads
    and the whole fused buffers, gaps included)."""
    note(f"[parity] e2e {name}: R={R} S={S} op={op} buckets={len(buckets)}")
    shapes = [sh for b in buckets for sh in b]
    w = W.Workload(name, seed, R, S, tuple(shapes), dtype, ("normal", 1.0), ("normal", 1e-3),
                   (op,), W.ALL_STEPS)
    g_cpu = W.grads(w)
    gnp = [[t.numpy() for t in g_cpu[g]] for g in range(R)]
    res_o, fused_o, offs_o, lays = O.reduce_grads_fused(gnp, buckets, R, S, op)
    D = R // S
    lays_h = [hp.fsdp_bucket_layout(b, S) for b in buckets]
    offs, F = hp.fsdp_fused_layout([l.I for l in lays_h], 4)
    fused = [torch.zeros(F, dtype=torch.float32, device="cuda") for _ in range(R)]
    j0 = 0
    for b, lay, off in zip(buckets, lays_h, offs):
        P = len(b)
        grads = [g_cpu[g][j0 + i].cuda().reshape(-1) for g in range(R) for i in range(P)]
        rs_in = [torch.empty(S * lay.I, dtype=torch.float32, device="cuda") for _ in range(R)]
        hp.fsdp_rs_copy_in(b, R, S, grads, rs_in)
        hp.fsdp_rs_reduce(b, R, S, D, op, rs_in, [f[off:off + lay.I] for f in fused])
        j0 += P
    rs, ar = hp.fsdp_group_ranks(R, S)
    if ar:
        hp.fsdp_fused_ar([l.I for l in lays_h], R, S, D, op, fused)
    torch.cuda.synchronize()
    for g in range(R):
        m = first_mismatch(bits(fused[g]), np_bits(fused_o[g]))
        assert m == "", f"e2e fused buffer rank {g}: {m}"
    # write-back by sharded_size: the optimizer's views match the oracle's
    j0 = 0
    for k, (b, lay) in enumerate(zip(buckets, lays_h)):
        for g in range(R):
            s = g % S
            for i, sh in enumerate(b):
                n = lay.row_len[i][s] * _numel(sh[1:])
                v = fused[g][offs[k] + lay.in_off[i]: offs[k] + lay.in_off[i] + n]
                assert np.array_equal(bits(v), np_bits(res_o[g][j0 + i].reshape(-1)))
        j0 += len(b)


@pytest.mark.parametrize("R,S", [(8, 4), (8, 2), (6, 2), (16, 8), (12, 6), (18, 3)])
@pytest.mark.parametrize("op", [O.AVG, O.SUM])
def test_hsdp_end_to_end_multi_bucket(R, S, op):
    shapes = [(7, 8), (5, 3), (16,), (3,), (1000, 3), (129,), (4097, 2)]
    run_hsdp_end_to_end(f"multi_bucket_{R}_{S}", [shapes[:3], shapes[3:5], shapes[5:]], R, S, op)
    run_hsdp_end_to_end(f"per_param_{R}_{S}", [[s] for s in shapes], R, S, op)


def test_hsdp_block_end_to_end_flat_bucket():
    """The HSDP block through FlatBucket (the benchmark's object): all five
    steps, RS outputs written as fused-buffer views, AR(2) with AVG."""
    w = W.HSDP_BLOCK
    R, S, D = w.rank_size, w.shard_size, w.dp_size
    note(f"[parity] {w.name} FlatBucket step")
    params = W.params(w)
    g_cpu = W.grads(w)
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG)
    dparams = [p.cuda() for p in params]
    dgrads = [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(len(w.param_shapes))]
    fb.bind(fb.shard_views(dparams), dgrads)
    assert fb.steps() == list(W.ALL_STEPS)
    fb.step()
    torch.cuda.synchronize()
    for i, p in enumerate(params):
        assert np.array_equal(bits(fb.full[i]), bits(p.reshape(-1)))
    gnp = [[t.numpy() for t in g_cpu[g]] for g in range(R)]
    res_o, fused_o, _, _ = O.reduce_grads_fused(gnp, [list(w.param_shapes)], R, S, O.AVG)
    for g in range(R):
        m = first_mismatch(bits(fb.fused[g]), np_bits(fused_o[g]))
        assert m == "", f"fused rank {g}: {m}"


@pytest.mark.parametrize("grad_dtype,on_dim_1", [(torch.bfloat16, False), (torch.float32, True),
                                                (torch.bfloat16, True), (torch.float16, False),
                                                (torch.float16, True)])
def test_flat_bucket_bf16_grads_and_shard_dim_1(grad_dtype, on_dim_1):
    """FlatBucket with bfloat16 gradients and/or its 2-D parameters sharded
    on dim 1 (the benchmark's variants), on a scaled-down HSDP block: the
    gathered parameters and the fused buffers (unfused and fused RS) against
    the oracle."""
    w = W.scaled(W.HSDP_BLOCK, [(97, 64), (32, 64), (130, 32), (33, 128), (64,), (3,)])
    R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
    dims = [1 if on_dim_1 and len(sh) > 1 and sh[1] % S == 0 else 0 for sh in w.param_shapes]
    note(f"[parity] FlatBucket grad_dtype={grad_dtype} shard_dims={dims} shapes={w.param_shapes}")
    params, g_cpu = W.params(w), W.grads(w, dtype=grad_dtype)
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG, grad_dtype=grad_dtype,
                       shard_dims=dims if on_dim_1 else None)
    fb.bind(fb.shard_views([p.cuda() for p in params]),
            [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)])
    lay = O.bucket_layout(w.param_shapes, S, shard_dims=dims)
    gnp = [[to_oracle_values(t) for t in g_cpu[g]] for g in range(R)]
    rs_o = O.rs_copy_reduce(gnp, lay, R, O.AVG)
    _, F = O.fused_layout([lay.I], grad_dtype.itemsize)
    fused_o = O.fused_ar([np.concatenate([rs_o[g], np.zeros(F - lay.I, rs_o[g].dtype)]) for g in range(R)],
                         R, S, O.AVG)
    for fused_rs in (False, True):
        for v in fb.rs_out:
            v.fill_(float("nan"))
        fb.step(fused_rs=fused_rs)
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            assert np.array_equal(bits(fb.full[i]), bits(p.reshape(-1))), f"full param {i}"
        for g in range(R):
            m = first_mismatch(bits(fb.fused[g]), np_bits(fused_o[g]))
            assert m == "", f"fused_rs={fused_rs} rank {g}: {m}"


# ---------------------------------------------------------------------------
# RS copy-in fused into the RS, and bfloat16 gradients
# ---------------------------------------------------------------------------

def run_rs_copy_reduce(name, shapes, R, S, grads, ops=(O.SUM, O.AVG), out_offset=0):
    """fsdp_rs_copy_reduce against the oracle's RS of the RS inputs."""
    dtype = grads[0][0].dtype if shapes else torch.float32
    note(f"[parity] rs_copy_reduce {name}: R={R} S={S} P={len(shapes)} dtype={dtype} out_offset={out_offset}")
    lay = O.bucket_layout(shapes, S)
    P = len(shapes)
    gnp = [[to_oracle_values(g) for g in grads[r]] for r in range(R)]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    for op in ops:
        want = O.rs_copy_reduce(gnp, lay, R, op)
        out = [Guarded(lay.I, dtype, out_offset + g % 3) for g in range(R)]
        hp.fsdp_rs_copy_reduce(shapes, R, S, R // S, op, dgrads, [o.t for o in out])
        torch.cuda.synchronize()
        for g in range(R):
            assert out[g].guards_intact(), f"rs_copy_reduce wrote outside rs_out[{g}]"
            m = first_mismatch(bits(out[g].t), np_bits(want[g]))
            assert m == "", f"rs_copy_reduce {op} rank {g}: {m}"


def test_rs_copy_reduce_tiny_and_misaligned():
    w = W.TINY_FSDP
    for off in (0, 1, 3):
        run_rs_copy_reduce(w.name, w.param_shapes, w.rank_size, w.shard_size, W.grads(w), out_offset=off)


def test_rs_copy_reduce_ragged_heavy_scaled():
    w = W.scaled(W.RAGGED_HEAVY, [(4097, 8), (11009, 8), (32001, 8), (5, 64), (3,)])
    run_rs_copy_reduce(w.name, w.param_shapes, w.rank_size, w.shard_size, W.grads(w), out_offset=1)


def test_rs_copy_reduce_hsdp_block_full_size():
    w = W.HSDP_BLOCK
    run_rs_copy_reduce(w.name, w.param_shapes, w.rank_size, w.shard_size, W.grads(w), ops=(O.AVG,))


def test_rs_copy_reduce_random_buckets():
    rng = np.random.default_rng(404)
    for case in range(12):
        S = int(rng.choice([1, 2, 3, 4, 8]))
        D = int(rng.choice([1, 2, 3]))
        shapes = []
        for _ in range(int(rng.integers(1, 6))):
            n0 = int(rng.integers(0, 3 * S + 40))
            rest = [int(rng.choice([1, 2, 3, 7, 64, 129]))] if rng.random() < 0.6 else []
            shapes.append(tuple([n0] + rest))
        dtype = [torch.float32, torch.bfloat16][case % 2]
        w = W.Workload(f"rcr_random_{case}", 300 + case, S * D, S, tuple(shapes), dtype, ("normal", 1.0),
                       ("normal", 1.0), ("sum", "avg"), W.ALL_STEPS)
        run_rs_copy_reduce(w.name, shapes, S * D, S, W.grads(w, dtype=dtype), out_offset=int(rng.integers(0, 5)))


NP16 = {torch.bfloat16: np.uint16, torch.float16: np.float16}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("R,S", [(8, 4), (16, 8), (6, 3), (4, 1), (12, 6)])
def test_16bit_rs_copy_in_and_reduce(R, S, dtype):
    """bf16 / fp16 gradients: RS copy-in (a bit copy), RS (fp32 sum, one
    rounding) and the fused form agree with the oracle bit for bit."""
    shapes = [(1001, 7), (17,), (3, 3, 3), (0,), (40001,), (5, 64)]
    w = W.Workload(f"{str(dtype)[6:]}_rs_{R}_{S}", 21, R, S, tuple(shapes), dtype, ("normal", 1.0),
                   ("normal", 1e-3), ("sum", "avg"), W.ALL_STEPS)
    grads = W.grads(w, dtype=dtype)
    note(f"[parity] {dtype} RS R={R} S={S}")
    lay = O.bucket_layout(shapes, S)
    P = len(shapes)
    gnp = [[to_oracle_values(g) for g in grads[r]] for r in range(R)]
    rs_o = [O.rs_copy_in(gnp[g], lay, NP16[dtype]) for g in range(R)]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    rs_in = [Guarded(S * lay.I, dtype, 1) for _ in range(R)]
    hp.fsdp_rs_copy_in(shapes, R, S, dgrads, [b.t for b in rs_in])
    for op in (O.SUM, O.AVG):
        out = [Guarded(lay.I, dtype, g % 4) for g in range(R)]
        hp.fsdp_rs_reduce(shapes, R, S, R // S, op, [b.t for b in rs_in], [o.t for o in out])
        torch.cuda.synchronize()
        want = O.rs_reduce(rs_o, lay.I, R, S, op)
        for g in range(R):
            assert rs_in[g].guards_intact() and out[g].guards_intact()
            assert first_mismatch(bits(rs_in[g].t), np_bits(rs_o[g])) == ""
            m = first_mismatch(bits(out[g].t), np_bits(want[g]))
            assert m == "", f"{dtype} rs_reduce {op} rank {g}: {m}"
    run_rs_copy_reduce(w.name, shapes, R, S, grads)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("op", [O.AVG, O.SUM])
def test_16bit_fused_ar_pure_tp(op, dtype):
    """bf16 / fp16 fused AR over 300 segments (512-byte alignment = 256
    elements)."""
    sizes = [s[0] for s in W.PURE_TP.param_shapes[:300]]
    w = W.scaled(W.PURE_TP, [(n,) for n in sizes], name=f"pure_tp_{str(dtype)[6:]}")
    R, S = w.rank_size, w.shard_size
    note(f"[parity] {dtype} fused_ar {op}: {len(sizes)} segments")
    g_cpu = W.grads(w, dtype=dtype)
    offs, F = O.fused_layout(sizes, elem_bytes=2)
    fused_o = []
    for g in range(R):
        buf = np.zeros(F, NP16[dtype])
        for o, t in zip(offs, g_cpu[g]):
            buf[o:o + t.numel()] = to_oracle_values(t)
        fused_o.append(buf)
    want = O.fused_ar(fused_o, R, S, op)
    assert hp.fsdp_fused_layout(sizes, 2) == (offs, F)
    fused = [torch.from_numpy(f.view(np.int16).copy()).view(dtype).cuda() for f in fused_o]
    hp.fsdp_fused_ar(sizes, R, S, R // S, op, fused)
    torch.cuda.synchronize()
    for g in range(R):
        m = first_mismatch(bits(fused[g]), np_bits(want[g]))
        assert m == "", f"{dtype} fused_ar rank {g}: {m}"


def test_zero_copy_ag_views_one_parameter_buckets():
    """Per-parameter buckets: after AG copy-in the gathered buffer's prefix
    view is the full parameter (no copy-out)."""
    note("[parity] zero-copy AG views")
    for shape, S in [((7, 8), 4), ((5, 3), 4), ((3,), 8), ((4097, 16), 8), ((100003,), 8), ((0, 4), 4),
                     ((1024, 1024), 4)]:
        x = torch.randn(shape, device="cuda").to(torch.bfloat16)
        fb = hp.FlatBucket([shape], 8, S, torch.bfloat16)
        lay = O.bucket_layout([shape], S)
        shards, _ = make_shards([x], lay, torch.bfloat16)
        hp.fsdp_ag_copy_in([shape], S, shards, fb.ag)
        torch.cuda.synchronize()
        (v,) = fb.full_views()
        assert v.data_ptr() == fb.ag.data_ptr() and v.shape == x.shape
        assert torch.equal(v.view(torch.int16), x.view(torch.int16))
    with pytest.raises(ValueError):
        hp.FlatBucket([(4, 4), (3,)], 8, 4, torch.bfloat16).full_views()


@pytest.mark.parametrize("fused_rs", [True, False])
def test_backward_pipeline_two_streams_matches_serial_and_oracle(fused_rs):
    """The 4-step RS/AR overlap over 5 layers on two streams gives the same
    fused buffers as the serial order, eagerly and replayed from captured HIP
    graphs, and all match the oracle."""
    R, S = 8, 4
    layer_shapes = [[(7, 8), (5, 3), (16,)], [(1000, 3), (129,)], [(4097, 2)], [(3,), (33, 7)],
                    [(2048, 64), (64,)]]
    note(f"[parity] backward pipeline fused_rs={fused_rs}")
    layers, want = [], []
    for l, shapes in enumerate(layer_shapes):
        w = W.Workload(f"pipe_{l}", 500 + l, R, S, tuple(shapes), torch.float32, ("normal", 1.0),
                       ("normal", 1.0), ("avg",), W.ALL_STEPS)
        g_cpu = W.grads(w)
        fb = hp.FlatBucket(shapes, R, S, torch.float32, op=O.AVG)
        params = [torch.zeros(sh, device="cuda") for sh in shapes]
        fb.bind(fb.shard_views(params), [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(len(shapes))])
        layers.append(fb)
        _, fused_o, _, _ = O.reduce_grads_fused([[t.numpy() for t in g_cpu[g]] for g in range(R)], [shapes], R, S,
                                                O.AVG)
        want.append(fused_o)
    pipe = hp.BackwardPipeline(layers, fused_rs=fused_rs)
    graphs = {}
    for rep in range(7):
        for fb in layers:  # the RS must rewrite its views; the gaps stay zero
            for v in fb.rs_out:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        if rep < 3:
            (pipe.run_pipelined if rep % 2 == 0 else pipe.run_serial)()
        else:  # replays of the captured backward, eager work between them
            pipelined = rep % 2 == 1
            if pipelined not in graphs:
                graphs[pipelined] = pipe.graph(pipelined=pipelined)
                for fb in layers:
                    for v in fb.rs_out:
                        v.fill_(float("nan"))
                torch.cuda.synchronize()
            graphs[pipelined].replay()
        torch.cuda.synchronize()
        for l, fb in enumerate(layers):
            for g in range(R):
                m = first_mismatch(bits(fb.fused[g]), np_bits(want[l][g]))
                assert m == "", f"rep {rep} layer {l} rank {g}: {m}"
    graphs.clear()


@pytest.mark.parametrize("S,R,dtype", [(4, 8, torch.float32), (2, 4, torch.bfloat16), (1, 2, torch.float32),
                                       (8, 8, torch.float32)])
def test_nonzero_shard_dims_all_steps(S, R, dtype):
    """A bucket mixing dim-0 (ragged) parameters with parameters sharded on
    dims 1 and 2 (divisible): every step against the oracle, buffers at
    every element offset (chunks moved one row at a time)."""
    shapes = [(6, 8), (4, 16, 3), (5, 3, 8), (7, 3), (16,), (64, 1024), (3, 4, 8)]
    dims = [1, 1, 2, 0, 0, 1, 2]
    run_nonzero_dims(shapes, dims, S, R, dtype, aligned=False)


@pytest.mark.parametrize("S,R,dtype", [(4, 8, torch.float32), (4, 8, torch.bfloat16), (2, 4, torch.float32),
                                       (8, 8, torch.bfloat16)])
def test_strided_blocks_all_steps(S, R, dtype):
    """Chunks of dim-1 parameters as strided blocks (16-byte-aligned buffers,
    rows of whole vectors): several rows per chunk, a short last chunk, a
    row as large as a chunk, and rows that are not whole vectors beside
    them; every step against the oracle."""
    shapes = [(64, 1024), (300, 256), (2, 8192), (3, 24, 2), (7, 3), (16,), (5, 32, 8), (0, 8), (2, 0, 8)]
    dims = [1, 1, 1, 1, 0, 0, 1, 1, 2]
    run_nonzero_dims(shapes, dims, S, R, dtype, aligned=True)


@pytest.mark.parametrize("S,R,dtype,aligned", [(2, 4, torch.float16, True), (2, 4, torch.float32, True),
                                               (2, 2, torch.bfloat16, False), (2, 6, torch.float16, False)])
def test_chunk_filling_rows_all_steps(S, R, dtype, aligned):
    """Dim-1 parameters over 2 ranks with many rows per item: 4,120-byte
    rank rows of 8-byte units (strided copy blocks whose chunks take the
    fewest rows that fill them, one row crossing the chunk size; fold
    reductions of 8-byte units, two rows per chunk) and rows of 8 to 128
    bytes whose fold reductions take 16 KiB chunks of the unit loop, several
    chunks each and a short last one; every step against the oracle."""
    shapes = [(50, 1030, 4), (3001, 4), (3000, 8), (1000, 64), (77, 1030, 2), (5,)]
    dims = [1, 1, 1, 1, 1, 0]
    run_nonzero_dims(shapes, dims, S, R, dtype, aligned)


@pytest.mark.parametrize("S,R,dtype,aligned", [(2, 4, torch.float32, False), (2, 4, torch.bfloat16, True),
                                               (4, 8, torch.bfloat16, False), (4, 8, torch.float16, True),
                                               (2, 6, torch.float16, False), (4, 4, torch.float32, True)])
def test_odd_pitch_blocks_all_steps(S, R, dtype, aligned):
    """Parameters sharded on dim 1 whose chunk rows have pitches that are
    not multiples of 16 bytes: short rows and rows of 8-byte units move as
    unit-wise blocks, long rows of 2-byte units one item per row; every
    step against the oracle."""
    shapes = [(64, 6), (33, 12, 3), (9, 20), (1000, 6), (3, 2050, 1), (5, 8, 3), (2, 1030, 4), (7, 4, 5),
              (33, 4, 3), (9, 12), (100, 12), (5,)]
    dims = [1 if len(sh) > 1 and sh[1] % S == 0 else 0 for sh in shapes]
    run_nonzero_dims(shapes, dims, S, R, dtype, aligned)


@pytest.mark.parametrize("S,R,dtype,aligned", [(2, 4, torch.float32, True), (3, 6, torch.bfloat16, True),
                                               (4, 8, torch.float16, True), (8, 8, torch.float32, True),
                                               (16, 16, torch.bfloat16, True), (4, 8, torch.float32, False),
                                               (8, 16, torch.bfloat16, False), (3, 3, torch.float16, False)])
def test_narrow_fold_paths_all_steps(S, R, dtype, aligned):
    """Dim-1 chunks whose rank pieces are 2-12 bytes (2- and 4-byte units):
    AG copy-out, RS copy-in and the RS copy-reduce stage their chunks through
    LDS; with buffers at other offsets modulo 16 (aligned=False) the fold
    reduce takes its unit fallback.  Group sizes cover the compiled operand
    counts and the runtime-count path; every step against the oracle."""
    shapes = [(5000, S), (1700, 3 * S), (900, 2 * S, 1), (333, S, 3), (7,), (40, 5 * S)]
    dims = [1, 1, 1, 1, 0, 1]
    run_nonzero_dims(shapes, dims, S, R, dtype, aligned)


@pytest.mark.parametrize("shapes,S,R,dtype", [
    ([(2000000, 6)], 2, 4, torch.float32),  # 4-byte pieces: LDS-staged folds, ~1500 copy chunks
    ([(20000, 2050, 1)], 2, 2, torch.bfloat16),  # 2050-byte rows at every alignment: folded long rows
    ([(300000, 12), (5000, 1028, 4)], 4, 8, torch.float16),  # 6-byte pieces; 2056-byte rows (8 mod 16)
    ([(10000, 4098)], 2, 2, torch.float32),  # 8196-byte pieces: a full row spans two flat chunks
    ([(3000, 8248)], 8, 8, torch.bfloat16),  # 2062-byte pieces over 8 ranks: flat chunks
    # 2-byte elements in runs of 16 bytes or more: destination vectors read
    # from LDS whole (inside a run) or merged from two reads (across a run end)
    ([(400000, 12, 3)], 4, 4, torch.bfloat16),  # 18-byte pieces
    ([(200000, 40), (30000, 16, 2)], 4, 8, torch.float16),  # 20- and 16-byte pieces
    ([(60000, 22, 3)], 2, 2, torch.bfloat16),  # 66-byte pieces
])
def test_fold_paths_at_scale(shapes, S, R, dtype):
    """The fold kernels over thousands of chunks (tens of MB per rank), every
    step against the oracle bit for bit."""
    run_nonzero_dims(shapes, [1] * len(shapes), S, R, dtype, True)


@pytest.mark.parametrize("shapes,S,R,dtype", [
    ([(7, 4098), (9, 8)], 2, 4, torch.float32),
    ([(5, 8248), (3, 16390)], 2, 2, torch.float16),
    ([(6, 8248)], 4, 8, torch.bfloat16),
    ([(4, 8248), (5, 2056)], 8, 8, torch.float32),
])
@pytest.mark.parametrize("aligned", [True, False])
def test_long_rows_in_flat_chunks(shapes, S, R, dtype, aligned):
    """Dim-1 chunk rows too long for the S pieces of a full row to fit one
    chunk, at per-row alignments: the full tensor is cut into flat chunks
    (fold and fold-reduce items staged through LDS); every step against the
    oracle, buffers at every element offset or at multiples of 16 bytes."""
    run_nonzero_dims(shapes, [1] * len(shapes), S, R, dtype, aligned)


def run_nonzero_dims(shapes, dims, S, R, dtype, aligned):
    note(f"[parity] non-zero shard dims S={S} R={R} dtype={dtype} aligned={aligned}")
    # element offsets of the buffers: any, or multiples of 16 bytes
    v = (16 // (4 if dtype == torch.float32 else 2)) if aligned else 1
    w = W.Workload(f"dims_{S}", 600 + S, R, S, tuple(shapes), dtype, ("normal", 1.0), ("normal", 1.0),
                   ("sum", "avg"), W.ALL_STEPS)
    params, grads = W.params(w), W.grads(w, dtype=dtype)
    lay = O.bucket_layout(shapes, S, shard_dims=dims)
    P, I = len(shapes), lay.I
    xs = [to_oracle(p) for p in params]
    np_dt = np.float32 if dtype == torch.float32 else np.uint16
    ag_o = O.ag_copy_in(O.shard_params(xs, lay), lay, np_dt)
    dparams = [p.cuda() for p in params]
    keep, shards = [], []
    for s in range(S):
        for i in range(P):
            x = dparams[i].narrow(dims[i], lay.row_off[i][s], lay.row_len[i][s]).contiguous().reshape(-1)
            g = Guarded(x.numel(), dtype, v * ((s + i) % 5))
            g.t.copy_(x)
            keep.append(g)
            shards.append(g.t)
    ag = Guarded(S * I, dtype, 3 * v)
    hp.fsdp_ag_copy_in(shapes, S, shards, ag.t, shard_dims=dims)
    full = [Guarded(p.numel(), dtype, v) for p in params]
    hp.fsdp_ag_copy_out(shapes, S, ag.t, [f.t for f in full], shard_dims=dims)
    torch.cuda.synchronize()
    assert ag.guards_intact() and first_mismatch(bits(ag.t), np_bits(ag_o)) == ""
    for i in range(P):
        assert full[i].guards_intact() and np.array_equal(bits(full[i].t), np_bits(xs[i]))
    # reduction operands in the oracle's value forms (fp16 as numpy float16)
    gnp = [[to_oracle_values(g) for g in grads[r]] for r in range(R)]
    rs_o = [O.rs_copy_in(gnp[g], lay, NP16.get(dtype, np.float32)) for g in range(R)]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    rs_in = [Guarded(S * I, dtype, v * (g % 3)) for g in range(R)]
    hp.fsdp_rs_copy_in(shapes, R, S, dgrads, [b.t for b in rs_in], shard_dims=dims)
    for op in (O.SUM, O.AVG):
        want = O.rs_reduce(rs_o, I, R, S, op)
        out = [Guarded(I, dtype, v * (1 + g % 2)) for g in range(R)]
        hp.fsdp_rs_reduce(shapes, R, S, R // S, op, [b.t for b in rs_in], [o.t for o in out], shard_dims=dims)
        out2 = [Guarded(I, dtype, v * (g % 4)) for g in range(R)]
        hp.fsdp_rs_copy_reduce(shapes, R, S, R // S, op, dgrads, [o.t for o in out2], shard_dims=dims)
        torch.cuda.synchronize()
        for g in range(R):
            assert rs_in[g].guards_intact() and first_mismatch(bits(rs_in[g].t), np_bits(rs_o[g])) == ""
            assert out[g].guards_intact() and first_mismatch(bits(out[g].t), np_bits(want[g])) == ""
            assert out2[g].guards_intact() and first_mismatch(bits(out2[g].t), np_bits(want[g])) == ""


def test_plan_cache_reuse_and_eviction():
    """Distinct calls get their own plans; more distinct calls than the
    cache holds evict old plans (after the device drains) without changing
    any result; repeated calls reuse plans."""
    note("[parity] plan cache eviction")
    shapes = [(7, 8), (5, 3), (16,)]
    S = 4
    lay = O.bucket_layout(shapes, S)
    xs = [torch.randn(sh) for sh in shapes]
    want = O.ag_copy_in(O.shard_params([x.numpy() for x in xs], lay), lay, np.float32)
    dparams = [x.cuda() for x in xs]
    shards, _ = make_shards(dparams, lay, torch.float32)
    outs = [torch.full((S * lay.I,), float("nan"), device="cuda") for _ in range(300)]
    for rnd in range(2):
        for o in outs:
            o.fill_(float("nan"))
        for o in outs:  # 300 distinct signatures (the output pointer differs)
            hp.fsdp_ag_copy_in(shapes, S, shards, o)
        for o in outs[:20]:  # repeats: cached or re-planned, same result
            hp.fsdp_ag_copy_in(shapes, S, shards, o)
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(bits(o), np_bits(want))


# ---------------------------------------------------------------------------
# IEEE special values through the reductions
# ---------------------------------------------------------------------------

SPECIAL_F32 = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 3.0, np.inf, -np.inf, np.nan, 1e-40, -1e-41, 1.4e-45,
                        3.4028235e38, -3.4028235e38, 1e38, 2.0 ** -126, 7.0, -2.5], dtype=np.float32)


# fp16's own edges: its largest finite value, denormals, the smallest
# normal, values whose sums overflow
SPECIAL_F16 = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 3.0, np.inf, -np.inf, np.nan, 65504.0, -65504.0, 6e-8, -3e-8,
                        6.1035156e-05, 3e4, 7.0, -2.5, 1e-3], dtype=np.float32)


def _special(n, rng, dtype):
    pool = SPECIAL_F16 if dtype == torch.float16 else SPECIAL_F32
    t = torch.from_numpy(pool[rng.integers(0, len(pool), n)])
    return t if dtype == torch.float32 else t.to(dtype)


def _same_up_to_nan_payload(got_t, want_np):
    """Bit-equal everywhere the oracle is not NaN; NaN where it is (fp32 and
    fp16 NaN payloads are not part of the result; bf16 NaN is one pattern,
    0x7FC0, on both sides and compared bit for bit)."""
    got = bits(got_t)
    want = np_bits(want_np)
    if want_np.dtype in (np.float32, np.float16):
        nan = np.isnan(want_np.reshape(-1))
        g = got_t.detach().cpu().float().numpy().reshape(-1)
        if not np.array_equal(np.isnan(g), nan):
            return "NaN positions differ"
        got, want = got[~nan], want[~nan]
    return first_mismatch(got, want)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("R,S", [(8, 4), (6, 3), (8, 8), (6, 2), (6, 1), (12, 6)])
def test_special_values_rs_and_fused_ar(dtype, R, S):
    """Signed zeros, infinities, NaN, denormals and values that overflow when
    added, through the RS (from the RS input and straight from the
    gradients) and the fused AR, SUM and AVG (AVG by 3 included): the fixed
    ascending order, IEEE fp32 with denormals kept, and one rounding to
    bf16."""
    note(f"[parity] special values dtype={dtype} R={R} S={S}")
    rng = np.random.default_rng(R * 10 + S + (dtype == torch.bfloat16) + 2 * (dtype == torch.float16))
    shapes = [(1027, 3), (5,), (2049,)]
    lay = O.bucket_layout(shapes, S)
    I, P, D = lay.I, len(shapes), R // S
    grads = [[_special(int(np.prod(sh)), rng, dtype).reshape(sh) for sh in shapes] for _ in range(R)]
    gnp = [[to_oracle_values(t) for t in grads[g]] for g in range(R)]
    np_dt = np.float32 if dtype == torch.float32 else NP16[dtype]
    dgrads = [grads[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    rs_in = [torch.empty(S * I, dtype=dtype, device="cuda") for _ in range(R)]
    hp.fsdp_rs_copy_in(shapes, R, S, dgrads, rs_in)
    rs_o = [O.rs_copy_in(gnp[g], lay, np_dt) for g in range(R)]
    with np.errstate(all="ignore"):
        for op in (O.SUM, O.AVG):
            want = O.rs_reduce(rs_o, I, R, S, op)
            out = [torch.empty(I, dtype=dtype, device="cuda") for _ in range(R)]
            out2 = [torch.empty(I, dtype=dtype, device="cuda") for _ in range(R)]
            hp.fsdp_rs_reduce(shapes, R, S, D, op, rs_in, out)
            hp.fsdp_rs_copy_reduce(shapes, R, S, D, op, dgrads, out2)
            torch.cuda.synchronize()
            for g in range(R):
                assert _same_up_to_nan_payload(out[g], want[g]) == "", f"rs_reduce {op} rank {g}"
                assert _same_up_to_nan_payload(out2[g], want[g]) == "", f"rs_copy_reduce {op} rank {g}"
            if D > 1:
                segs = [I, 300]
                offs, F = O.fused_layout(segs, 4 if dtype == torch.float32 else 2)
                fused_np = []
                for g in range(R):
                    f = np.zeros(F, np_dt)
                    f[offs[0]:offs[0] + I] = want[g]
                    f[offs[1]:offs[1] + 300] = to_oracle_values(_special(300, rng, dtype))
                    fused_np.append(f)
                fused = [torch.from_numpy(f.view(np.int16) if np_dt == np.uint16 else f).cuda() for f in fused_np]
                if dtype == torch.bfloat16:
                    fused = [f.view(torch.bfloat16) for f in fused]
                want_ar = O.fused_ar(fused_np, R, S, op)
                hp.fsdp_fused_ar(segs, R, S, D, op, fused)
                torch.cuda.synchronize()
                for g in range(R):
                    assert _same_up_to_nan_payload(fused[g], want_ar[g]) == "", f"fused_ar {op} rank {g}"


def test_concurrent_calls_from_threads_on_their_own_streams():
    """Four host threads, each with its own bucket and stream, issue passes
    concurrently (ctypes releases the GIL, so the library's plan cache is
    shared by truly concurrent callers); every thread's results match the
    oracle."""
    import threading
    R, S = 8, 4
    shape_sets = [[(7, 8), (5, 3), (16,)], [(1000, 3), (129,)], [(4097, 2), (3,)], [(33, 7), (2048, 64)]]
    note("[parity] concurrent threads")
    work = []
    for t, shapes in enumerate(shape_sets):
        w = W.Workload(f"thread_{t}", 700 + t, R, S, tuple(shapes), torch.float32, ("normal", 1.0), ("normal", 1.0),
                       ("avg",), W.ALL_STEPS)
        g_cpu = W.grads(w)
        params = W.params(w)
        fb = hp.FlatBucket(shapes, R, S, torch.float32, op=O.AVG)
        fb.bind(fb.shard_views([p.cuda() for p in params]),
                [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(len(shapes))])
        _, fused_o, _, _ = O.reduce_grads_fused([[x.numpy() for x in g_cpu[g]] for g in range(R)], [shapes], R, S,
                                                O.AVG)
        work.append((fb, params, fused_o, torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def run(fb, stream):
        try:
            for k in range(20):
                fb.step(stream, fused_rs=bool(k % 2))
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(fb, st)) for fb, _, _, st in work]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for fb, params, fused_o, _ in work:
        for i, p in enumerate(params):
            assert np.array_equal(bits(fb.full[i]), bits(p.reshape(-1)))
        for g in range(R):
            assert first_mismatch(bits(fb.fused[g]), np_bits(fused_o[g])) == "", f"rank {g}"


def test_many_passes_stay_bit_identical():
    """600 passes of the HSDP block (unfused and fused RS alternating in
    runs of 100, on the current stream and a side stream) leave every
    output bit-identical to the first pass's, which matches the oracle."""
    w = W.HSDP_BLOCK
    R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
    note(f"[parity] {w.name}: 600 passes")
    params, g_cpu = W.params(w), W.grads(w)
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG)
    fb.bind(fb.shard_views([p.cuda() for p in params]),
            [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)])
    fb.step()
    torch.cuda.synchronize()
    gnp = [[t.numpy() for t in g_cpu[g]] for g in range(R)]
    _, fused_o, _, _ = O.reduce_grads_fused(gnp, [list(w.param_shapes)], R, S, O.AVG)
    for g in range(R):
        assert first_mismatch(bits(fb.fused[g]), np_bits(fused_o[g])) == "", f"first pass rank {g}"
    first_full = [f.clone() for f in fb.full]
    first_fused = [f.clone() for f in fb.fused]
    side = torch.cuda.Stream()
    for run in range(6):
        stream = side if run % 2 else None
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())
        for _ in range(100):
            fb.step(stream, fused_rs=bool(run % 3 == 1))
        if stream is not None:
            torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        for a, b in zip(fb.full, first_full):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"full params after run {run}"
        for g, (a, b) in enumerate(zip(fb.fused, first_fused)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"fused rank {g} after run {run}"


@pytest.mark.parametrize("fused_rs", [False, True])
def test_fused_group_one_ar_over_per_parameter_buckets(fused_rs):
    """The HSDP block with one bucket per parameter: six RS outputs as
    512-byte-aligned segments of one fused buffer per rank, one fused AR;
    the fused buffers (gaps included) and the gathered parameters against
    the oracle's fused path, issued eagerly and replayed from the step
    captured over three streams."""
    w = W.scaled(W.HSDP_BLOCK, [(97, 64), (32, 64), (130, 32), (33, 128), (64,), (3,)])
    R, S = w.rank_size, w.shard_size
    buckets = [[sh] for sh in w.param_shapes]
    note(f"[parity] FusedGroup of {len(buckets)} buckets fused_rs={fused_rs}")
    params, g_cpu = W.params(w), W.grads(w)
    grp = hp.FusedGroup(buckets, R, S, w.param_dtype, op=O.AVG)
    dparams = [p.cuda() for p in params]
    shards = [fb.shard_views([dparams[k]]) for k, fb in enumerate(grp.buckets)]
    grads = [[g_cpu[g][k].cuda().reshape(-1) for g in range(R)] for k in range(len(buckets))]
    grp.bind(shards, grads)
    graph = None
    for rep in range(5):
        if rep == 2:  # then replays of the step captured over three streams
            graph = grp.graph(n_streams=3, fused_rs=fused_rs)
        for fb in grp.buckets:
            for v in fb.rs_out:
                v.fill_(float("nan"))
            fb.full[0].view(torch.int16).fill_(0x7FA5)
        torch.cuda.synchronize()
        if graph is None:
            grp.step(fused_rs=fused_rs)
        else:
            graph.replay()
        torch.cuda.synchronize()
        gnp = [[t.numpy() for t in g_cpu[g]] for g in range(R)]
        _, fused_o, offs_o, _ = O.reduce_grads_fused(gnp, buckets, R, S, O.AVG)
        assert [fb.fused_off for fb in grp.buckets] == offs_o
        for g in range(R):
            m = first_mismatch(bits(grp.fused[g]), np_bits(fused_o[g]))
            assert m == "", f"rep {rep} fused rank {g}: {m}"
        for k, fb in enumerate(grp.buckets):
            assert np.array_equal(bits(fb.full[0]), bits(params[k].reshape(-1))), f"rep {rep} param {k}"
    del graph


def test_backward_pipeline_over_shared_fused_buffers():
    """BackwardPipeline over the buckets of one FusedGroup (their RS outputs
    are segments of shared fused buffers): each bucket's own fused AR covers
    only its segment and gap, so the per-layer ARs never re-reduce another
    bucket's segment (SUM would multiply it by D per extra AR) nor race with
    the next bucket's RS into the same buffers.  Eager and replayed, both
    orders, against the oracle's fused path over the same buckets."""
    w = W.scaled(W.HSDP_BLOCK, [(97, 64), (32, 64), (130, 32), (33, 128), (64,), (3,)])
    R, S = w.rank_size, w.shard_size
    buckets = [[sh] for sh in w.param_shapes]
    note(f"[parity] backward pipeline over a FusedGroup of {len(buckets)} buckets (SUM)")
    g_cpu = W.grads(w)
    grp = hp.FusedGroup(buckets, R, S, w.param_dtype, op=O.SUM)
    zeros = [torch.zeros(sh, dtype=w.param_dtype, device="cuda") for sh in w.param_shapes]
    grp.bind([fb.shard_views([zeros[k]]) for k, fb in enumerate(grp.buckets)],
             [[g_cpu[g][k].cuda().reshape(-1) for g in range(R)] for k in range(len(buckets))])
    gnp = [[t.numpy() for t in g_cpu[g]] for g in range(R)]
    _, fused_o, offs_o, _ = O.reduce_grads_fused(gnp, buckets, R, S, O.SUM)
    assert [fb.fused_off for fb in grp.buckets] == offs_o
    pipe = hp.BackwardPipeline(grp.buckets, fused_rs=True)
    graphs = {}
    for rep in range(6):
        for fb in grp.buckets:
            for v in fb.rs_out:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        if rep < 2:
            (pipe.run_pipelined if rep == 0 else pipe.run_serial)()
        else:
            pipelined = rep % 2 == 0
            if pipelined not in graphs:
                graphs[pipelined] = pipe.graph(pipelined=pipelined)
                for fb in grp.buckets:
                    for v in fb.rs_out:
                        v.fill_(float("nan"))
                torch.cuda.synchronize()
            graphs[pipelined].replay()
        torch.cuda.synchronize()
        for g in range(R):
            m = first_mismatch(bits(grp.fused[g]), np_bits(fused_o[g]))
            assert m == "", f"rep {rep} fused rank {g}: {m}"
    graphs.clear()


def test_fused_group_with_shard_dims():
    """A FusedGroup whose buckets shard some parameters on dim 1: every
    bucket's RS output lands in its segment of the shared fused buffers and
    one AR covers them; the buffers against the oracle's RS copy-in, RS,
    fused layout and fused AR composed per bucket."""
    R, S = 8, 4
    buckets = [[(64, 48), (7,)], [(33, 16, 3)], [(100,)]]
    dims = [[1, 0], [1], None]
    note("[parity] FusedGroup with shard dims")
    grp = hp.FusedGroup(buckets, R, S, torch.bfloat16, op=O.AVG, shard_dims=dims)
    flat = [sh for b in buckets for sh in b]
    w = W.Workload("fused_group_dims", 31, R, S, tuple(flat), torch.bfloat16, ("normal", 0.02), ("normal", 1.0),
                   ("avg",), W.ALL_STEPS)
    params, g_cpu = W.params(w), W.grads(w)
    j, shards, grads, segs_o = 0, [], [], [[] for _ in range(R)]
    for k, (b, d) in enumerate(zip(buckets, dims)):
        P = len(b)
        shards.append(grp.buckets[k].shard_views([p.cuda() for p in params[j:j + P]]))
        grads.append([g_cpu[g][j + i].cuda().reshape(-1) for g in range(R) for i in range(P)])
        lay = O.bucket_layout(b, S, shard_dims=d)
        rs_in = [O.rs_copy_in([g_cpu[g][j + i].numpy() for i in range(P)], lay) for g in range(R)]
        for g, out in enumerate(O.rs_reduce(rs_in, lay.I, R, S, O.AVG)):
            segs_o[g].append(out)
        j += P
    grp.bind(shards, grads)
    offs, F = O.fused_layout(grp.seg_numel)
    fused_o = []
    for g in range(R):
        buf = np.zeros(F, np.float32)
        for o, seg in zip(offs, segs_o[g]):
            buf[o:o + seg.size] = seg
        fused_o.append(buf)
    want = O.fused_ar(fused_o, R, S, O.AVG)
    for fused_rs in (False, True):
        for f in grp.fused:
            f.zero_()
        grp.step(fused_rs=fused_rs)
        torch.cuda.synchronize()
        for g in range(R):
            m = first_mismatch(bits(grp.fused[g]), np_bits(want[g]))
            assert m == "", f"fused_rs={fused_rs} rank {g}: {m}"
        j = 0
        for k, b in enumerate(buckets):
            for i in range(len(b)):
                assert np.array_equal(bits(grp.buckets[k].full[i]), bits(params[j + i].reshape(-1)))
            j += len(b)


@pytest.mark.parametrize("fused_rs", [False, True])
def test_hip_graph_capture_of_cached_plans(fused_rs):
    """Once a call signature's plan is cached, issuing it only launches a
    kernel, so a whole pass can be captured in a HIP graph
    (torch.cuda.graph) and replayed: every replay, with new gradient values
    written eagerly between replays, matches the oracle."""
    import dataclasses
    w = W.scaled(W.HSDP_BLOCK, [(97, 64), (32, 64), (130, 32), (33, 128), (64,), (3,)])
    R, S, P = w.rank_size, w.shard_size, len(w.param_shapes)
    note(f"[parity] HIP graph capture fused_rs={fused_rs}")
    params, g_cpu = W.params(w), W.grads(w)
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG)
    grads_dev = [g_cpu[g][i].cuda().reshape(-1) for g in range(R) for i in range(P)]
    fb.bind(fb.shard_views([p.cuda() for p in params]), grads_dev)
    fb.step(fused_rs=fused_rs)  # plans cached (tables uploaded) before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fb.step(fused_rs=fused_rs)
    for rep in range(3):
        new = W.grads(dataclasses.replace(w, number=w.number + 100 + rep))
        for t, v in zip(grads_dev, [new[g][i].reshape(-1) for g in range(R) for i in range(P)]):
            t.copy_(v)
        for f in fb.full:
            f.view(torch.int16).fill_(0x7FA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gnp = [[t.numpy() for t in new[g]] for g in range(R)]
        _, fused_o, _, _ = O.reduce_grads_fused(gnp, [list(w.param_shapes)], R, S, O.AVG)
        for g in range(R):
            m = first_mismatch(bits(fb.fused[g]), np_bits(fused_o[g]))
            assert m == "", f"replay {rep} fused rank {g}: {m}"
        for i in range(P):
            assert np.array_equal(bits(fb.full[i]), bits(params[i].reshape(-1))), f"replay {rep} param {i}"


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_captured_plans_are_pinned_through_eviction():
    """A plan launched into a graph capture is pinned: after more new call
    signatures than the cache holds, it is still cached and the graph still
    replays correctly.  The first call of a signature under capture is
    refused before anything is enqueued, and works once issued eagerly."""
    note("[parity] captured plans pinned through eviction")
    hp.fsdp_release_cache()
    shapes, S = [(97, 64), (3,), (130, 32), (5,)], 4
    lay = O.bucket_layout(shapes, S)
    gen = torch.Generator().manual_seed(99)
    xs = [torch.randn(sh, generator=gen) for sh in shapes]
    dparams = [x.cuda() for x in xs]
    shards, _ = make_shards(dparams, lay, torch.float32)
    ag = torch.empty(S * lay.I, device="cuda")
    full = [torch.empty(_numel(sh), device="cuda") for sh in shapes]
    hp.fsdp_ag_copy_in(shapes, S, shards, ag)
    hp.fsdp_ag_copy_out(shapes, S, ag, full)
    torch.cuda.synchronize()
    assert hp.fsdp_cache_info()["pinned"] == 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hp.fsdp_ag_copy_in(shapes, S, shards, ag)
        hp.fsdp_ag_copy_out(shapes, S, ag, full)
    assert hp.fsdp_cache_info()["pinned"] == 2

    # 300 new signatures (one destination offset each): more than the cache
    # holds, so every plan that is not pinned is evicted at least once
    src = torch.randn(16, device="cuda")
    dst = torch.empty(16 + 300, device="cuda")
    for k in range(300):
        hp.fsdp_ag_copy_in([(16,)], 1, [src], dst[k:k + 16])
    torch.cuda.synchronize()
    info = hp.fsdp_cache_info()
    assert info["plans"] < 300 and info["pinned"] == 2, info
    assert torch.equal(dst[299:315], src)

    for rep in range(2):
        ys = [torch.randn(sh, generator=gen) for sh in shapes]
        for d, y in zip(dparams, ys):
            d.copy_(y)
        ag.view(torch.int32).fill_(0x7FA5A5A5)
        for f in full:
            f.view(torch.int32).fill_(0x7FA5A5A5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = O.ag_copy_in(O.shard_params([y.numpy() for y in ys], lay), lay, np.float32)
        assert first_mismatch(bits(ag), np_bits(want)) == "", f"replay {rep}"
        for i in range(len(shapes)):
            assert np.array_equal(bits(full[i]), np_bits(ys[i].numpy().reshape(-1))), f"replay {rep} param {i}"

    # an uncached signature under capture: refused, nothing enqueued
    new_shapes = [(9, 5), (2,)]
    lay2 = O.bucket_layout(new_shapes, 2)
    zs = [torch.randn(sh, generator=gen) for sh in new_shapes]
    shards2, _ = make_shards([z.cuda() for z in zs], lay2, torch.float32)
    ag2 = torch.full((2 * lay2.I,), float("nan"), device="cuda")
    before = hp.fsdp_cache_info()
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(hp.FSDPError, match="captured"):
        with torch.cuda.graph(g2):
            hp.fsdp_ag_copy_in(new_shapes, 2, shards2, ag2)
    del g2
    assert hp.fsdp_cache_info() == before
    torch.cuda.synchronize()
    assert torch.isnan(ag2).all()
    hp.fsdp_ag_copy_in(new_shapes, 2, shards2, ag2)
    torch.cuda.synchronize()
    want2 = O.ag_copy_in(O.shard_params([z.numpy() for z in zs], lay2), lay2, np.float32)
    assert first_mismatch(bits(ag2), np_bits(want2)) == ""
    del graph
    hp.fsdp_release_cache()
    assert hp.fsdp_cache_info() == {"plans": 0, "pinned": 0, "table_bytes": 0}


def test_time_next_launch_records_the_kernel():
    """fsdp_time_next_launch: the next kernel's dispatch records the event
    pair (a duration no shorter than its bytes at 8 TB/s); later launches
    leave the events alone; a call that launches nothing (an AR over one
    replica) leaves the request pending for the next launch."""
    note("[parity] fsdp_time_next_launch")
    n = 1 << 26  # 256 MiB of fp32 per side
    src = torch.randn(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    b.record()
    torch.cuda.synchronize()
    hp.fsdp_time_next_launch(a, b)
    hp.fsdp_ag_copy_in([(n,)], 1, [src], dst)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3
    assert torch.equal(dst, src)
    assert 2 * n * 4 / (8000e9) * 1e6 <= us < 100000, us
    hp.fsdp_ag_copy_in([(n,)], 1, [dst], src)  # not timed
    torch.cuda.synchronize()
    assert a.elapsed_time(b) * 1e3 == us
    # pending across a call with nothing to launch (D = 1: the AR is the identity)
    f = torch.zeros(128, device="cuda")
    hp.fsdp_time_next_launch(a, b)
    hp.fsdp_fused_ar([128], 1, 1, 1, "avg", [f])
    hp.fsdp_ag_copy_in([(n // 4,)], 1, [src[:n // 4]], dst[:n // 4])
    torch.cuda.synchronize()
    us2 = a.elapsed_time(b) * 1e3
    assert us2 != us and 0 < us2 < us, (us2, us)
    # pending across a launch into a graph capture (the graph records no
    # events), taken by the next launch outside it
    m = n // 16
    hp.fsdp_ag_copy_in([(m,)], 1, [src[:m]], dst[:m])  # cached before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    hp.fsdp_time_next_launch(a, b)
    with torch.cuda.graph(graph):
        hp.fsdp_ag_copy_in([(m,)], 1, [src[:m]], dst[:m])
    torch.cuda.synchronize()
    dst[:m].zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(dst[:m], src[:m])
    assert a.elapsed_time(b) * 1e3 == us2  # the capture and the replay left the events alone
    hp.fsdp_ag_copy_in([(n // 2,)], 1, [src[:n // 2]], dst[:n // 2])
    torch.cuda.synchronize()
    us3 = a.elapsed_time(b) * 1e3
    assert us3 != us2 and 0 < us3 < us, (us3, us2, us)
    del graph
    hp.fsdp_time_next_launch(None, None)
