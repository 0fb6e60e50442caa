"""Full-size parity on the two big workloads, in the launch configuration the
benchmark times (FlatBucket, inputs resident in HBM).

The oracle cannot materialise these buffers quickly, so it is evaluated
element by element (oracle/pointwise.py) at a few hundred thousand random
positions plus every position next to a region, padding or slice edge, and
compared bit for bit.  Properties that hold at any size are checked on the
whole buffers: all_gather(shard(x)) == x and every padding element is 0.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import bits, note, require_gpu
from oracle import pointwise as PW

hp = pytest.importorskip("hsdp_parameter_gradient_amd")

pytestmark = pytest.mark.gpu

N_RANDOM = 300_000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    hp.lib()
    yield
    hp.fsdp_release_cache()
    torch.cuda.empty_cache()


def _np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _fetcher(tensors):
    """fetch(i, flat) -> host values (float32 or uint16 bits) of tensors[i]."""
    def fetch(i, flat):
        idx = torch.from_numpy(np.asarray(flat, dtype=np.int64)).cuda()
        v = tensors[i].reshape(-1)[idx]
        return v.cpu().numpy() if v.dtype == torch.float32 else _np16(v)
    return fetch


def _gpu_vals(t, pos):
    idx = torch.from_numpy(np.asarray(pos, dtype=np.int64)).cuda()
    return bits(t.reshape(-1)[idx])


@pytest.mark.parametrize("wname", ["llama7b_4layer_r8_s8", "ragged_heavy_r8_s8"])
def test_full_size_sampled(wname):
    w = W.WORKLOADS[wname]
    R, S, D = w.rank_size, w.shard_size, w.dp_size
    P = len(w.param_shapes)
    lay = O.bucket_layout(w.param_shapes, S)
    I = lay.I
    rng = np.random.default_rng(w.number)
    note(f"[fullsize] {w.name}: P={P} I={I} R={R} S={S}")

    params = W.params(w, device="cuda")
    grads = W.grads(w, device="cuda")
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG)
    fb.bind(fb.shard_views(params), [grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
    for step in ("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"):
        fb.run(step)
    torch.cuda.synchronize()
    np_dtype = np.float32 if w.param_dtype == torch.float32 else np.uint16
    to_bits = (lambda a: a.view(np.int32)) if np_dtype == np.float32 else (lambda a: a.view(np.int16))

    # --- AG copy-in: sampled values, and all padding is zero -------------
    edges = PW.boundary_positions(lay)
    pos = np.unique(np.concatenate([rng.integers(0, S * I, N_RANDOM),
                                    (np.arange(S)[:, None] * I + edges[None, :]).reshape(-1)]))
    want = PW.packed_values(lay, pos, _fetcher(params), np_dtype)
    got = _gpu_vals(fb.ag, pos)
    assert np.array_equal(got, to_bits(want)), "ag_copy_in sampled mismatch"
    pad_nonzero = 0
    for s in range(S):
        for i in range(P):
            a = s * I + lay.in_off[i] + lay.row_len[i][s] * lay.inner[i]
            b = s * I + lay.in_off[i] + lay.padded[i]
            if b > a:
                pad_nonzero += int(torch.count_nonzero(fb.ag[a:b].view(torch.int16 if np_dtype == np.uint16 else torch.int32)))
    assert pad_nonzero == 0

    # --- AG copy-out: the round trip is exact on every element -----------
    for i in range(P):
        it = torch.int16 if np_dtype == np.uint16 else torch.int32
        assert torch.equal(fb.full[i].reshape(-1).view(it), params[i].reshape(-1).view(it)), \
            f"ag_copy_out param {i} differs from the parameter"
        n = fb.full[i].numel()
        if n:
            flat = np.unique(np.concatenate([rng.integers(0, n, 2000), [0, n - 1]]))
            src = PW.unpacked_sources(lay, i, flat)
            assert np.array_equal(_gpu_vals(fb.full[i], flat), _gpu_vals(fb.ag, src))

    # --- RS copy-in: sampled per rank -------------------------------------
    for g in range(R):
        pos = np.unique(np.concatenate([rng.integers(0, S * I, N_RANDOM // R),
                                        (np.arange(S)[:, None] * I + edges[None, :]).reshape(-1)]))
        want = PW.packed_values(lay, pos, _fetcher(grads[g]), np.float32)
        assert np.array_equal(_gpu_vals(fb.rs_in[g], pos), want.view(np.int32)), f"rs_copy_in rank {g}"

    # --- RS reduce (AVG, then SUM): sampled, from the gradients directly ---
    fetch_rs_in = lambda m, p: PW.packed_values(lay, p, _fetcher(grads[m]), np.float32)  # noqa: E731
    for op in (O.AVG, O.SUM):
        if op == O.SUM:
            hp.fsdp_rs_reduce(w.param_shapes, R, S, D, op, fb.rs_in, fb.rs_out)
            torch.cuda.synchronize()
        for g in range(R):
            k = np.unique(np.concatenate([rng.integers(0, I, N_RANDOM // R), edges]))
            want = PW.rs_reduce_values(I, R, S, op, g, k, fetch_rs_in)
            assert np.array_equal(_gpu_vals(fb.rs_out[g], k), want.view(np.int32)), f"rs_reduce {op} rank {g}"
    # --- RS copy-in fused into the RS: the whole result equals the two-step
    # one (SUM, just computed) bit for bit, and samples match the oracle ---
    fused_out = [torch.empty(I, dtype=torch.float32, device="cuda") for _ in range(R)]
    hp.fsdp_rs_copy_reduce(w.param_shapes, R, S, D, O.SUM, [grads[g][i].reshape(-1) for g in range(R) for i in range(P)],
                           fused_out)
    torch.cuda.synchronize()
    for g in range(R):
        assert torch.equal(fused_out[g].view(torch.int32), fb.rs_out[g].view(torch.int32)), f"rs_copy_reduce rank {g}"
        k = np.unique(np.concatenate([rng.integers(0, I, N_RANDOM // R), edges]))
        want = PW.rs_reduce_values(I, R, S, O.SUM, g, k, fetch_rs_in)
        assert np.array_equal(_gpu_vals(fused_out[g], k), want.view(np.int32)), f"rs_copy_reduce sampled rank {g}"
    del fb, params, grads, fused_out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wname,grad_dtype,on_dim_1", [
    ("hsdp_block_h1024_r8_s4_d2", torch.float32, True), ("llama7b_4layer_r8_s8", torch.float32, True),
    ("hsdp_block_h1024_r8_s4_d2", torch.bfloat16, False), ("hsdp_block_h1024_r8_s4_d2", torch.float16, False),
    ("hsdp_block_h1024_r8_s4_d2", torch.bfloat16, True)])
def test_full_size_properties(wname, grad_dtype, on_dim_1):
    """The benchmark's variants at full size (the 2-D weights sharded on dim
    1 as strided blocks; bf16 and fp16 gradients), in the benchmark's
    configuration, checked on every element by properties that hold at any
    size: each AG slice region is the dense chunk of its parameter, copy-out
    restores the parameters bit for bit, each RS input region is the dense
    chunk of the gradient, and with integer-valued gradients (every sum and
    quotient exact in the gradient dtype, whatever the order) the RS output
    is the chunk of the group's sum divided by S, and the fused AR output
    that divided by D."""
    w = W.WORKLOADS[wname]
    R, S, D = w.rank_size, w.shard_size, w.dp_size
    P = len(w.param_shapes)
    dims = [1 if on_dim_1 and len(sh) > 1 and sh[1] % S == 0 else 0 for sh in w.param_shapes]
    lay = O.bucket_layout(w.param_shapes, S, shard_dims=dims)
    I = lay.I
    note(f"[fullsize] {w.name} {grad_dtype} shard dims {sorted(set(dims))}: P={P} I={I} R={R} S={S}")
    params = W.params(w, device="cuda")
    grads = [[t.to(grad_dtype) for t in row] for row in W.integer_grads(w, device="cuda")]
    fb = hp.FlatBucket(w.param_shapes, R, S, w.param_dtype, op=O.AVG, shard_dims=dims, grad_dtype=grad_dtype)
    fb.bind(fb.shard_views(params), [grads[g][i].reshape(-1) for g in range(R) for i in range(P)])
    fb.step()
    torch.cuda.synchronize()
    it = torch.int16 if w.param_dtype != torch.float32 else torch.int32

    def chunk(x, i, s):
        c = x.narrow(dims[i], lay.row_off[i][s], lay.row_len[i][s]).contiguous().reshape(-1)
        return c

    def region(buf, s, i, n):
        a = s * I + lay.in_off[i]
        return buf[a:a + n]

    for i in range(P):
        assert torch.equal(fb.full[i].reshape(-1).view(it), params[i].reshape(-1).view(it)), f"ag_copy_out {i}"
        for s in range(S):
            c = chunk(params[i], i, s)
            r = region(fb.ag, s, i, lay.padded[i])
            assert torch.equal(r[:c.numel()].view(it), c.view(it)), f"ag_copy_in slice {s} param {i}"
            assert int(torch.count_nonzero(r[c.numel():].view(it))) == 0, f"ag padding {s} {i}"
    for g in range(R):
        for i in range(P):
            for s in range(S):
                c = chunk(grads[g][i], i, s)
                r = region(fb.rs_in[g], s, i, lay.padded[i])
                assert torch.equal(r[:c.numel()], c) and int(torch.count_nonzero(r[c.numel():])) == 0, \
                    f"rs_copy_in rank {g} slice {s} param {i}"
    for d in range(D):
        for s in range(S):
            g = d * S + s
            for i in range(P):
                want = sum(chunk(grads[d * S + t][i], i, s) for t in range(S)) / S
                if D > 1:  # the fused AR over the replicate group of g
                    want = sum(sum(chunk(grads[e * S + t][i], i, s) for t in range(S)) / S for e in range(D)) / D
                got = fb.rs_out[g][lay.in_off[i]:lay.in_off[i] + want.numel()]
                assert torch.equal(got, want), f"reduced rank {g} param {i}"
    # the fused RS pass gives the same fused buffers bit for bit
    before = [f.clone() for f in fb.fused]
    for v in fb.rs_out:
        v.fill_(float("nan"))
    fb.step(fused_rs=True)
    torch.cuda.synchronize()
    gi = torch.int32 if grad_dtype == torch.float32 else torch.int16
    for g in range(R):
        assert torch.equal(fb.fused[g].view(gi), before[g].view(gi)), f"fused RS rank {g}"
    del fb, params, grads, before
    torch.cuda.empty_cache()


def test_items_beyond_4gib():
    """A copy segment and a reduction job each larger than 4 GiB (64-bit
    offsets everywhere): AG copy-in of one bf16 parameter of 2^31 + 1001
    elements with shard_size 1 (one 4 GiB + 2 KiB segment), and the fused
    AR of two replicas of 2^30 + 1000 fp32 elements (integer-valued, so the
    sum is exact)."""
    note("[fullsize] items beyond 4 GiB")
    n = (1 << 31) + 1001
    x = torch.empty(n, dtype=torch.int16, device="cuda").random_().view(torch.bfloat16)
    ag = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    hp.fsdp_ag_copy_in([(n,)], 1, [x], ag)
    torch.cuda.synchronize()
    assert torch.equal(ag.view(torch.int16), x.view(torch.int16))
    del x, ag
    torch.cuda.empty_cache()

    m = (1 << 30) + 1000
    _, F = hp.fsdp_fused_layout([m], 4)
    fused = [torch.zeros(F, dtype=torch.float32, device="cuda") for _ in range(2)]
    for k, f in enumerate(fused):
        f[:m] = torch.randint(-8, 9, (m,), device="cuda", generator=torch.Generator("cuda").manual_seed(k)).float()
    want = fused[0] + fused[1]
    hp.fsdp_fused_ar([m], 2, 1, 2, O.SUM, fused)
    torch.cuda.synchronize()
    for f in fused:
        assert torch.equal(f, want)
    del fused, want
    torch.cuda.empty_cache()
