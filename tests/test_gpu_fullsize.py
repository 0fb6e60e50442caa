"""Full-size parity on the two largest workloads, every element, in the
launch configuration the benchmark times (FlatBucket with prepared calls,
inputs resident in HBM).

The oracle runs at full size on the host, streamed rank by rank: the AG
buffer and the full parameters from the host copy of the parameters, each
rank's RS input from that rank's gradients (copied back from the device,
where the workload draws them), the RS outputs from the oracle's own RS
inputs.  Every element of ag, full[i], rs_in[g], rs_out[g] (AVG and SUM)
and of the fused RS copy-reduce output (AVG and SUM) is compared bit for
bit.  Every output buffer is filled with a NaN pattern before the kernels
run, so an element (padding included) that a kernel skipped cannot match.

Host memory: the 4-layer Llama-7B-shaped bucket keeps its eight oracle RS
inputs (8 x 3.24 GB) while its RS is checked; everything else is per rank.
Properties that hold at any size (the 16-bit and dim-1 variants) and items
beyond 4 GiB are checked at the end.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import bits, first_mismatch, note, np_bits, require_gpu, to_oracle

hp = pytest.importorskip("hsdp_parameter_gradient_amd")

pytestmark = pytest.mark.gpu

BIG = ["llama7b_4layer_r8_s8", "ragged_heavy_r8_s8"]
NAN_PATTERN = {torch.float32: (torch.int32, 0x7FA5A5A5), torch.bfloat16: (torch.int16, 0x7FA5),
               torch.float16: (torch.int16, 0x7FA5)}


def _poison(t: torch.Tensor) -> None:
    it, pat = NAN_PATTERN[t.dtype]
    t.view(it).fill_(pat)


def _same(t: torch.Tensor, want: np.ndarray, what: str) -> None:
    got = bits(t)
    exp = np_bits(want)
    assert got.shape == exp.shape and np.array_equal(got, exp), f"{what}: {first_mismatch(got, exp)}"


class FullSize:
    """One workload at full size on the GPU, its steps run once in the
    benchmark's configuration, and the host side of the oracle, computed on
    demand and kept for the checks that need it."""

    def __init__(self, wname: str):
        w = W.WORKLOADS[wname]
        self.w = w
        self.R, self.S, self.D = w.rank_size, w.shard_size, w.dp_size
        self.P = len(w.param_shapes)
        self.lay = O.bucket_layout(w.param_shapes, self.S)
        self.I = self.lay.I
        note(f"[fullsize] {w.name}: P={self.P} I={self.I} R={self.R} S={self.S}: drawing inputs, running the steps")
        self.params = W.params(w, device="cuda")
        self.grads = W.grads(w, device="cuda")
        self.flat_grads = [self.grads[g][i].reshape(-1) for g in range(self.R) for i in range(self.P)]
        fb = hp.FlatBucket(w.param_shapes, self.R, self.S, w.param_dtype, op=O.AVG)
        for t in [fb.ag, *fb.full, *fb.rs_in, *fb.fused]:
            _poison(t)
        fb.bind(fb.shard_views(self.params), self.flat_grads)
        for step in ("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"):
            fb.run(step)
        torch.cuda.synchronize()
        self.fb = fb
        self.host_params = [to_oracle(p) for p in self.params]
        self._ag = None
        self._rs_in = {}
        self._rs_out = {}

    def oracle_ag(self) -> np.ndarray:
        if self._ag is None:
            dt = np.float32 if self.w.param_dtype == torch.float32 else np.uint16
            self._ag = O.ag_copy_in(O.shard_params(self.host_params, self.lay), self.lay, dt)
        return self._ag

    def oracle_rs_in(self, g: int) -> np.ndarray:
        if g not in self._rs_in:
            host = [t.cpu().numpy() for t in self.grads[g]]
            self._rs_in[g] = O.rs_copy_in(host, self.lay)
        return self._rs_in[g]

    def oracle_rs_out(self, op: str):
        if op not in self._rs_out:
            rs_in = [self.oracle_rs_in(g) for g in range(self.R)]
            self._rs_out[op] = O.rs_reduce(rs_in, self.I, self.R, self.S, op)
        return self._rs_out[op]

    def release(self) -> None:
        self.fb = self.params = self.grads = self.flat_grads = None
        self._ag = None
        self._rs_in.clear()
        self._rs_out.clear()


@pytest.fixture(scope="module", params=BIG)
def big(request):
    require_gpu()
    hp.lib()
    st = FullSize(request.param)
    yield st
    st.release()
    hp.fsdp_release_cache()
    torch.cuda.empty_cache()


def test_ag_copy_in_every_element(big):
    note(f"[fullsize] {big.w.name}: ag_copy_in, {big.S * big.I} elements")
    _same(big.fb.ag, big.oracle_ag(), "ag_copy_in")


def test_ag_copy_out_every_element(big):
    note(f"[fullsize] {big.w.name}: ag_copy_out, {big.P} parameters")
    want = O.ag_copy_out(O.all_gather(big.oracle_ag()), big.lay)
    for i in range(big.P):
        _same(big.fb.full[i], want[i], f"ag_copy_out param {i}")
        # the round trip restores the parameter itself
        _same(big.fb.full[i], big.host_params[i], f"ag_copy_out param {i} vs the parameter")


@pytest.mark.parametrize("g", range(8))
def test_rs_copy_in_every_element(big, g):
    note(f"[fullsize] {big.w.name}: rs_copy_in rank {g}, {big.S * big.I} elements")
    _same(big.fb.rs_in[g], big.oracle_rs_in(g), f"rs_copy_in rank {g}")


def test_rs_reduce_avg_every_element(big):
    note(f"[fullsize] {big.w.name}: rs_reduce AVG, {big.R} x {big.I} elements")
    want = big.oracle_rs_out(O.AVG)
    for g in range(big.R):
        _same(big.fb.rs_out[g], want[g], f"rs_reduce AVG rank {g}")


def test_rs_reduce_sum_every_element(big):
    note(f"[fullsize] {big.w.name}: rs_reduce SUM, {big.R} x {big.I} elements")
    out = [torch.empty(big.I, dtype=torch.float32, device="cuda") for _ in range(big.R)]
    for t in out:
        _poison(t)
    hp.fsdp_rs_reduce(big.w.param_shapes, big.R, big.S, big.D, O.SUM, big.fb.rs_in, out)
    torch.cuda.synchronize()
    want = big.oracle_rs_out(O.SUM)
    for g in range(big.R):
        _same(out[g], want[g], f"rs_reduce SUM rank {g}")


@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_rs_copy_reduce_every_element(big, op):
    """RS copy-in fused into the RS: by the oracle's definition the RS of the
    RS inputs, so every element equals the oracle's RS output."""
    note(f"[fullsize] {big.w.name}: rs_copy_reduce {op}, {big.R} x {big.I} elements")
    out = [torch.empty(big.I, dtype=torch.float32, device="cuda") for _ in range(big.R)]
    for t in out:
        _poison(t)
    hp.fsdp_rs_copy_reduce(big.w.param_shapes, big.R, big.S, big.D, op, big.flat_grads, out)
    torch.cuda.synchronize()
    want = big.oracle_rs_out(op)
    for g in range(big.R):
        _same(out[g], want[g], f"rs_copy_reduce {op} rank {g}")


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
    require_gpu()
    hp.lib()
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
    hp.fsdp_release_cache()
    torch.cuda.empty_cache()


def test_items_beyond_4gib():
    """A copy segment and a reduction job each larger than 4 GiB (64-bit
    offsets everywhere): AG copy-in of one bf16 parameter of 2^31 + 1001
    elements with shard_size 1 (one 4 GiB + 2 KiB segment), and the fused
    AR of two replicas of 2^30 + 1000 fp32 elements (integer-valued, so the
    sum is exact)."""
    require_gpu()
    hp.lib()
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
    hp.fsdp_release_cache()
    torch.cuda.empty_cache()
