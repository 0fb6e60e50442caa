"""One FSDP/HSDP bucket on one GPU: its communication buffers and its steps.

FlatBucket owns (through torch, which supplies device memory) the buffers
of one bucket of parameters with all R simulated ranks resident in HBM:

  ag        [S*I]   AG buffer (parameter dtype); slice s is shard rank s's
                    send buffer
  full[i]           the full parameters written by AG copy-out
  rs_in[g]  [S*I]   rank g's padded RS input (gradient dtype: fp32, bf16 or fp16)
  fused[g]  [F]     rank g's 512-byte-aligned fused AR buffer; the RS output
                    of rank g is the view fused[g][off : off + I]
                    (zero-copy, PR #758 write-up of the Hyper
                    communication-overlap scheme, section 2.1); the
                    bucket's own fused_ar step reduces that segment and
                    its trailing gap (FusedGroup reduces the whole buffer
                    once for all its buckets)

and runs the hot path with one library call per step.  Which gradient
collectives run follows the decision matrix of the FullyShard
multi-dimensional RFC (sections 2.2.2 and 2.2.5): RS when shard_size > 1,
AR when dp_size > 1.  The shard views (AG inputs) and the per-rank full
gradients (RS copy-in inputs) belong to the caller.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import _binding as B


class FlatBucket:
    def __init__(self, shapes: Sequence[Sequence[int]], rank_size: int, shard_size: int,
                 param_dtype: torch.dtype = torch.bfloat16, op: str = B.AVG,
                 device: str = "cuda", fused_segments: Optional[Sequence[int]] = None,
                 fused_index: int = 0, grad_dtype: torch.dtype = torch.float32,
                 shard_dims: Optional[Sequence[int]] = None,
                 fused: Optional[Sequence[torch.Tensor]] = None):
        """fused_segments: sizes of the segments of the fused buffer (default:
        this bucket's RS output alone); fused_index: which one is this
        bucket's; grad_dtype: float32, bfloat16 or float16 (the reduce dtype);
        shard_dims: one shard dim per parameter (default 0); fused: the R
        fused buffers to write the RS output into, shared with other buckets
        (default: this bucket's own, zero-initialised)."""
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.R, self.S = int(rank_size), int(shard_size)
        rs, ar = B.fsdp_group_ranks(self.R, self.S)
        if not rs:
            raise ValueError("shard_size 1 has no AG / RS buffers (pure-TP compatible path): "
                             "call fsdp_fused_ar on the gradients' fused buffers")
        self.D = self.R // self.S
        self.do_rs, self.do_ar = bool(rs), bool(ar)
        self.op = op
        self.param_dtype = param_dtype
        self.grad_dtype = grad_dtype
        self.shard_dims = list(shard_dims) if shard_dims is not None else None
        self.layout = B.fsdp_bucket_layout(self.shapes, self.S, shard_dims=self.shard_dims)
        I = self.layout.I
        self.seg_numel = list(fused_segments) if fused_segments is not None else [I]
        offs, self.F = B.fsdp_fused_layout(self.seg_numel, grad_dtype.itemsize)
        self.fused_off = offs[fused_index]
        if self.seg_numel[fused_index] != I:
            raise ValueError("the bucket's fused segment must hold I elements")
        dev = torch.device(device)
        self.ag = torch.empty(self.S * I, dtype=param_dtype, device=dev)
        self.full = [torch.empty(s, dtype=param_dtype, device=dev) for s in self.shapes]
        self.rs_in = [torch.empty(self.S * I, dtype=grad_dtype, device=dev) for _ in range(self.R)]
        # fused buffers are fully defined (gaps zero) before the first RS writes
        # its views; torch's allocator returns 512-byte-aligned storage.
        if fused is None:
            self.fused = [torch.zeros(self.F, dtype=grad_dtype, device=dev) for _ in range(self.R)]
        else:
            self.fused = list(fused)
            if len(self.fused) != self.R or any(f.numel() != self.F or f.dtype != grad_dtype for f in self.fused):
                raise ValueError(f"fused: expected {self.R} buffers of {self.F} {grad_dtype} elements")
        self.rs_out = [f[self.fused_off:self.fused_off + I] for f in self.fused]
        # this bucket's own fused AR covers its segment and the zero gap up to
        # the next 512-byte boundary only: with buffers shared by several
        # buckets it never reduces another bucket's segment a second time, nor
        # touches memory that another bucket's RS writes meanwhile
        _, self.ar_numel = B.fsdp_fused_layout([I], grad_dtype.itemsize)
        self.ar_buffers = [f[self.fused_off:self.fused_off + self.ar_numel] for f in self.fused]
        self._calls = None

    # -- the caller's inputs ------------------------------------------------
    def shard_views(self, params: Sequence[torch.Tensor]) -> List[torch.Tensor]:
        """Rank-major shards [s*P + i] of full parameters: views of the rows
        (dim-0 chunk rule) for dim 0, dense copies of the chunks for a
        non-zero shard dim (a rank stores its chunk densely)."""
        out = []
        dims = self.shard_dims or [0] * len(self.shapes)
        for s in range(self.S):
            for i, x in enumerate(params):
                a, n = self.layout.row_off[i][s], self.layout.row_len[i][s]
                c = x.reshape(self.shapes[i]).narrow(dims[i], a, n)
                out.append(c.reshape(-1) if dims[i] == 0 else c.contiguous().reshape(-1))
        return out

    def full_views(self) -> List[torch.Tensor]:
        """Zero-copy AG for a one-parameter bucket: the parameter is the view
        ag[:N] of the gathered buffer, so copy-out can be skipped.  With
        fixed-size dim-0 chunks every padding element lies after the last
        data row, so that prefix is exactly the full parameter (the
        unsharded-parameter-as-view option of the Hyper PR #758 write-up,
        section 4; it needs the AG buffer to stay alive while the view is
        used)."""
        if len(self.shapes) != 1 or (self.shard_dims and self.shard_dims[0] != 0):
            raise ValueError("a view of the gathered buffer is the full parameter only for a "
                             "one-parameter bucket sharded on dim 0; use the ag_copy_out step")
        n = 1
        for d in self.shapes[0]:
            n *= d
        return [self.ag[:n].view(self.shapes[0])]

    def bind(self, shards: Sequence[torch.Tensor], grads: Sequence[torch.Tensor]) -> "FlatBucket":
        """Marshal the five calls once: shards [S*P] rank-major, grads [R*P]."""
        S, R, dims = self.S, self.R, self.shard_dims
        self._calls = {
            "ag_copy_in": B.prepare("fsdp_ag_copy_in", self.shapes, S, list(shards), self.ag, dims),
            "ag_copy_out": B.prepare("fsdp_ag_copy_out", self.shapes, S, self.ag, self.full, dims),
            "rs_copy_in": B.prepare("fsdp_rs_copy_in", self.shapes, R, S, list(grads), self.rs_in, dims),
            "rs_reduce": B.prepare("fsdp_rs_reduce", self.shapes, R, S, self.D, self.op, self.rs_in, self.rs_out,
                                   dims),
            "rs_copy_reduce": B.prepare("fsdp_rs_copy_reduce", self.shapes, R, S, self.D, self.op, list(grads),
                                        self.rs_out, dims),
            "fused_ar": B.prepare("fsdp_fused_ar", [self.layout.I], R, S, self.D, self.op, self.ar_buffers),
        }
        return self

    def steps(self, fused_rs: bool = False) -> List[str]:
        """The steps one pass runs, in order (forward AG, then backward).
        fused_rs: RS copy-in and RS as one pass (the RS input is never
        materialised; same results)."""
        st = ["ag_copy_in", "ag_copy_out"]
        st += ["rs_copy_reduce"] if fused_rs else ["rs_copy_in", "rs_reduce"]
        if self.do_ar:
            st.append("fused_ar")
        return st

    def _call(self, step: str):
        if self._calls is None:
            raise RuntimeError("FlatBucket: call bind(shards, grads) before running its steps")
        return self._calls[step]

    def run(self, step: str, stream=None) -> None:
        self._call(step)(stream)

    def step(self, stream=None, fused_rs: bool = False) -> None:
        for name in self.steps(fused_rs):
            self._call(name)(stream)


class FusedGroup:
    """Several buckets whose RS outputs share one fused buffer per rank and
    one fused AR (the AllReduceParamGroup of the PR #758 write-up of the
    Hyper communication-overlap scheme, section 2.1): bucket k's RS output
    is segment k, on a 512-byte boundary; the AR runs once over the whole
    buffer, gaps included.  Each bucket keeps its own AG and RS buffers."""

    def __init__(self, buckets: Sequence[Sequence[Sequence[int]]], rank_size: int, shard_size: int,
                 param_dtype: torch.dtype = torch.bfloat16, op: str = B.AVG, device: str = "cuda",
                 grad_dtype: torch.dtype = torch.float32,
                 shard_dims: Optional[Sequence[Optional[Sequence[int]]]] = None):
        """buckets: the parameter shapes of each bucket; shard_dims: per
        bucket, one shard dim per parameter (or None for dim 0)."""
        self.R, self.S = int(rank_size), int(shard_size)
        dims = list(shard_dims) if shard_dims is not None else [None] * len(buckets)
        if len(dims) != len(buckets):
            raise ValueError(f"shard_dims: {len(dims)} entries for {len(buckets)} buckets")
        seg = [B.fsdp_bucket_layout(b, self.S, shard_dims=d).I for b, d in zip(buckets, dims)]
        _, F = B.fsdp_fused_layout(seg, grad_dtype.itemsize)
        self.seg_numel = seg
        self.fused = [torch.zeros(F, dtype=grad_dtype, device=torch.device(device)) for _ in range(self.R)]
        self.buckets = [FlatBucket(b, rank_size, shard_size, param_dtype, op, device, seg, k, grad_dtype,
                                   shard_dims=dims[k], fused=self.fused) for k, b in enumerate(buckets)]
        self.op = op
        self.D = self.R // self.S
        self.do_ar = self.buckets[0].do_ar if self.buckets else False
        self._ar = None

    def bind(self, shards: Sequence[Sequence[torch.Tensor]], grads: Sequence[Sequence[torch.Tensor]]) -> "FusedGroup":
        """shards[k] and grads[k]: bucket k's inputs, as FlatBucket.bind."""
        if len(shards) != len(self.buckets) or len(grads) != len(self.buckets):
            raise ValueError(f"bind: {len(shards)} shard lists and {len(grads)} gradient lists "
                             f"for {len(self.buckets)} buckets")
        for fb, sh, gr in zip(self.buckets, shards, grads):
            fb.bind(sh, gr)
        self._ar = B.prepare("fsdp_fused_ar", self.seg_numel, self.R, self.S, self.D, self.op, self.fused)
        return self

    def step(self, stream=None, fused_rs: bool = False) -> None:
        """Every bucket's AG and RS, then the one fused AR."""
        if self._ar is None:
            raise RuntimeError("FusedGroup: call bind(shards, grads) before step()")
        for fb in self.buckets:
            for name in fb.steps(fused_rs):
                if name != "fused_ar":
                    fb.run(name, stream)
        if self.do_ar:
            self._ar(stream)

    def graph(self, n_streams: int = 3, fused_rs: bool = False) -> torch.cuda.CUDAGraph:
        """The step captured once into a HIP graph (replay() re-runs it), with
        the buckets' AG and RS spread round-robin over n_streams streams (the
        buckets are independent: their own buffers, disjoint fused segments)
        and the fused AR after all of them.  Each call is issued once eagerly
        first, so that the capture records kernel launches only.  Replayed,
        the short kernels of different buckets run side by side (measured on
        MI355X, the hidden-1024 HSDP block as 6 one-parameter buckets, R 8,
        S 4: 299 us per pass eager, 266-275 us replayed over 3 streams across
        runs)."""
        if self._ar is None:
            raise RuntimeError("FusedGroup: call bind(shards, grads) before graph()")
        if n_streams < 1:
            raise ValueError(f"n_streams {n_streams} < 1")
        streams = [torch.cuda.Stream(device=self.fused[0].device) for _ in range(n_streams)] if self.fused else []

        def run():
            cur = torch.cuda.current_stream()
            for st in streams:
                st.wait_stream(cur)
            for k, fb in enumerate(self.buckets):
                for name in fb.steps(fused_rs):
                    if name != "fused_ar":
                        fb.run(name, streams[k % n_streams])
            for st in streams:
                cur.wait_stream(st)
            if self.do_ar:
                self._ar(None)

        run()
        torch.cuda.current_stream().synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        g.streams = streams  # the capture's side streams live as long as the graph
        return g
