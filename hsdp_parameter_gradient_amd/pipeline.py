"""The backward RS/AR overlap across layers, on two HIP streams.

The PR #758 write-up of the Hyper communication-overlap scheme (section 2.2,
the 4-step backward pipeline) runs, at each layer's backward hook: wait for
the previous layer's shard-domain ReduceScatter, apply it, start this
layer's ReduceScatter asynchronously, then start the previous layer's fused
replicate-domain AllReduce; the root waits for the last AllReduce.  The two
domains are independent, so a layer's RS and the previous layer's AR run
concurrently.

BackwardPipeline issues exactly that order over FlatBuckets (one per layer,
visited in backward order): the RS of layer l (RS copy-in + RS, or the fused
RS copy-reduce) on the RS stream, and the fused AR of layer l-1 on the AR
stream after an event recorded behind that layer's RS.  run_serial() issues
the same kernels in the same order on one stream, for comparison; both give
identical results (every kernel reads and writes the same buffers, only the
overlap differs).  graph() captures either order once into a HIP graph.
All streams keep the default priority.
"""

from __future__ import annotations

from typing import List, Sequence

import torch

from .flat_bucket import FlatBucket


class BackwardPipeline:
    def __init__(self, buckets: Sequence[FlatBucket], fused_rs: bool = True):
        self.buckets: List[FlatBucket] = list(buckets)
        self.fused_rs = fused_rs
        self.rs_stream = torch.cuda.Stream()
        self.ar_stream = torch.cuda.Stream()
        self._rs_done = [torch.cuda.Event() for _ in self.buckets]

    def _rs(self, b: FlatBucket, stream) -> None:
        if self.fused_rs:
            b.run("rs_copy_reduce", stream)
        else:
            b.run("rs_copy_in", stream)
            b.run("rs_reduce", stream)

    def run_pipelined(self) -> None:
        """Issue the whole backward; the current stream waits for it."""
        cur = torch.cuda.current_stream()
        self.rs_stream.wait_stream(cur)  # gradients and buffers are ready
        self.ar_stream.wait_stream(cur)
        for l, b in enumerate(self.buckets):
            # step 3: this layer's RS, asynchronously on the shard-domain stream
            self._rs(b, self.rs_stream)
            self._rs_done[l].record(self.rs_stream)
            # steps 1 and 4: the previous layer's fused AR once its RS is done
            if l > 0:
                self._ar(l - 1)
        if self.buckets:
            self._ar(len(self.buckets) - 1)  # the root's final AR
        cur.wait_stream(self.rs_stream)
        cur.wait_stream(self.ar_stream)

    def _ar(self, l: int) -> None:
        b = self.buckets[l]
        if b.do_ar:
            self.ar_stream.wait_event(self._rs_done[l])
            b.run("fused_ar", self.ar_stream)

    def graph(self, pipelined: bool = True) -> torch.cuda.CUDAGraph:
        """The backward captured once into a HIP graph (replay() re-runs it):
        the two-stream order, or the serial one.  Every call is issued once
        eagerly first, so that the capture records kernel launches only.  A
        replay runs without the per-layer host work of the eager issue (the
        event records and cross-stream waits), which on one GPU is what lets
        the overlap pay."""
        run = self.run_pipelined if pipelined else self.run_serial
        run()
        torch.cuda.current_stream().synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        return g

    def run_serial(self) -> None:
        """The same kernels in the same order on the current stream."""
        for l, b in enumerate(self.buckets):
            self._rs(b, None)
            if l > 0 and self.buckets[l - 1].do_ar:
                self.buckets[l - 1].run("fused_ar", None)
        if self.buckets and self.buckets[-1].do_ar:
            self.buckets[-1].run("fused_ar", None)
