"""Seeded synthetic workloads (shapes, sizes and value distributions).

This module only draws inputs.  It holds none of the sharding arithmetic:
no chunking, offsets, padding, reductions or fused-buffer layout.  Both
sides of every check (the oracle and the HIP path) receive the tensors it
draws.

Recipe: tensor number k of workload number n is drawn by a torch.Generator
on the target device seeded with n * 1000003 + k.  Parameters are tensors
0 .. P-1 in bucket order; the gradient of parameter i on simulated rank g is
tensor P + g * P + i.  uniform[-1, 1] is 2 * rand - 1; N(0, sigma) is
sigma * randn; bfloat16 tensors are drawn in float32 and rounded to nearest
even.  torch's CPU and GPU generators give different streams for the same
seed, so a check draws on one device and copies to the other.

The five workloads are the stand-ins for the transformer-shaped parameter
sets these pages talk about (a Qwen3 block for HSDP, Llama-7B-shaped
layers): synthetic shapes and distributions, no weights or datasets.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

Shape = Tuple[int, ...]


@dataclass(frozen=True)
class Workload:
    name: str
    number: int                      # seed base (workload number)
    rank_size: int
    shard_size: int
    param_shapes: Tuple[Shape, ...]
    param_dtype: torch.dtype
    param_dist: Tuple[str, float]    # ("uniform", 1.0) or ("normal", sigma)
    grad_dist: Tuple[str, float]
    reduce_ops: Tuple[str, ...]      # reduce ops the workload is run with
    ops: Tuple[str, ...]             # hot-path steps the workload exercises
    description: str = ""

    @property
    def dp_size(self) -> int:
        return self.rank_size // self.shard_size


def _llama_layers(n_layers: int, hidden: int, ffn: int) -> Tuple[Shape, ...]:
    shapes: List[Shape] = []
    for _ in range(n_layers):
        shapes += [(hidden, hidden)] * 4          # q, k, v, o (32 heads x 128)
        shapes += [(ffn, hidden), (ffn, hidden)]  # gate, up
        shapes += [(hidden, ffn)]                 # down
        shapes += [(hidden,), (hidden,)]          # attention norm, mlp norm
    return tuple(shapes)


def log_uniform_sizes(count: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    """Sizes log-uniform on [lo, hi]: rint(exp(U[ln lo, ln hi])), clipped."""
    u = np.random.default_rng(seed).random(count)
    n = np.rint(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return tuple(int(v) for v in np.clip(n, lo, hi))


ALL_STEPS = ("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce", "fused_ar")

TINY_FSDP = Workload(
    name="tiny_fsdp_r4_s4", number=1, rank_size=4, shard_size=4,
    param_shapes=((7, 8), (5, 3), (16,)), param_dtype=torch.float32,
    param_dist=("uniform", 1.0), grad_dist=("uniform", 1.0),
    reduce_ops=("sum", "avg"), ops=("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"),
    description="three fp32 params (7,8), (5,3), (16,); ragged dim 0 and a zero-length shard")

HSDP_BLOCK = Workload(
    name="hsdp_block_h1024_r8_s4_d2", number=2, rank_size=8, shard_size=4,
    param_shapes=((3072, 1024), (1024, 1024), (4096, 1024), (1024, 4096), (1024,), (1024,)),
    param_dtype=torch.bfloat16, param_dist=("normal", 0.02), grad_dist=("normal", 1e-3),
    reduce_ops=("avg",), ops=ALL_STEPS,
    description="one transformer block, hidden 1024: qkv, o, up, down, two norms; HSDP 8 = 2 x 4")

LLAMA7B_4L = Workload(
    name="llama7b_4layer_r8_s8", number=3, rank_size=8, shard_size=8,
    param_shapes=_llama_layers(4, 4096, 11008), param_dtype=torch.bfloat16,
    param_dist=("normal", 0.02), grad_dist=("normal", 1e-3),
    reduce_ops=("sum", "avg"), ops=("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"),
    description="4 Llama-7B-shaped layers (hidden 4096, ffn 11008, 32 heads): 36 params, 809.5M elements")

RAGGED_HEAVY = Workload(
    name="ragged_heavy_r8_s8", number=4, rank_size=8, shard_size=8,
    param_shapes=((4097, 4096), (11009, 4096), (32001, 4096), (5, 64), (3,)),
    param_dtype=torch.float32, param_dist=("uniform", 1.0), grad_dist=("uniform", 1.0),
    reduce_ops=("sum", "avg"), ops=("ag_copy_in", "ag_copy_out", "rs_copy_in", "rs_reduce"),
    description="fp32 dim-0 4097 / 11009 / 32001 (x4096) plus (5,64) and (3,)")

PURE_TP = Workload(
    name="pure_tp_2000grads_r8_s1_d8", number=5, rank_size=8, shard_size=1,
    param_shapes=tuple((n,) for n in log_uniform_sizes(2000, 1, 65536, seed=5)),
    param_dtype=torch.float32, param_dist=("normal", 1.0), grad_dist=("normal", 1.0),
    reduce_ops=("avg",), ops=("fused_ar",),
    description="2000 fp32 grads, log-uniform 1..65536 elements, one 512B-aligned segment each")

WORKLOADS = {w.name: w for w in (TINY_FSDP, HSDP_BLOCK, LLAMA7B_4L, RAGGED_HEAVY, PURE_TP)}


def scaled(w: Workload, shapes: Sequence[Shape], name: Optional[str] = None) -> Workload:
    """The same workload (ranks, dtypes, distributions, seed) on other shapes."""
    return replace(w, param_shapes=tuple(tuple(s) for s in shapes), name=name or (w.name + "_scaled"))


def _numel(shape: Shape) -> int:
    n = 1
    for d in shape:
        n *= d
    return n


def _draw(shape: Shape, dist: Tuple[str, float], dtype: torch.dtype,
          gen: torch.Generator, device) -> torch.Tensor:
    kind, scale = dist
    if kind == "uniform":
        t = torch.rand(shape, generator=gen, device=device, dtype=torch.float32).mul_(2 * scale).sub_(scale)
    elif kind == "normal":
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).mul_(scale)
    else:
        raise ValueError(kind)
    return t if dtype == torch.float32 else t.to(dtype)


def _gen(w: Workload, k: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.number * 1000003 + k)
    return g


def params(w: Workload, device="cpu") -> List[torch.Tensor]:
    """The bucket's full parameters (tensors 0 .. P-1)."""
    return [_draw(sh, w.param_dist, w.param_dtype, _gen(w, k, device), device)
            for k, sh in enumerate(w.param_shapes)]


def grads(w: Workload, device="cpu", ranks: Optional[Sequence[int]] = None,
          dtype: torch.dtype = torch.float32) -> List[List[torch.Tensor]]:
    """grads[g][i]: full gradient of parameter i on simulated rank g."""
    P = len(w.param_shapes)
    ranks = range(w.rank_size) if ranks is None else ranks
    return [[_draw(sh, w.grad_dist, dtype, _gen(w, P + g * P + i, device), device)
             for i, sh in enumerate(w.param_shapes)] for g in ranks]


def integer_grads(w: Workload, lo: int = -8, hi: int = 8, device="cpu") -> List[List[torch.Tensor]]:
    """Integer-valued float32 gradients in [lo, hi]: every sum of a few of
    them is exact in float32, whatever the order."""
    P = len(w.param_shapes)
    return [[torch.randint(lo, hi + 1, sh, generator=_gen(w, P + g * P + i, device),
                           device=device).to(torch.float32)
             for i, sh in enumerate(w.param_shapes)] for g in range(w.rank_size)]


def element_count(w: Workload) -> int:
    return sum(_numel(s) for s in w.param_shapes)
