"""Seeded random bucket configurations (not collected by pytest).

One generator serves the CPU emulation of the planner's tables
(test_host_sanitizers.py) and the GPU parity run of the same cases
(test_gpu_random.py).  It only draws sizes, shard dims, group sizes, dtypes
and buffer offsets; it holds none of the layout or reduction arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

DTYPES = ("f32", "bf16", "f16")
ES = {"f32": 4, "bf16": 2, "f16": 2}
MAX_NUMEL = 1 << 18  # per parameter


@dataclass(frozen=True)
class Case:
    index: int
    S: int
    R: int
    shapes: Tuple[Tuple[int, ...], ...]
    dims: Tuple[int, ...]
    param_dtype: str
    grad_dtype: str
    misaligned: bool  # buffers at element offsets that are not 16-byte multiples
    extra_segments: Tuple[int, ...]  # fused-buffer segments after the bucket's RS output


def _dim(rng) -> int:
    return int(rng.choice([0, 1, 2, 3, 5, 7, 8, 13, 16, 31, 64, 100, 129, 257, 1000, 4097]))


def random_cases(seed: int, n: int) -> List[Case]:
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        S = int(rng.choice([1, 2, 3, 4, 5, 8]))
        D = int(rng.choice([1, 2, 3, 4]))
        P = int(rng.integers(1, 8))
        shapes, dims = [], []
        for _ in range(P):
            nd = int(rng.choice([1, 2, 3], p=[0.3, 0.5, 0.2]))
            shape = [_dim(rng) for _ in range(nd)]
            k = 0
            if nd > 1 and rng.random() < 0.4:
                k = int(rng.integers(1, nd))
                shape[k] = S * int(rng.choice([0, 1, 2, 3, 8, 16, 64, 256]))
            numel = int(np.prod(shape))
            if numel > MAX_NUMEL:  # keep the oracle fast: shrink the first dim
                shape[0 if k != 0 else -1] = max(0, shape[0 if k != 0 else -1] * MAX_NUMEL // max(numel, 1))
            shapes.append(tuple(int(v) for v in shape))
            dims.append(k)
        if any(k != 0 and s[k] % S for s, k in zip(shapes, dims)):
            continue
        extra = tuple(int(v) for v in rng.choice([0, 1, 3, 100, 513, 4096], size=int(rng.integers(0, 3))))
        out.append(Case(len(out), S, S * D, tuple(shapes), tuple(dims), str(rng.choice(DTYPES)),
                        str(rng.choice(DTYPES)), bool(rng.random() < 0.6), extra))
    return out


def case_line(c: Case) -> str:
    """One line of the sanitizer driver's case file: S R es misaligned P,
    then per parameter ndim, its dims and its shard dim."""
    es = ES[c.grad_dtype]
    parts = [c.S, c.R, es, int(c.misaligned), len(c.shapes)]
    for s, k in zip(c.shapes, c.dims):
        parts += [len(s), *s, k]
    return " ".join(str(v) for v in parts)
