"""Helpers for the GPU parity tests (not collected by pytest).

Output buffers are carved out of larger allocations whose guard bands and
whose own contents are filled with a NaN bit pattern first: a kernel that
writes outside its buffer breaks a guard, and one that skips an element
(padding included) leaves the pattern behind, which no oracle value equals.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

GUARD = 1024  # elements on each side
_INT = {torch.float32: (torch.int32, np.int32, 0x7FA5A5A5),
        torch.bfloat16: (torch.int16, np.int16, 0x7FA5),
        torch.float16: (torch.int16, np.int16, 0x7FA5)}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; none is visible")


def note(msg: str) -> None:
    """Name the case on stdout before the GPU runs it."""
    print(msg, flush=True)
    sys.stdout.flush()


class Guarded:
    """A device buffer of `numel` elements at `offset` elements past a
    guard band, everything pre-filled with a NaN pattern."""

    def __init__(self, numel: int, dtype: torch.dtype, offset: int = 0, device: str = "cuda"):
        it, _, pat = _INT[dtype]
        self.G = GUARD + offset
        self.numel = numel
        self.base = torch.empty(numel + self.G + GUARD, dtype=dtype, device=device)
        self.base.view(it).fill_(pat)
        self.t = self.base[self.G:self.G + numel]
        self.dtype = dtype

    def guards_intact(self) -> bool:
        it, _, pat = _INT[self.dtype]
        b = self.base.view(it)
        return bool((b[:self.G] == pat).all()) and bool((b[self.G + self.numel:] == pat).all())


def bits(t: torch.Tensor) -> np.ndarray:
    """Bit pattern of a tensor (device or host) as a numpy integer array."""
    it, nt, _ = _INT[t.dtype]
    return t.detach().contiguous().view(it).cpu().numpy().reshape(-1)


def np_bits(a: np.ndarray) -> np.ndarray:
    """Bit pattern of an oracle array (float32 or the uint16 bits of a
    16-bit type) as the same integer type bits() returns."""
    a = np.ascontiguousarray(a).reshape(-1)
    if a.dtype == np.float32:
        return a.view(np.int32)
    if a.dtype in (np.uint16, np.float16):
        return a.view(np.int16)
    raise TypeError(a.dtype)


def to_oracle_values(t: torch.Tensor) -> np.ndarray:
    """Host numpy form of reduction operands: float32, bfloat16 as uint16
    bits (the oracle's bf16 form), float16 as numpy float16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float16:
        return t.numpy()
    return to_oracle(t)


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy form the oracle works on: float32, or uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def first_mismatch(got: np.ndarray, want: np.ndarray) -> str:
    if got.shape != want.shape:
        return f"shape {got.shape} != {want.shape}"
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    if bad.size == 0:
        return ""
    k = int(bad[0])
    return f"{bad.size} mismatches, first at {k}: got {got.reshape(-1)[k]:#x} want {want.reshape(-1)[k]:#x}"
