"""Element-at-a-time form of the oracle, for sampled checks at full size.

TEST INFRASTRUCTURE ONLY (same rule as fsdp_oracle: imported by the test
suite, the smoke check and the benchmark's CPU-baseline leg, never by the
product path).

Each function evaluates the definition in fsdp_oracle at a set of output
positions, reading only the input elements that those positions depend on,
through a caller-supplied fetch callback.  The layout it walks is the
oracle's own (fsdp_oracle.bucket_layout); nothing here comes from the HIP
path.  The positions are numpy int64 arrays; every step is a direct
consequence of the buffer definitions of the FSDP dim-0 non-uniform
sharding RFC (issue 319) section 6.4 and the PR #758 write-up of the Hyper
communication-overlap scheme (issue 184) section 2.1:

  rank slice s of an AG / RS buffer = [s*I, (s+1)*I);
  parameter i inside a slice = [in_off[i], in_off[i] + padded[i]);
  inside that region, row r of the shard sits at r*inner, and positions at
  or beyond row_len rows are padding (zero).
"""

from __future__ import annotations

from typing import Callable, Dict, List, Tuple

import numpy as np

from .fsdp_oracle import AVG, SUM, BucketLayout, group_sizes

# fetch(param_index, flat_element_indices) -> values (numpy array)
Fetch = Callable[[int, np.ndarray], np.ndarray]


def _locate(lay: BucketLayout, q: np.ndarray) -> np.ndarray:
    """Parameter index owning in-slice offset q (q < I)."""
    ends = np.cumsum(np.asarray(lay.padded, dtype=np.int64))
    # the first parameter whose region end is beyond q; empty regions
    # (padded == 0) share an end with their predecessor and are skipped.
    return np.searchsorted(ends, q, side="right")


def packed_sources(lay: BucketLayout, pos: np.ndarray):
    """For positions of a packed S*I buffer, the source each one reads.

    Returns (param, flat_index_in_full_param, is_data); padding positions
    have is_data False.
    """
    pos = np.asarray(pos, dtype=np.int64)
    s = pos // lay.I
    q = pos % lay.I
    i = _locate(lay, q)
    in_off = np.asarray(lay.in_off, dtype=np.int64)[i]
    inner = np.asarray(lay.inner, dtype=np.int64)[i]
    r = q - in_off
    row = r // np.maximum(inner, 1)
    col = r % np.maximum(inner, 1)
    row_len = np.asarray(lay.row_len, dtype=np.int64)[i, s]
    row_off = np.asarray(lay.row_off, dtype=np.int64)[i, s]
    is_data = row < row_len
    flat = (row_off + row) * inner + col
    return i, flat, is_data


def packed_values(lay: BucketLayout, pos: np.ndarray, fetch: Fetch, dtype) -> np.ndarray:
    """Expected AG copy-in (or one rank's RS copy-in) values at pos."""
    i, flat, is_data = packed_sources(lay, pos)
    out = np.zeros(pos.shape, dtype=dtype)
    for p in np.unique(i[is_data]):
        m = is_data & (i == p)
        out[m] = fetch(int(p), flat[m])
    return out


def unpacked_sources(lay: BucketLayout, i: int, flat: np.ndarray) -> np.ndarray:
    """Position in the gathered S*I buffer that element `flat` of full
    parameter i is copied from (AG copy-out)."""
    flat = np.asarray(flat, dtype=np.int64)
    inner = max(lay.inner[i], 1)
    row = flat // inner
    col = flat % inner
    chunk = lay.chunk_rows[i]
    s = row // chunk
    return s * lay.I + lay.in_off[i] + (row - s * chunk) * inner + col


def rs_reduce_values(lay_I: int, rank_size: int, shard_size: int, op: str, g: int,
                     k: np.ndarray, fetch_rs_in: Callable[[int, np.ndarray], np.ndarray]) -> np.ndarray:
    """Expected RS output of rank g at in-slice positions k.

    fetch_rs_in(m, positions) returns float32 values of rank m's RS input.
    The shard group of g = d*S + s is ranks d*S .. d*S+S-1; the sum runs in
    ascending rank order and AVG divides by S.
    """
    S, D = group_sizes(rank_size, shard_size)
    d, s = divmod(g, S)
    k = np.asarray(k, dtype=np.int64)
    acc = np.array(fetch_rs_in(d * S, s * lay_I + k), dtype=np.float32)
    for m in range(1, S):
        acc = acc + np.asarray(fetch_rs_in(d * S + m, s * lay_I + k), dtype=np.float32)
    if op == AVG:
        acc = acc / np.float32(S)
    elif op != SUM:
        raise ValueError(op)
    return acc


def fused_ar_values(rank_size: int, shard_size: int, op: str, g: int, k: np.ndarray,
                    fetch_fused: Callable[[int, np.ndarray], np.ndarray]) -> np.ndarray:
    """Expected fused-AR result of rank g at positions k.

    The replicate group of g = d*S + s is ranks s, S+s, ...; the sum runs in
    ascending rank order and AVG divides by D.
    """
    S, D = group_sizes(rank_size, shard_size)
    s = g % S
    k = np.asarray(k, dtype=np.int64)
    acc = np.array(fetch_fused(s, k), dtype=np.float32)
    for d in range(1, D):
        acc = acc + np.asarray(fetch_fused(d * S + s, k), dtype=np.float32)
    if op == AVG:
        acc = acc / np.float32(D)
    elif op != SUM:
        raise ValueError(op)
    return acc


def boundary_positions(lay: BucketLayout) -> np.ndarray:
    """In-slice offsets next to every region, data/padding and slice edge:
    the places where an offset or padding mistake shows first."""
    pts: List[int] = []
    for i in range(len(lay.shapes)):
        a = lay.in_off[i]
        for s in range(lay.S):
            n = lay.row_len[i][s] * lay.inner[i]
            for b in (a, a + n, a + lay.padded[i]):
                pts.extend((b - 2, b - 1, b, b + 1))
    pts = [p for p in pts if 0 <= p < lay.I]
    return np.unique(np.asarray(pts, dtype=np.int64))
