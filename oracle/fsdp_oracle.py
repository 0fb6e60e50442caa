"""Plain CPU oracle for FSDP/HSDP flat-buffer sharding.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check of the package entry point and the CPU-baseline leg of the
benchmark may import it; the product path never does, and this module imports
nothing from the product package.

Sources (the pages, cited by title and section):
  [FS-MD]  "FullyShard multi-dimensional parallel adaptation" RFC
           (gitcode yide12/hyper-parallel issue 1): 2.2.1 GroupInfo two-group
           model, 2.2.2 backward communication decision matrix, 2.2.5
           rank_size / shard_size / dp_size, 3.3 pseudocode.
  [HYPER]  "Hyper communication-overlap scheme" and the PR #758 write-up
           (gitcode mindspore/hyper-parallel issue 184): section 2.1 fused
           communication packing (AG pack into the rank slice, copy-out,
           RS copy-in, AllReduceParamGroup with a 512-byte-aligned fused
           buffer), section 2.3 gradient scaling (SUM / AVG, fused AR as SUM
           followed by division by the replicate world size), section 3
           (fused vs non-fused bit-identical results), section 4.1 (send
           buffer = this rank's slice of the AG output).
  [RAGGED] FSDP dim-0 non-uniform sharding RFC (gitcode mindspore/
           hyper-parallel issue 319): 5.2 usage example (7, 8) on 4 ranks,
           6.4 key logic (chunk formula, sharded_size vs
           padded_sharded_param_size, padded communication storage, AG / RS
           padding rules), 9.1 unit-test boundary list.

Readings where the pages are silent:
  * rank g = d * S + s (mesh order (replicate, shard));
  * reductions add the group's operands one at a time in ascending rank
    order, the accumulator starting from the first operand;
  * AVG divides the finished sum by the group's own size, in the gradient
    dtype (float32), correctly rounded;
  * parameters inside a bucket follow the given order, with no alignment
    between them: offsets advance by the padded element count only;
  * the fused buffer places each segment on a 512-byte boundary and rounds
    its total size up to 512 bytes; the gaps are zero.

Precision: copies move elements bit for bit (bfloat16 is carried as its
uint16 bit pattern).  Reductions run in float32 because the pages reduce the
float32 gradients in their own dtype; the test suite checks them against a
float64 sum within the float32 rounding bound.  bfloat16 or float16
gradients (a 16-bit reduce dtype) are widened exactly, summed in float32 in
the same order, scaled, and rounded once to nearest even.

Pins: every function here is pinned by tests that do not re-state its
formula (worked examples, torch.chunk, brute-force inverse maps, exact
integer sums, float64 bounds, group lists).  The bit pattern of a non-exact
float32 sum depends on the summation order: the reductions use the fixed
rank order, ascending within each group and starting from the first operand
(the pages leave the order open; the ascending fold is the reading taken
here), and a test pins every output bit of them to NumPy's float32
add.accumulate over the group's operands in that order.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

SUM = "sum"
AVG = "avg"
FUSED_ALIGN_BYTES = 512


# ---------------------------------------------------------------------------
# Layout  ([RAGGED] 6.4; [FS-MD] 2.2.5; [HYPER] 2.1)
# ---------------------------------------------------------------------------

def group_sizes(rank_size: int, shard_size: int) -> Tuple[int, int]:
    """Return (shard_size, dp_size) with dp_size = rank_size // shard_size.

    [FS-MD] 2.2.5: the replicate group size is the integer quotient of the
    data-parallel domain size by the shard group size.  A rank count that
    the shard size does not divide has no (replicate, shard) mesh, so it is
    rejected.
    """
    if shard_size < 1 or rank_size < 1:
        raise ValueError("rank_size and shard_size must be >= 1")
    if rank_size % shard_size != 0:
        raise ValueError("rank_size must be a multiple of shard_size")
    return shard_size, rank_size // shard_size


def dim0_chunk(n0: int, shard_size: int) -> Tuple[int, List[int], List[int]]:
    """Fixed-size dim-0 chunking of one parameter ([RAGGED] 6.4).

    The chunk length is the ceiling of dim-0 over the shard count; rank s
    starts at s chunks, clamped to the end of dim 0, and holds at most one
    chunk, clamped the same way.  Trailing ranks may hold zero rows.
    Returns (chunk_rows, row_offset[s], row_length[s]).
    """
    if n0 < 0:
        raise ValueError("negative dim-0")
    S = shard_size
    chunk = (n0 + S - 1) // S
    offsets, lengths = [], []
    for s in range(S):
        start = min(s * chunk, n0)
        offsets.append(start)
        lengths.append(min(chunk, n0 - start))
    return chunk, offsets, lengths


@dataclass
class BucketLayout:
    """Per-bucket layout of the AG / RS communication buffers.

    shapes        logical parameter shapes, bucket order
    S             shard group size
    shard_dims[i] the dim parameter i is sharded on
    outer[i]      product of the dims before the shard dim (1 for dim 0)
    chunk_rows[i] padded length of the shard dim per rank (for dim 0 the
                  padded_sharded_param_size dim 0 of [RAGGED] 6.4)
    inner[i]      product of the dims after the shard dim
    padded[i]     outer[i] * chunk_rows[i] * inner[i], elements per rank slice
    in_off[i]     offset of parameter i inside one rank slice; advances by
                  padded elements only ([RAGGED] 6.4, fused RS copy-in)
    I             elements per rank slice (sum of padded)
    row_off[i][s], row_len[i][s]   the actual shard rows of rank s
    """

    shapes: List[Tuple[int, ...]]
    S: int
    shard_dims: List[int] = field(default_factory=list)
    outer: List[int] = field(default_factory=list)
    chunk_rows: List[int] = field(default_factory=list)
    inner: List[int] = field(default_factory=list)
    padded: List[int] = field(default_factory=list)
    in_off: List[int] = field(default_factory=list)
    I: int = 0
    row_off: List[List[int]] = field(default_factory=list)
    row_len: List[List[int]] = field(default_factory=list)


def bucket_layout(shapes: Sequence[Sequence[int]], shard_size: int,
                  shard_dim: int = 0, shard_dims: Sequence[int] = None) -> BucketLayout:
    """Layout of a bucket of parameters, each sharded on its shard dim.

    Dim 0 may be non-uniform ([RAGGED] 6.4, fixed-size chunks, zero padding
    at the tail).  Any other dim must divide evenly ([RAGGED] 3.2 keeps it on
    the plain chunk/concatenate path, and the interface table of 5.1 raises
    NotImplementedError for an uneven non-zero dim): no padding, rank s holds
    the s-th of S equal chunks along that dim.  shard_dims gives one dim per
    parameter (default: shard_dim for all); a 0-d parameter has no dim to
    shard and is rejected.
    """
    if shard_size < 1:
        raise ValueError("shard_size must be >= 1")
    S = shard_size
    shapes = [tuple(int(d) for d in sh) for sh in shapes]
    dims = [shard_dim] * len(shapes) if shard_dims is None else [int(k) for k in shard_dims]
    if len(dims) != len(shapes):
        raise ValueError("one shard dim per parameter")
    lay = BucketLayout(shapes=shapes, S=S)
    offset = 0
    for shape, k in zip(lay.shapes, dims):
        if len(shape) < 1:
            raise ValueError("a parameter needs at least one dimension")
        if any(d < 0 for d in shape):
            raise ValueError("negative dimension")
        if not 0 <= k < len(shape):
            raise ValueError("shard dim out of range")
        outer = 1
        for d in shape[:k]:
            outer *= d
        inner = 1
        for d in shape[k + 1:]:
            inner *= d
        if k == 0:
            chunk, offs, lens = dim0_chunk(shape[0], S)
        else:
            if shape[k] % S:
                raise NotImplementedError("a non-zero shard dim must divide evenly by the shard size")
            chunk = shape[k] // S
            offs, lens = [s * chunk for s in range(S)], [chunk] * S
        lay.shard_dims.append(k)
        lay.outer.append(outer)
        lay.chunk_rows.append(chunk)
        lay.inner.append(inner)
        lay.padded.append(outer * chunk * inner)
        lay.in_off.append(offset)
        lay.row_off.append(offs)
        lay.row_len.append(lens)
        offset += outer * chunk * inner
    lay.I = offset
    return lay


def _shard_shape(lay: BucketLayout, i: int, s: int) -> Tuple[int, ...]:
    shape = list(lay.shapes[i])
    shape[lay.shard_dims[i]] = lay.row_len[i][s]
    return tuple(shape)


def _chunk(x: np.ndarray, lay: BucketLayout, i: int, s: int) -> np.ndarray:
    """Rank s's chunk of a full parameter or gradient of parameter i."""
    k = lay.shard_dims[i]
    a, n = lay.row_off[i][s], lay.row_len[i][s]
    idx = [slice(None)] * x.ndim
    idx[k] = slice(a, a + n)
    return x[tuple(idx)]


def fused_layout(seg_numel: Sequence[int], elem_bytes: int = 4,
                 align_bytes: int = FUSED_ALIGN_BYTES) -> Tuple[List[int], int]:
    """Offsets (in elements) of segments in the fused AR buffer and its size.

    [HYPER] 2.1 (AllReduceParamGroup): one contiguous buffer, aligned to 512
    bytes, receives the RS outputs as views.  Reading: every segment starts
    on a 512-byte boundary and the total is rounded up to 512 bytes.
    """
    offsets = []
    end_bytes = 0
    for n in seg_numel:
        if n < 0:
            raise ValueError("negative segment")
        start = -(-end_bytes // align_bytes) * align_bytes
        if start % elem_bytes:
            raise ValueError("alignment is not a multiple of the element size")
        offsets.append(start // elem_bytes)
        end_bytes = start + n * elem_bytes
    total = -(-end_bytes // align_bytes) * align_bytes
    return offsets, total // elem_bytes


# ---------------------------------------------------------------------------
# Forward: shard, AG copy-in, gather, AG copy-out  ([RAGGED] 6.4; [HYPER] 2.1)
# ---------------------------------------------------------------------------

def shard_params(params: Sequence[np.ndarray], lay: BucketLayout) -> List[List[np.ndarray]]:
    """shards[s][i]: rank s's chunk of parameter i along its shard dim
    (rows [row_off, row_off + row_len) for dim 0), stored contiguously.

    [RAGGED] 6.4: the sharded parameter is the actual local rows, possibly
    zero rows; padding is not part of it.
    """
    out = []
    for s in range(lay.S):
        out.append([np.ascontiguousarray(_chunk(x, lay, i, s)) for i, x in enumerate(params)])
    return out


def ag_copy_in(shards: Sequence[Sequence[np.ndarray]], lay: BucketLayout,
               dtype) -> np.ndarray:
    """Pack every rank's shards into its slice of the AG buffer.

    [HYPER] 2.1 and 4.1: each rank's send buffer is its own slice
    [s*I, (s+1)*I) of the AG output; [RAGGED] 6.4: each parameter occupies
    its padded region, the actual shard at the front and zeros after it.
    All S simulated ranks are packed, so the gather that follows is the
    identity.
    """
    ag = np.zeros(lay.S * lay.I, dtype=dtype)
    for s in range(lay.S):
        for i in range(len(lay.shapes)):
            flat = np.ascontiguousarray(shards[s][i]).reshape(-1)
            base = s * lay.I + lay.in_off[i]
            ag[base:base + flat.size] = flat
    return ag


def all_gather(ag: np.ndarray) -> np.ndarray:
    """The AllGather over one shard group.

    With all S slices already resident in one buffer the exchange is the
    identity ([RAGGED] 6.3 sequence: the collective returns the padded full
    buffer).  Replicate groups hold identical copies, so one is simulated.
    """
    return ag


def ag_copy_out(ag: np.ndarray, lay: BucketLayout) -> List[np.ndarray]:
    """Split the gathered buffer into the full parameters.

    [HYPER] 2.1 (copy-out of the fused AG output into per-parameter outputs)
    and [RAGGED] 6.4 (only the logical shape is exposed; padding never
    enters the module): parameter i is the concatenation over ranks of the
    actual-row prefixes of its padded regions.
    """
    out = []
    for i, shape in enumerate(lay.shapes):
        pieces = []
        for s in range(lay.S):
            base = s * lay.I + lay.in_off[i]
            n = lay.outer[i] * lay.row_len[i][s] * lay.inner[i]
            pieces.append(ag[base:base + n].reshape(_shard_shape(lay, i, s)))
        out.append(np.concatenate(pieces, axis=lay.shard_dims[i]).reshape(shape))
    return out


# ---------------------------------------------------------------------------
# Backward: RS copy-in, RS reduce, fused AR  ([RAGGED] 6.4; [FS-MD] 2.2;
# [HYPER] 2.1, 2.3)
# ---------------------------------------------------------------------------

def rs_copy_in(grads: Sequence[np.ndarray], lay: BucketLayout, dtype=np.float32) -> np.ndarray:
    """One rank's RS input: every gradient chunked along its shard dim and
    zero padded.

    [RAGGED] 6.4: the RS input of a non-uniform gradient is padded at the
    tail with zeros; with fused communication each gradient goes straight
    into its region and offsets advance by the padded element count.
    Slice s of the buffer holds chunk s of every gradient.
    """
    buf = np.zeros(lay.S * lay.I, dtype=dtype)
    for i in range(len(lay.shapes)):
        g = np.ascontiguousarray(grads[i]).reshape(lay.shapes[i])
        for s in range(lay.S):
            flat = np.ascontiguousarray(_chunk(g, lay, i, s)).reshape(-1)
            base = s * lay.I + lay.in_off[i]
            buf[base:base + flat.size] = flat
    return buf


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float32: the bf16 bits are the top
    half of the float32 bits, so the conversion is exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 to bfloat16 bits, round to nearest, ties to even; every NaN
    becomes the quiet NaN 0x7FC0.  Written out on the bit pattern: keep the
    top 16 bits, add one unit when the dropped 16 bits exceed half a unit, or
    equal it and the kept part is odd (carries may round up to infinity)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    top = u >> 16
    low = u & 0xFFFF
    up = (low > 0x8000) | ((low == 0x8000) & ((top & 1) == 1))
    out = (top + up).astype(np.uint16)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    out[nan] = 0x7FC0
    return out


def _as_f32(x: np.ndarray) -> np.ndarray:
    """Gradient values in float32, exactly (bfloat16 is carried as uint16
    bits; float16 widens exactly)."""
    return bf16_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32, copy=False)


def _ordered_sum(operands: Sequence[np.ndarray]) -> np.ndarray:
    """Sum operands one at a time in the given order (reading R2), in
    float32 (bfloat16 operands are widened exactly first)."""
    acc = np.array(_as_f32(operands[0]), dtype=np.float32, copy=True)
    for x in operands[1:]:
        acc = acc + _as_f32(x)
    return acc


def _scale(acc: np.ndarray, op: str, n: int) -> np.ndarray:
    """Apply the reduce op's scaling ([HYPER] 2.3): AVG divides by n."""
    if op == SUM:
        return acc
    if op == AVG:
        return acc / np.float32(n)
    raise ValueError("unknown reduce op")


def _store(acc: np.ndarray, like: np.ndarray) -> np.ndarray:
    """The reduced value in the gradients' dtype: float32 as is, bfloat16 or
    float16 rounded once, to nearest even (the reduce dtype of [FS-MD] 5.2;
    float16 by NumPy's IEEE conversion: ties to even, overflow to infinity,
    denormals kept)."""
    if like.dtype == np.uint16:
        return f32_to_bf16(acc)
    if like.dtype == np.float16:
        return acc.astype(np.float16)
    return acc


def shard_groups(rank_size: int, shard_size: int) -> List[List[int]]:
    """Shard groups (the RS groups of [FS-MD] 2.2.1), rank g = d*S + s."""
    S, D = group_sizes(rank_size, shard_size)
    return [[d * S + s for s in range(S)] for d in range(D)]


def replicate_groups(rank_size: int, shard_size: int) -> List[List[int]]:
    """Replicate groups (the AR groups of [FS-MD] 2.2.1), rank g = d*S + s."""
    S, D = group_sizes(rank_size, shard_size)
    return [[d * S + s for d in range(D)] for s in range(S)]


def rs_reduce(rs_in: Sequence[np.ndarray], I: int, rank_size: int, shard_size: int,
              op: str) -> List[np.ndarray]:
    """ReduceScatter within every shard group.

    [FS-MD] 2.2.1 / 3.3: the shard group reduces, and rank s of the group
    keeps slice s.  Output of rank g = d*S + s is slice s summed over the
    group's ranks in ascending order; AVG then divides by S.
    """
    S, D = group_sizes(rank_size, shard_size)
    out: List[np.ndarray] = [None] * rank_size  # type: ignore[list-item]
    for group in shard_groups(rank_size, shard_size):
        for s, g in enumerate(group):
            operands = [rs_in[m][s * I:(s + 1) * I] for m in group]
            out[g] = _store(_scale(_ordered_sum(operands), op, S), rs_in[group[0]])
    return out


def fused_ar(fused: Sequence[np.ndarray], rank_size: int, shard_size: int,
             op: str) -> List[np.ndarray]:
    """AllReduce of the fused buffers within every replicate group.

    [HYPER] 2.1 / 2.3: one all-reduce over the contiguous fused buffer, done
    as SUM and then divided by the replicate world size for AVG; every
    replica receives the result.
    """
    S, D = group_sizes(rank_size, shard_size)
    out: List[np.ndarray] = [None] * rank_size  # type: ignore[list-item]
    for group in replicate_groups(rank_size, shard_size):
        acc = _store(_scale(_ordered_sum([fused[m] for m in group]), op, D), fused[group[0]])
        for m in group:
            out[m] = acc.copy()
    return out


def rs_copy_reduce(grads: Sequence[Sequence[np.ndarray]], lay: BucketLayout, rank_size: int,
                   op: str) -> List[np.ndarray]:
    """RS copy-in and RS as one step: by definition the RS of the RS inputs
    (the fused form only skips materialising them)."""
    first = grads[0][0].dtype if rank_size > 0 and len(lay.shapes) > 0 else np.dtype(np.float32)
    dtype = first if first in (np.uint16, np.float16) else np.float32
    rs_in = [rs_copy_in(grads[g], lay, dtype) for g in range(rank_size)]
    return rs_reduce(rs_in, lay.I, rank_size, lay.S, op)


def grad_sync_plan(rank_size: int, shard_size: int) -> List[Tuple[str, List[List[int]]]]:
    """Backward communication decision matrix ([FS-MD] 2.2.2, 2.2.5, 3.3).

    RS on the shard groups when shard_size > 1; AR on the replicate groups
    when dp_size > 1 (with shard_size == 1 this is the pure-TP compatible
    path: AR only); no communication when both are 1.
    """
    S, D = group_sizes(rank_size, shard_size)
    calls = []
    if S > 1:
        calls.append(("RS", shard_groups(rank_size, shard_size)))
    if D > 1:
        calls.append(("AR", replicate_groups(rank_size, shard_size)))
    return calls


def sharded_grad(rs_out_g: np.ndarray, lay: BucketLayout, i: int, s: int) -> np.ndarray:
    """Gradient handed to the optimizer for parameter i on shard rank s.

    [RAGGED] 6.4: only the sharded_size rows are written back; the padded
    tail of the RS output region is dropped.
    """
    n = lay.outer[i] * lay.row_len[i][s] * lay.inner[i]
    a = lay.in_off[i]
    return rs_out_g[a:a + n].reshape(_shard_shape(lay, i, s))


# ---------------------------------------------------------------------------
# End-to-end gradient synchronisation, fused and non-fused
# ---------------------------------------------------------------------------

def reduce_grads_fused(grads: Sequence[Sequence[np.ndarray]],
                       buckets: Sequence[Sequence[Sequence[int]]],
                       rank_size: int, shard_size: int, op: str):
    """Fused path: per bucket RS copy-in and RS, outputs placed as segments
    of the 512-byte-aligned fused buffer, then one AR over that buffer.

    grads[g][j] is rank g's gradient j; buckets lists, per bucket, the
    shapes of its gradients (the gradients are taken in bucket order).
    With shard_size == 1 there is no RS and every gradient is its own
    segment (pure-TP compatible path).  Returns (sharded grads[g][j], fused
    buffers, fused offsets, layouts).
    """
    S, D = group_sizes(rank_size, shard_size)
    layouts = [bucket_layout(b, S) for b in buckets]
    segs: List[List[np.ndarray]] = [[] for _ in range(rank_size)]
    seg_numel: List[int] = []
    j0 = 0
    for lay in layouts:
        P = len(lay.shapes)
        if S > 1:
            rs_in = [rs_copy_in(grads[g][j0:j0 + P], lay) for g in range(rank_size)]
            outs = rs_reduce(rs_in, lay.I, rank_size, S, op)
            for g in range(rank_size):
                segs[g].append(outs[g])
            seg_numel.append(lay.I)
        else:
            for j in range(P):
                for g in range(rank_size):
                    segs[g].append(np.ascontiguousarray(grads[g][j0 + j], np.float32).reshape(-1))
                seg_numel.append(lay.padded[j])
        j0 += P
    offs, F = fused_layout(seg_numel)
    fused = []
    for g in range(rank_size):
        buf = np.zeros(F, np.float32)
        for o, seg in zip(offs, segs[g]):
            buf[o:o + seg.size] = seg
        fused.append(buf)
    if D > 1:
        fused = fused_ar(fused, rank_size, S, op)
    result: List[List[np.ndarray]] = [[] for _ in range(rank_size)]
    j0 = 0
    k = 0
    for lay in layouts:
        P = len(lay.shapes)
        for g in range(rank_size):
            s = g % S
            if S > 1:
                region = fused[g][offs[k]:offs[k] + lay.I]
                for i in range(P):
                    result[g].append(sharded_grad(region, lay, i, s))
            else:
                for i in range(P):
                    o = offs[k + i]
                    result[g].append(fused[g][o:o + lay.padded[i]].reshape(lay.shapes[i]))
        k += 1 if S > 1 else P
        j0 += P
    return result, fused, offs, layouts


def reduce_grads_nonfused(grads: Sequence[Sequence[np.ndarray]],
                          shapes: Sequence[Sequence[int]],
                          rank_size: int, shard_size: int, op: str):
    """Non-fused path: every gradient gets its own RS and its own AR.

    [HYPER] 2.3 / 3: the non-fused HSDP path scales the replicate-dim
    all-reduce by the replicate world size, and its results equal the fused
    path's bit for bit.
    """
    S, D = group_sizes(rank_size, shard_size)
    result: List[List[np.ndarray]] = [[] for _ in range(rank_size)]
    for j, shape in enumerate(shapes):
        lay = bucket_layout([shape], S)
        if S > 1:
            rs_in = [rs_copy_in([grads[g][j]], lay) for g in range(rank_size)]
            outs = rs_reduce(rs_in, lay.I, rank_size, S, op)
        else:
            outs = [np.ascontiguousarray(grads[g][j], np.float32).reshape(-1) for g in range(rank_size)]
        if D > 1:
            outs = fused_ar(outs, rank_size, S, op)
        for g in range(rank_size):
            s = g % S
            if S > 1:
                result[g].append(sharded_grad(outs[g], lay, 0, s))
            else:
                result[g].append(outs[g].reshape(tuple(shape)))
    return result
