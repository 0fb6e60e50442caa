"""CPU emulation of the kernels' work decomposition (no GPU).

Mirrors, line for line in Python, the address arithmetic of seg_copy_kernel,
reduce_kernel and fold_copy_kernel (hsdp_parameter_gradient_amd/csrc/
kernels.hip): the 64-ary chunk search of the reductions and fold kernels
(the copy kernel reads a per-chunk item map; the host checker compares that
map with the chunk prefix), the chunk windows, the whole-vector
ranges, the strided and unit-wise row blocks, the fold items' unit
decomposition, the zero-fill range and the element-wise edge vectors.  For
many segment tables it checks that

  * every destination byte is written exactly once, with data from the
    right source offset before the data/padding edge and zero after it;
  * no byte outside the destination segments is written;
  * every 16-byte source block read lies inside the aligned envelope of its
    source range (so no read leaves the source's pages);
  * the chunk search finds the right item for every chunk (reductions and
    fold kernels; the copy's per-chunk map is built from the same prefix).

This is the host-side bounds check of the kernels' indexing; it runs before
any GPU does.
"""

import numpy as np
import pytest

CHUNK_SHIFTS = (9, 10, 15)


def align_down16(a):
    return a & ~15


def align_up16(a):
    return (a + 15) & ~15


def chunk_count(dst, nbytes, shift):
    return ((dst + nbytes - 1) >> shift) - (dst >> shift) + 1


def find_item(begin, n, c):
    """The kernel's 64-ary search (every lane probes one entry)."""
    lo, cnt = 0, n
    while cnt > 1:
        step = (cnt + 63) >> 6
        m = [off < cnt and begin[lo + off] <= c for off in (lane * step for lane in range(64))]
        k = sum(m) - 1
        assert m[:k + 1] == [True] * (k + 1) and not any(m[k + 1:])  # monotone ballot
        lo += k * step
        rest = cnt - k * step
        cnt = rest if rest < step else step
    return lo


def seg8(sg):
    """A copy segment with the strided-block fields (rows, src_pitch,
    dst_pitch, rows_per_chunk) filled in; a 4-tuple is one row."""
    return tuple(sg) if len(sg) == 8 else tuple(sg) + (1, 0, 0, 1)


def item_chunks(dst, row_bytes, rows, per, shift):
    return -(-rows // per) if rows > 1 else chunk_count(dst, row_bytes, shift)



def row_vectors(k, rows, per, row_bytes, CH):
    """Chunk k of a strided block: (row, byte column) of every vector, in
    the kernel's flat order (row = q // vpr)."""
    r0 = k * per
    nr = min(per, rows - r0)
    assert nr >= 1 and nr * row_bytes <= CH
    vpr = row_bytes >> 4
    return [(r0 + q // vpr, (q % vpr) * 16) for q in range(nr * vpr)]


def emulate_copy(segs, es, shift):
    """Writes as (dst_lo, dst_hi, kind, src_lo, item, row) and reads as
    aligned source ranges, per segment, following seg_copy_kernel."""
    CH = 1 << shift
    segs = [seg8(sg) for sg in segs]
    begin, n = [], 0
    for (src, dst, copy, total, rows, sp, dp, per) in segs:
        begin.append(n)
        n += item_chunks(dst, total, rows, per, shift)
    writes, reads = [], []
    for c in range(n):
        j = find_item(begin, len(segs), c)
        assert begin[j] <= c and (j + 1 == len(segs) or c < begin[j + 1])
        src, dst, copy, total, rows, sp, dp, per = segs[j]
        k = c - begin[j]
        if rows > 1:
            # the block contract the planner guarantees
            assert copy == total
            r0 = k * per
            nr = min(per, rows - r0)
            # at most a chunk of vector rows; unit-wise rows may cross it by one row
            assert nr >= 1 and (nr * copy <= CH if (sp | dp) % 16 == 0 else nr * copy < CH + copy)
            d0, s0 = dst + r0 * dp, src + r0 * sp
            if (sp | dp) % 16:  # rows_units: W-byte units, one flat range
                m = s0 | d0 | sp | dp | copy
                W = 8 if m % 8 == 0 else 4 if m % 4 == 0 else es
                upr = copy // W
                # 32-bit offsets from the chunk's first row on both sides
                assert (nr - 1) * max(sp, dp) + copy < 1 << 32
                for q in range(nr * upr):
                    row, col = r0 + q // upr, (q % upr) * W
                    a, sa = dst + row * dp + col, src + row * sp + col
                    assert a % W == 0 and sa % W == 0
                    writes.append((a, a + W, "data", sa, j, row))
                    reads.append((sa, sa + W, j, row))
                continue
            head = min((16 - (d0 & 15)) & 15, copy)
            vpr = (copy - head) >> 4
            tail = head + 16 * vpr
            for q in range(nr * vpr):  # rows_run's flat range
                row, col = r0 + q // vpr, head + (q % vpr) * 16
                a, sa = dst + row * dp + col, src + row * sp + col
                assert a % 16 == 0
                writes.append((a, a + 16, "data", sa, j, row))
                r = sa & 15
                reads.append((sa - r, sa - r + (32 if r else 16), j, row))
            for t in range(2 * nr):  # heads and tails, one row end per lane
                row = r0 + (t >> 1)
                lo, hi = (tail, copy) if t & 1 else (0, head)
                for x in range(lo, hi, es):
                    a, sa = dst + row * dp + x, src + row * sp + x
                    writes.append((a, a + es, "data", sa, j, row))
                    reads.append((sa, sa + es, j, row))
            continue
        base = (dst >> shift) << shift
        seg_end, cend = dst + total, dst + copy
        w0 = base + k * CH
        lo = max(w0, dst)
        hi = min(w0 + CH, seg_end)
        assert lo < hi
        ca, cb = align_up16(lo), align_down16(min(hi, cend))
        if ca < cb:
            s0 = src + (ca - dst)
            r = s0 & 15
            nv = (cb - ca) >> 4
            writes.append((ca, cb, "data", s0, j, 0))
            first = s0 - r
            last = first + 16 * (nv - 1) + (16 if r else 0)  # s[j] and, when shifted, s[j+1]
            reads.append((first, last + 16, j, 0))
        za, zb = align_up16(max(lo, cend)), align_down16(hi)
        if za < zb:
            writes.append((za, zb, "zero", None, j, 0))
        a_lo, a_c, a_hi = align_down16(lo), align_down16(cend), align_down16(hi)
        p_lo = (lo & 15) != 0
        p_c = (cend & 15) != 0 and lo < cend < hi and not (p_lo and a_c == a_lo)
        p_hi = (hi & 15) != 0 and not (p_lo and a_hi == a_lo) and not (p_c and a_hi == a_c)
        for flag, a in ((p_lo, a_lo), (p_c, a_c), (p_hi, a_hi)):
            if not flag:
                continue
            x0, x1 = max(a, lo), min(a + 16, hi)
            for x in range(x0, x1, es):
                if x < cend:
                    writes.append((x, x + es, "data", src + (x - dst), j, 0))
                    reads.append((src + (x - dst), src + (x - dst) + es, j, 0))
                else:
                    writes.append((x, x + es, "zero", None, j, 0))
    return writes, reads


def seg_row(sg, row):
    """(src, dst, copy_bytes, total_bytes) of one row of a segment."""
    src, dst, copy, total, rows, sp, dp, per = seg8(sg)
    assert 0 <= row < rows
    return src + row * sp, dst + row * dp, copy, total


def check_copy(segs, es, shift):
    writes, reads = emulate_copy(segs, es, shift)
    # exact cover of every row of every segment, no write outside
    ws = sorted(writes)
    spans = sorted((seg_row(sg, r)[1], seg_row(sg, r)[1] + seg_row(sg, r)[3])
                   for sg in segs for r in range(seg8(sg)[4]))
    merged = []
    for a, b in spans:
        if merged and a < merged[-1][1]:
            raise AssertionError("segments overlap")
        merged.append((a, b))
    cover = []
    for (a, b, kind, s0, j, row) in ws:
        if cover and a < cover[-1][1]:
            raise AssertionError(f"byte {a:#x} written twice")
        cover.append((a, b))
        src, dst, copy, total = seg_row(segs[j], row)
        assert dst <= a and b <= dst + total, "write outside its segment"
        if kind == "data":
            assert b <= dst + copy and s0 == src + (a - dst), "data write with a wrong source"
        else:
            assert a >= dst + copy, "zero write over data"
    # the union of writes equals the union of segments
    def union(iv):
        out = []
        for a, b in sorted(iv):
            if out and a == out[-1][1]:
                out[-1] = (out[-1][0], b)
            else:
                out.append((a, b))
        return out
    assert union(cover) == union([s for s in merged if s[0] < s[1]])
    for (a, b, j, row) in reads:
        src, dst, copy, total = seg_row(segs[j], row)
        assert align_down16(src) <= a and b <= align_up16(src + copy), "read outside the source envelope"
    return writes, reads


def job10(jb):
    """A reduce job with the strided-block fields (rows, src_pitch,
    dst_pitch, rows_per_chunk) filled in; a 6-tuple is one row."""
    return tuple(jb) if len(jb) == 10 else tuple(jb) + (1, 0, 0, 1)


def emulate_reduce(jobs, ptr, shift, es=4):
    """Writes per destination as (lo, hi, kind, job, dst, row) byte ranges
    and operand reads, following reduce_kernel.  A job is (nbytes,
    data_bytes, src0, nsrc, dst0, ndst[, rows, src_pitch, dst_pitch,
    rows_per_chunk]): the first data_bytes of each row are reduced, the rest
    zero filled."""
    CH = 1 << shift
    jobs = [job10(jb) for jb in jobs]
    begin, n = [], 0
    for (nbytes, data, src0, nsrc, dst0, ndst, rows, sp, dp, per) in jobs:
        begin.append(n)
        n += item_chunks(ptr[dst0], nbytes, rows, per, shift)
    writes, reads = [], []
    for c in range(n):
        j = find_item(begin, len(jobs), c)
        nbytes, data, src0, nsrc, dst0, ndst, rows, sp, dp, per = jobs[j]
        k = c - begin[j]
        if rows > 1:
            assert data == nbytes
            assert len({ptr[dst0 + m] & 15 for m in range(ndst)}) == 1
            r0 = k * per
            nr = min(per, rows - r0)
            assert nr >= 1 and nr * nbytes <= CH
            soff, doff = r0 * sp, r0 * dp
            if (sp | dp) % 16:  # reduce_rows_elems: element by element
                epr = nbytes // es
                for q in range(nr * epr):
                    row, col = r0 + q // epr, (q % epr) * es
                    for t in range(nsrc):
                        sa = ptr[src0 + t] + row * sp + col
                        reads.append((sa, sa + es, j, t, row))
                    for m in range(ndst):
                        a = ptr[dst0 + m] + row * dp + col
                        writes.append((a, a + es, "data", j, m, row))
                continue
            head = min((16 - ((ptr[dst0] + doff) & 15)) & 15, nbytes)
            vpr = (nbytes - head) >> 4
            tail = head + 16 * vpr
            for q in range(nr * vpr):
                row, col = r0 + q // vpr, head + (q % vpr) * 16
                for t in range(nsrc):
                    sa = ptr[src0 + t] + row * sp + col
                    r = sa & 15
                    reads.append((sa - r, sa - r + (32 if r else 16), j, t, row))
                for m in range(ndst):
                    a = ptr[dst0 + m] + row * dp + col
                    assert a % 16 == 0
                    writes.append((a, a + 16, "data", j, m, row))
            for t in range(2 * nr):
                row = r0 + (t >> 1)
                lo, hi = (tail, nbytes) if t & 1 else (0, head)
                for x in range(lo, hi, es):
                    for i in range(nsrc):
                        sa = ptr[src0 + i] + row * sp + x
                        reads.append((sa, sa + es, j, i, row))
                    for m in range(ndst):
                        a = ptr[dst0 + m] + row * dp + x
                        writes.append((a, a + es, "data", j, m, row))
            continue
        d0 = ptr[dst0]
        base = (d0 >> shift) << shift
        w0 = base + k * CH
        lo = max(w0, d0)
        hi = min(w0 + CH, d0 + nbytes)
        cend = d0 + data
        ca, cb = align_up16(lo), align_down16(min(hi, cend))
        if ca < cb:
            va, nv = ca - d0, (cb - ca) >> 4
            sa = [ptr[src0 + t] + va for t in range(nsrc)]
            rs = [a & 15 for a in sa]
            sb = [a - r for a, r in zip(sa, rs)]
            # compile-time operand counts rotate their lanes by the common
            # line phase (blocks before the first one in its 128-byte line)
            phase = {(a >> 4) & 7 for a in sb}
            e = phase.pop() if nsrc in COMPILED_K and len(phase) == 1 and len(set(rs)) == 1 else 0
            for t in range(nsrc):
                reads.append((sb[t] - 16 * e, sb[t] + 16 * nv + (16 if rs[t] else 0), j, t, 0))
            for m in range(ndst):
                writes.append((ptr[dst0 + m] + va, ptr[dst0 + m] + va + 16 * nv, "data", j, m, 0))
        za, zb = align_up16(max(lo, cend)), align_down16(hi)
        if za < zb:
            for m in range(ndst):
                writes.append((ptr[dst0 + m] + za - d0, ptr[dst0 + m] + zb - d0, "zero", j, m, 0))
        a_lo, a_c, a_hi = align_down16(lo), align_down16(cend), align_down16(hi)
        p_lo = (lo & 15) != 0
        p_c = (cend & 15) != 0 and lo < cend < hi and not (p_lo and a_c == a_lo)
        p_hi = (hi & 15) != 0 and not (p_lo and a_hi == a_lo) and not (p_c and a_hi == a_c)
        for flag, a in ((p_lo, a_lo), (p_c, a_c), (p_hi, a_hi)):
            if not flag:
                continue
            for x in range(max(a, lo), min(a + 16, hi), es):
                off = x - d0
                kind = "data" if x < cend else "zero"
                if kind == "data":
                    for t in range(nsrc):
                        reads.append((ptr[src0 + t] + off, ptr[src0 + t] + off + es, j, t, 0))
                for m in range(ndst):
                    writes.append((ptr[dst0 + m] + off, ptr[dst0 + m] + off + es, kind, j, m, 0))
    return writes, reads


COMPILED_K = (1, 2, 3, 4, 6, 8)  # the reduce kernel's compile-time operand counts


def align_down128(a):
    return a & ~127


def check_reduce(jobs, ptr, shift, es=4):
    writes, reads = emulate_reduce(jobs, ptr, shift, es)
    per = {}
    for (a, b, kind, j, m, row) in writes:
        per.setdefault((j, m, row), []).append((a, b, kind))
    for j, jb in enumerate(jobs):
        nbytes, data, src0, nsrc, dst0, ndst, rows, sp, dp, _ = job10(jb)
        for m in range(ndst):
            for row in range(rows):
                iv = sorted(per.pop((j, m, row), []))
                start = ptr[dst0 + m] + row * dp
                pos = start
                for a, b, kind in iv:
                    assert a == pos, f"job {j} dst {m} row {row}: gap or double write at {a:#x} (expected {pos:#x})"
                    edge = start + data
                    assert (b <= edge) if kind == "data" else (a >= edge), f"job {j}: {kind} write across the data end"
                    pos = b
                assert pos == start + nbytes
    assert not per, "writes attributed to no row"
    for (a, b, j, t, row) in reads:
        nbytes, data, src0, nsrc, dst0, ndst, rows, sp, dp, _ = job10(jobs[j])
        s = ptr[src0 + t] + row * sp
        # reads may start anywhere in the 128-byte line of the operand's
        # first byte (never in another page) and end in its last 16-byte block
        assert align_down128(s) <= a and b <= align_up16(s + data), "operand read outside its envelope"
    return writes, reads


# ---------------------------------------------------------------------------
# tables like the planner's, on fake addresses
# ---------------------------------------------------------------------------

def layout(shapes, S, dims=None):
    dims = dims or [0] * len(shapes)
    chunk, inner, outer, dk, padded, in_off, ro, rl = [], [], [], [], [], [], [], []
    off = 0
    for sh, k in zip(shapes, dims):
        n0 = sh[k]
        inn = int(np.prod(sh[k + 1:])) if len(sh) > k + 1 else 1
        out = int(np.prod(sh[:k])) if k else 1
        c = -(-n0 // S) if k == 0 else n0 // S
        chunk.append(c)
        inner.append(inn)
        outer.append(out)
        dk.append(n0)
        padded.append(out * c * inn)
        in_off.append(off)
        ro.append([min(s * c, n0) for s in range(S)])
        rl.append([min(c, n0 - min(s * c, n0)) for s in range(S)])
        off += out * c * inn
    return dict(I=off, inner=inner, outer=outer, dk=dk, padded=padded, in_off=in_off, ro=ro, rl=rl)


def ag_copy_in_segs(shapes, S, es, ag, shard_addr):
    L = layout(shapes, S)
    segs = []
    for s in range(S):
        for i in range(len(shapes)):
            nb = L["rl"][i][s] * L["inner"][i] * es
            total = L["padded"][i] * es
            if total:
                segs.append((shard_addr(s, i) if nb else 0, ag + (s * L["I"] + L["in_off"][i]) * es, nb, total))
    return segs


SHORT_ROW = 1024


def block_rows(sp, dp, row_bytes, shift):
    """Rows per chunk of a strided copy block (block_rows_per_chunk): as many
    as a chunk holds, or for unit-wise rows the fewest that fill it."""
    CH = 1 << shift
    return CH // row_bytes if sp % 16 == 0 and dp % 16 == 0 else -(-CH // row_bytes)


def copy_block_ok(src, dst, sp, dp, row_bytes, rows, shift):
    """When the planner emits one strided copy block instead of one item
    per row: the rows fit a chunk, and either both pitches are multiples of
    16 (vector rows) or the rows are short or move in 8-byte units."""
    if not (rows >= 2 and 0 < row_bytes <= (1 << shift)):
        return False
    if sp % 16 == 0 and dp % 16 == 0:
        return True
    if block_rows(sp, dp, row_bytes, shift) * max(sp, dp) >= 1 << 32:  # the kernel's 32-bit offsets
        return False
    return row_bytes <= SHORT_ROW or (src | dst | sp | dp | row_bytes) % 8 == 0


def reduce_block_ok(sp, dp, row_bytes, rows, shift):
    """The same for a reduction block (other pitches go element by element)."""
    return rows >= 2 and 0 < row_bytes <= (1 << shift) and ((sp % 16 == 0 and dp % 16 == 0) or row_bytes <= SHORT_ROW)


def push_rows(segs, src, dst, row_bytes, rows, sp, dp, shift):
    if row_bytes == 0 or rows == 0:
        return
    if copy_block_ok(src, dst, sp, dp, row_bytes, rows, shift):
        segs.append((src, dst, row_bytes, row_bytes, rows, sp, dp, block_rows(sp, dp, row_bytes, shift)))
    else:
        segs.extend((src + r * sp, dst + r * dp, row_bytes, row_bytes) for r in range(rows))


INTERLEAVE_ROW = 256


def interleave_rows(row_bytes, rows):
    """Short rows of a dim-k chunk: the S ranks' items of the same rows
    are emitted next to each other, one item per chunk of rows."""
    return 0 < row_bytes < INTERLEAVE_ROW and rows >= 2


def fold_rows(row_bytes, rows, S, CH, m=8):
    """Dim-k chunk rows the fold kernels take (fold_rows): short rows, or
    longer ones that are not a multiple of m bytes (8 for copies, 16 for the
    RS copy-reduce), when the S pieces of a full row fit a chunk."""
    if S < 2 or rows < 2 or row_bytes == 0 or S * row_bytes > CH:
        return False
    return row_bytes < INTERLEAVE_ROW or row_bytes % m != 0


def push_rows_interleaved(segs, base, row_bytes, rows, sp, dp, shift):
    per = (1 << shift) // row_bytes
    for r0 in range(0, rows, per):
        nr = min(per, rows - r0)
        for src, dst in base:
            push_rows(segs, src + r0 * sp, dst + r0 * dp, row_bytes, nr, sp, dp, shift)


def ag_copy_out_segs(shapes, S, es, ag, full_addr, dims=None, shift=14):
    """AG copy-out segments as fsdp_ag_copy_out builds them when short dim-k
    rows do not form fold items (its fallback; fold items are emulated by
    emulate_fold and checked on the planner's own tables)."""
    L = layout(shapes, S, dims)
    segs = []
    for i in range(len(shapes)):
        src = [ag + (s * L["I"] + L["in_off"][i]) * es for s in range(S)]
        dst = [full_addr(i) + L["ro"][i][s] * L["inner"][i] * es for s in range(S)]
        pitch = L["dk"][i] * L["inner"][i] * es
        row = L["rl"][i][0] * L["inner"][i] * es
        if L["outer"][i] > 1 and interleave_rows(row, L["outer"][i]):
            push_rows_interleaved(segs, list(zip(src, dst)), row, L["outer"][i], row, pitch, shift)
            continue
        for s in range(S):
            run = L["rl"][i][s] * L["inner"][i]
            push_rows(segs, src[s], dst[s], run * es, L["outer"][i], run * es, pitch, shift)
    return segs


def rs_copy_in_segs(shapes, S, es, grad_addr, rs_in_addr, dims=None, shift=14):
    """One rank's RS copy-in segments, as fsdp_rs_copy_in builds them when
    short dim-k rows do not form fold items (see ag_copy_out_segs)."""
    L = layout(shapes, S, dims)
    segs = []
    for s in range(S):
        for i in range(len(shapes)):
            if L["padded"][i] == 0:
                continue
            run = L["rl"][i][s] * L["inner"][i]
            src = grad_addr(i) + L["ro"][i][s] * L["inner"][i] * es
            d0 = rs_in_addr + (s * L["I"] + L["in_off"][i]) * es
            if L["outer"][i] == 1:
                segs.append((src if run else 0, d0, run * es, L["padded"][i] * es))
                continue
            if interleave_rows(run * es, L["outer"][i]):
                continue  # below
            push_rows(segs, src, d0, run * es, L["outer"][i], L["dk"][i] * L["inner"][i] * es, run * es, shift)
            data = L["outer"][i] * run
            if L["padded"][i] > data:
                segs.append((0, d0 + data * es, 0, (L["padded"][i] - data) * es))
    for i in range(len(shapes)):
        row = L["rl"][i][0] * L["inner"][i] * es
        if L["padded"][i] == 0 or L["outer"][i] == 1 or not interleave_rows(row, L["outer"][i]):
            continue
        base = [(grad_addr(i) + L["ro"][i][s] * L["inner"][i] * es, rs_in_addr + (s * L["I"] + L["in_off"][i]) * es)
                for s in range(S)]
        push_rows_interleaved(segs, base, row, L["outer"][i], L["dk"][i] * L["inner"][i] * es, row, shift)
    return segs


SHAPES = [
    [(7, 8), (5, 3), (16,)],
    [(4097, 8), (1009, 8), (5, 64), (3,)],
    [(100003,), (7, 3), (13,), (0, 5), (1,), (257, 33)],
    [(0,), (1,), (2,), (3,)],
]


@pytest.mark.parametrize("shapes", SHAPES)
@pytest.mark.parametrize("S", [1, 3, 4, 8])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", CHUNK_SHIFTS)
def test_copy_ops_cover_exactly(shapes, S, es, shift):
    base = 1 << 32
    rng = np.random.default_rng(S * 100 + es)
    ag = base + es * int(rng.integers(0, 9))
    # shards at scattered element offsets (every relative alignment)
    shard = {}
    a = base + (1 << 28)
    for s in range(S):
        for i in range(len(shapes)):
            shard[(s, i)] = a + es * int(rng.integers(0, 9))
            a += 1 << 22
    check_copy(ag_copy_in_segs(shapes, S, es, ag, lambda s, i: shard[(s, i)]), es, shift)
    full = {i: base + (1 << 30) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    check_copy(ag_copy_out_segs(shapes, S, es, ag, lambda i: full[i]), es, shift)


def test_random_segments():
    rng = np.random.default_rng(99)
    for trial in range(300):
        es = int(rng.choice([2, 4]))
        shift = int(rng.choice(CHUNK_SHIFTS[:2]))
        segs = []
        dst = (1 << 33) + es * int(rng.integers(0, 64))
        for _ in range(int(rng.integers(1, 12))):
            total = es * int(rng.choice([0, 1, 2, 3, 7, 8, 9, 63, 64, 65, 300, 1000, 5000]))
            copy = es * int(rng.integers(0, total // es + 1)) if total else 0
            src = (1 << 40) + int(rng.integers(0, 1 << 20)) * es
            if total:
                segs.append((src if copy else 0, dst, copy, total))
            dst += total + es * int(rng.choice([0, 0, 1, 5]))
        if segs:
            check_copy(segs, es, shift)


@pytest.mark.parametrize("shift", CHUNK_SHIFTS)
@pytest.mark.parametrize("es", [4, 2])
def test_reduce_jobs_cover_exactly(shift, es):
    rng = np.random.default_rng(shift + es)
    for trial in range(60):
        R, S = [(8, 4), (8, 8), (6, 3), (8, 1), (2, 2)][trial % 5]
        I = int(rng.choice([1, 2, 3, 5, 16, 17, 1000, 4097, 20000]))
        rs_in = [(1 << 36) + g * (1 << 26) + es * int(rng.integers(0, 8)) for g in range(R)]
        rs_out = [(1 << 38) + g * (1 << 26) + es * int(rng.integers(0, 8)) for g in range(R)]
        # RS jobs, as fsdp_rs_reduce builds them
        jobs, ptr = [], []
        for g in range(R):
            d, s = divmod(g, S)
            src0 = len(ptr)
            ptr += [rs_in[d * S + t] + s * I * es for t in range(S)]
            dst0 = len(ptr)
            ptr.append(rs_out[g])
            jobs.append((I * es, I * es, src0, S, dst0, 1))
        check_reduce(jobs, ptr, shift, es)
        # fused AR jobs (in place, 512-byte aligned bases, F*es a multiple of 512)
        D = R // S
        if D > 1:
            F = (512 // es) * int(rng.integers(1, 40))
            fused = [(1 << 39) + g * (1 << 26) for g in range(R)]
            jobs, ptr = [], []
            for s in range(S):
                src0 = len(ptr)
                ptr += [fused[d * S + s] for d in range(D)]
                jobs.append((F * es, F * es, src0, D, src0, D))
            check_reduce(jobs, ptr, shift, es)


def rs_copy_reduce_jobs(shapes, R, S, es, grad_addr, out_addr, dims=None, shift=13):
    """Jobs as fsdp_rs_copy_reduce builds them: one strided job per (rank,
    parameter) when the chunk's runs are whole aligned vectors, else one job
    per (rank, parameter, run of the chunk)."""
    L = layout(shapes, S, dims)
    jobs, ptr = [], []

    def push_block(g, i, r0, nr):
        d, s = divmod(g, S)
        run = L["rl"][i][s] * L["inner"][i]
        pitch = L["dk"][i] * L["inner"][i] * es
        src_off = L["ro"][i][s] * L["inner"][i] * es + r0 * pitch
        src0 = len(ptr)
        ptr.extend(grad_addr(d * S + t, i) + src_off for t in range(S))
        dst0 = len(ptr)
        ptr.append(out_addr(g) + L["in_off"][i] * es + r0 * run * es)
        if nr > 1:
            jobs.append((run * es, run * es, src0, S, dst0, 1, nr, pitch, run * es, (1 << shift) // (run * es)))
        else:
            jobs.append((run * es, run * es, src0, S, dst0, 1))

    interleaved = set()
    for g in range(R):
        d, s = divmod(g, S)
        for i, sh in enumerate(shapes):
            if L["padded"][i] == 0:
                continue
            run = L["rl"][i][s] * L["inner"][i]
            pitch = L["dk"][i] * L["inner"][i] * es
            if L["padded"][i] == L["outer"][i] * run and reduce_block_ok(pitch, run * es, run * es, L["outer"][i],
                                                                          shift):
                if interleave_rows(run * es, L["outer"][i]):
                    interleaved.add(i)
                else:
                    push_block(g, i, 0, L["outer"][i])
                continue
            for o in range(L["outer"][i]):
                last = o + 1 == L["outer"][i]
                src_off = (o * L["dk"][i] + L["ro"][i][s]) * L["inner"][i] * es
                src0 = len(ptr)
                ptr += [grad_addr(d * S + t, i) + src_off if run else 0 for t in range(S)]
                dst0 = len(ptr)
                ptr.append(out_addr(g) + (L["in_off"][i] + o * run) * es)
                nbytes = ((L["padded"][i] - o * run) if last else run) * es
                if nbytes:
                    jobs.append((nbytes, run * es, src0, S, dst0, 1))
    for d in range(R // S):
        for i in sorted(interleaved):
            per = (1 << shift) // (L["rl"][i][0] * L["inner"][i] * es)
            for r0 in range(0, L["outer"][i], per):
                for s in range(S):
                    push_block(d * S + s, i, r0, min(per, L["outer"][i] - r0))
    return jobs, ptr


@pytest.mark.parametrize("shapes", SHAPES)
@pytest.mark.parametrize("R,S", [(8, 4), (8, 8), (6, 3), (4, 1)])
@pytest.mark.parametrize("es", [4, 2])
@pytest.mark.parametrize("shift", (9, 13))
def test_rs_copy_reduce_jobs_cover_exactly(shapes, R, S, es, shift):
    rng = np.random.default_rng(R * 10 + S + es)
    grads = {(g, i): (1 << 40) + (g * 64 + i) * (1 << 24) + es * int(rng.integers(0, 8))
             for g in range(R) for i in range(len(shapes))}
    outs = {g: (1 << 44) + g * (1 << 26) + es * int(rng.integers(0, 8)) for g in range(R)}
    jobs, ptr = rs_copy_reduce_jobs(shapes, R, S, es, lambda g, i: grads[(g, i)], lambda g: outs[g])
    if jobs:
        check_reduce(jobs, ptr, shift, es)


def test_find_item_all_chunks():
    rng = np.random.default_rng(5)
    for n in (1, 2, 63, 64, 65, 100, 4095, 4096, 4097, 9000):
        sizes = rng.integers(1, 4, size=n)
        begin = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
        total = int(np.sum(sizes))
        for c in list(range(0, min(total, 300))) + list(range(max(0, total - 300), total)):
            j = find_item(begin, n, c)
            assert begin[j] <= c and (j + 1 == n or c < begin[j + 1])


# ---------------------------------------------------------------------------
# per-lane loops inside one window (copy_run / reduce_run / reduce_run_lds)
# ---------------------------------------------------------------------------

def lane_loop(nv, U, shifted, block=256):
    """Vectors written and source blocks read by every lane, following the
    kernels' loops: whole iterations of block*U vectors (wave-contiguous
    groups of 64 when the source is shifted, block-strided otherwise), then
    a block-strided tail.  Returns (writes, reads) as lists of
    (thread, index)."""
    writes, reads = [], []
    base = 0
    while base + block * U <= nv:
        for tid in range(block):
            lane, wave = tid & 63, tid >> 6
            if shifted:
                wb = base + wave * 64 * U
                for u in range(U):
                    writes.append((tid, wb + u * 64 + lane))
                    reads.append((tid, wb + u * 64 + lane))
                reads.append((tid, wb + 64 * U))  # the wave-uniform closing block
            else:
                for u in range(U):
                    writes.append((tid, base + tid + u * block))
                    reads.append((tid, base + tid + u * block))
        base += block * U
    for tid in range(block):
        j = base + tid
        while j < nv:
            writes.append((tid, j))
            reads.append((tid, j))
            if shifted:
                reads.append((tid, j + 1))
            j += block
    return writes, reads


@pytest.mark.parametrize("U", [1, 2, 4, 8])
@pytest.mark.parametrize("shifted", [False, True])
def test_lane_loops_cover_each_vector_once(U, shifted):
    for nv in (0, 1, 63, 64, 255, 256, 257, 511, 1024, 1025, 2048, 3000, 4096):
        writes, reads = lane_loop(nv, U, shifted)
        idx = sorted(v for _, v in writes)
        assert idx == list(range(nv)), (nv, U, shifted)
        top = nv if shifted else nv - 1  # a shifted source may read block nv
        assert all(0 <= r <= top for _, r in reads), (nv, U, shifted)


@pytest.mark.parametrize("block,U", [(1024, 1), (512, 2), (256, 4), (256, 1)])
@pytest.mark.parametrize("shifted", [False, True])
def test_copy_lane_loops_cover_each_vector_once(block, U, shifted):
    """copy_run at the copy kernel's workgroup shape (512 lanes, two vectors
    per lane per iteration) and the other shapes it can be built with."""
    for nv in (0, 1, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 3000, 4096, 16384 + 7):
        writes, reads = lane_loop(nv, U, shifted, block)
        assert sorted(v for _, v in writes) == list(range(nv)), (nv, block, U, shifted)
        top = nv if shifted else nv - 1
        assert all(0 <= r <= top for _, r in reads), (nv, block, U, shifted)


def fast_div(x, d):
    """FastDiv (kernels.hip): x / d as the high 32 bits of x * m, with
    m = 0xFFFFFFFF // d + 1 (= ceil(2**32 / d)) and d = 1 passed through."""
    x = np.asarray(x, dtype=np.uint64)
    if d == 1:
        return x
    m = np.uint64(0xFFFFFFFF // d + 1)
    return (x * m) >> np.uint64(32)


def test_fast_div_is_exact_inside_a_staging_window():
    """Every divisor and numerator below 2**15 (the fold kernels' LDS windows
    hold 18 KiB): exact at every multiple of d and one below it, and on a
    dense sample."""
    lim = 1 << 15
    for d in range(1, lim):
        k = np.arange(0, lim // d + 1, dtype=np.uint64) * np.uint64(d)
        x = np.concatenate([k, k[1:] - np.uint64(1)])
        x = x[x < lim]
        assert np.array_equal(fast_div(x, d), x // np.uint64(d)), d
    rng = np.random.default_rng(3)
    x = rng.integers(0, lim, 1 << 20).astype(np.uint64)
    for d in rng.integers(1, lim, 64):
        assert np.array_equal(fast_div(x, int(d)), x // np.uint64(d)), d


def stage_loop(n, stage, block=256):
    """stage_blocks: lane t takes blocks i0 + u*block (u < stage) per pass,
    i0 = t, t + stage*block, ...; returns (passes, [(thread, block)])."""
    done, passes = [], 0
    i0 = 0
    while i0 < n:
        passes += 1
        done += [(t, i0 + t + u * block) for t in range(block) for u in range(stage) if i0 + t + u * block < n]
        i0 += stage * block
    return passes, done


@pytest.mark.parametrize("stage", [4, 5, 6])
def test_fold_staging_covers_each_block_once(stage):
    lds_blocks = 18 * 1024 // 16  # the fold kernels' LDS staging buffer
    for n in (0, 1, 255, 256, 1023, 1024, 1025, 1027, 1100, lds_blocks):
        passes, done = stage_loop(n, stage)
        assert sorted(b for _, b in done) == list(range(n)), (stage, n)
        assert all(16 * b + 16 <= 18 * 1024 for _, b in done)
        if stage >= 5:  # the kernel's depth: one pass for any window that fits the buffer
            assert passes <= 1, (stage, n, passes)


def units_loop(n, U, block):
    """rows_units: whole iterations of block*U units (all loads before the
    stores), then the remainder as one predicated iteration.  Returns the
    units each lane moves, as (thread, unit)."""
    done, base = [], 0
    while base + block * U <= n:
        done += [(tid, base + tid + u * block) for tid in range(block) for u in range(U)]
        base += block * U
    if base < n:
        done += [(tid, q) for tid in range(block) for u in range(U)
                 for q in [base + tid + u * block] if q < n]
    return done


@pytest.mark.parametrize("W", [2, 4, 8])
@pytest.mark.parametrize("block", [1024, 512, 256])
def test_units_loop_moves_each_unit_once(W, block):
    U = max(1, min(4, 16384 // (block * W)))  # the kernel's units per lane
    for n in (0, 1, 63, 1023, 1024, 1025, 4095, 4096, 4097, 8192, 8193, 3 * block * U + 5):
        done = units_loop(n, U, block)
        assert sorted(q for _, q in done) == list(range(n)), (W, block, n)
        per_lane = {}
        for tid, _ in done:
            per_lane[tid] = per_lane.get(tid, 0) + 1
        # the units are spread evenly: no lane moves more than its share rounded up
        assert max(per_lane.values(), default=0) <= -(-n // block)


def tail_units_loop(n, U, UT, block=256):
    """fold_units / fold_reduce_units: whole iterations of block*U units
    (all loads before the stores), then the rest in predicated iterations
    of block*UT units (UT = 1: the loop of one unit per lane at a time).
    Returns (thread, unit) pairs and the iteration count."""
    done, base, iters = [], 0, 0
    while base + block * U <= n:
        done += [(tid, base + tid + u * block) for tid in range(block) for u in range(U)]
        base += block * U
        iters += 1
    while base < n:
        done += [(tid, q) for tid in range(block) for u in range(UT)
                 for q in [base + tid + u * block] if q < n]
        base += block * UT
        iters += 1
    return done, iters


@pytest.mark.parametrize("W", [2, 4, 8, 16])
@pytest.mark.parametrize("K", [None, 2, 3, 4, 6, 8])
def test_fold_unit_loops_move_each_unit_once(W, K):
    """K None: the fold copy (U = 4 for 16-byte units, else 8, one
    predicated iteration for the rest); K: the fold reduce over K operands
    (U = max(1, U0 // K), U0 = 8 for 16-byte units, else 16; over 2 ranks
    units under 16 bytes finish in one predicated iteration of U, or two of
    U // 2 for 16-bit elements, the rest one unit per lane at a time)."""
    if K is None:
        U = 4 if W >= 16 else 8
        UT = U
    else:
        U0 = 8 if W >= 16 else 16
        U = max(1, U0 // K)
        UT = U if K == 2 and W < 16 else 1  # fp32; 16-bit elements: U // 2 (below)
    uts = {UT, U // 2} if K == 2 and W < 16 else {UT}
    for ut in sorted(uts):
        for rows, run in ((1, 4120), (3, 4120), (1, 8240), (128, 32), (7, 24), (2, 2048)):
            n = rows * 2 * (run // W) if run % W == 0 else 0
            done, iters = tail_units_loop(n, U, ut)
            assert sorted(q for _, q in done) == list(range(n)), (W, K, ut, rows, run)
            # the whole iterations, then at most ceil(U / ut) predicated ones
            assert iters <= n // (256 * U) + -(-U // ut)
            per_lane = {}
            for tid, _ in done:
                per_lane[tid] = per_lane.get(tid, 0) + 1
            assert max(per_lane.values(), default=0) <= -(-n // 256)


def lds_piece_loop(nv, U, e=0, block=256, piece=512):
    """The shifted reduction's loops (reduce_run_lds): per piece of at most
    `piece` destination vectors, whole iterations of block*U result blocks
    then a block-strided tail load the piece's np + 1 aligned blocks of
    every operand and the e blocks of line phase before them, writing result
    block b to LDS slot b + e; after a barrier lane q writes destination
    vector p0 + q from LDS slots q + e and q + e + 1.  Returns (writes,
    reads, lds_writes, lds_reads, runs): global vector / block indices,
    (piece, slot) pairs, and the first block of every wave's 64-lane run."""
    writes, reads, lds_w, lds_r, runs = [], [], [], [], []
    p0 = 0
    while p0 < nv:
        np_ = min(piece, nv - p0)
        nb = np_ + 1 + e
        j0 = 0
        while j0 + block * U <= nb:
            for tid in range(block):
                for u in range(U):
                    j = j0 + tid + u * block
                    reads.append(p0 - e + j)
                    lds_w.append((p0, j))
                    if tid % 64 == 0:
                        runs.append(p0 - e + j)
            j0 += block * U
        for tid in range(block):
            j = j0 + tid
            while j < nb:
                reads.append(p0 - e + j)
                lds_w.append((p0, j))
                j += block
        written = {slot for (pp, slot) in lds_w if pp == p0}
        for tid in range(block):
            q = tid
            while q < np_:
                assert q + e in written and q + e + 1 in written  # the barrier sits between the phases
                lds_r.extend([(p0, q + e), (p0, q + e + 1)])
                writes.append(p0 + q)
                q += block
        p0 += piece
    return writes, reads, lds_w, lds_r, runs


@pytest.mark.parametrize("U", [1, 2, 4])
def test_shifted_reduce_lds_pieces(U):
    """Each destination vector is written once; each operand block in
    [-e, nv] (block nv holds the last vector's shifted bytes; the e blocks
    before block 0 share its 128-byte line) is read, once per piece; only the
    blocks around a piece edge are read twice; LDS slots stay below
    piece + 8; every wave's run of 64 blocks starts on a line (block index
    + e a multiple of 8, with the operand's block 0 at phase e)."""
    for piece in (512, 64):
        for e in (0, 1, 3, 7):
            for nv in (1, 2, 63, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 3000):
                writes, reads, lds_w, lds_r, runs = lds_piece_loop(nv, U, e, piece=piece)
                assert sorted(writes) == list(range(nv)), (nv, U, piece, e)
                assert min(reads) == -e and max(reads) == nv, (nv, U, piece, e)
                dup = sorted(b for b in set(reads) if reads.count(b) > 1)
                edges = sorted({b for p in range(piece, nv, piece) for b in range(p - e, p + 1)})
                assert dup == edges, (nv, U, piece, e, dup)
                assert len(lds_w) == len(set(lds_w)) and all(0 <= s < piece + 8 for _, s in lds_w + lds_r)
                assert all((r + e) % 8 == 0 for r in runs), (nv, U, piece, e)


def rotated_lane_loop(nv, U, e, block=256):
    """reduce_run's loops (aligned operands, MODE 0) with the lanes rotated
    by the line phase e: lane-linear index j reads vector j - e (blocks
    before vector 0 share its line) and writes it when j >= e.  Returns
    (writes, reads, runs)."""
    writes, reads, runs = [], [], []
    n = nv + e
    base = 0
    while base + block * U <= n:
        for tid in range(block):
            for u in range(U):
                j = base + tid + u * block
                reads.append(j - e)
                if tid % 64 == 0:
                    runs.append(j - e)
                if j >= e:
                    writes.append(j - e)
        base += block * U
    for tid in range(block):
        j = base + tid
        while j < n:
            reads.append(j - e)
            if j >= e:
                writes.append(j - e)
            j += block
    return writes, reads, runs


@pytest.mark.parametrize("U", [1, 2, 4])
def test_rotated_reduce_lanes(U):
    for e in range(8):
        for nv in (0, 1, 7, 8, 63, 255, 256, 257, 511, 512, 1024, 1025, 3000):
            writes, reads, runs = rotated_lane_loop(nv, U, e)
            assert sorted(writes) == list(range(nv)), (nv, U, e)
            assert len(reads) == len(set(reads)) and all(-e <= r < nv for r in reads), (nv, U, e)
            assert all((r + e) % 8 == 0 for r in runs), (nv, U, e)


def test_realign_neighbour_is_next_block():
    """Lane l of group u needs block wb + 64u + l + 1: lanes 0..62 take it
    from lane l+1 of the same group, lane 63 from lane 0 of group u+1 or
    from the closing block."""
    for U in (1, 2, 4):
        wb = 1000
        blocks = {(u, l): wb + u * 64 + l for u in range(U) for l in range(64)}
        tail = wb + 64 * U
        for u in range(U):
            for l in range(64):
                if l < 63:
                    got = blocks[(u, (l + 1) & 63)]
                else:
                    got = blocks[(u + 1, 0)] if u + 1 < U else tail
                assert got == blocks[(u, l)] + 1


MIXED_DIMS = [([(6, 8), (4, 12, 3), (5, 3, 8), (7, 3), (16,), (3, 4, 4)], [1, 1, 2, 0, 0, 2])]


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", (9, 14))
def test_nonzero_shard_dim_tables_cover_exactly(S, es, shift):
    shapes, dims = MIXED_DIMS[0]
    rng = np.random.default_rng(S + es)
    base = 1 << 32
    ag = base + es * int(rng.integers(0, 9))
    full = {i: base + (1 << 30) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    check_copy(ag_copy_out_segs(shapes, S, es, ag, lambda i: full[i], dims, shift), es, shift)
    grads = {i: (1 << 40) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    check_copy(rs_copy_in_segs(shapes, S, es, lambda i: grads[i], (1 << 44) + es * 3, dims, shift), es, shift)
    R = 2 * S
    gr = {(g, i): (1 << 40) + (g * 64 + i) * (1 << 24) + es * int(rng.integers(0, 8))
          for g in range(R) for i in range(len(shapes))}
    outs = {g: (1 << 46) + g * (1 << 26) + es * int(rng.integers(0, 8)) for g in range(R)}
    jobs, ptr = rs_copy_reduce_jobs(shapes, R, S, es, lambda g, i: gr[(g, i)], lambda g: outs[g], dims,
                                    shift)
    check_reduce(jobs, ptr, shift, es)


# Strided blocks: rows of whole aligned vectors (bf16 and fp32), several
# rows per chunk, a last chunk of fewer rows, rows as large as a chunk, and
# parameters whose rows are not whole vectors (one item per row) beside them.
BLOCK_SHAPES = ([(96, 64), (32, 64), (130, 32), (33, 128), (64,), (3,), (5, 24, 2), (7, 40), (3, 2048)],
                [1, 1, 1, 1, 0, 0, 1, 1, 1])


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", (9, 10, 14))
def test_strided_block_tables_cover_exactly(S, es, shift):
    shapes, dims = BLOCK_SHAPES
    dims = [k if k == 0 or shapes[i][k] % S == 0 else 0 for i, k in enumerate(dims)]
    rng = np.random.default_rng(S * 7 + es + shift)
    base = 1 << 32
    L = layout(shapes, S, dims)
    ag = base + 512 * int(rng.integers(0, 9))
    full = {i: base + (1 << 30) + i * (1 << 24) + 16 * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = ag_copy_out_segs(shapes, S, es, ag, lambda i: full[i], dims, shift)
    assert any(len(sg) == 8 for sg in segs), "no strided block planned"
    check_copy(segs, es, shift)
    grads = {i: (1 << 40) + i * (1 << 24) + 16 * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = rs_copy_in_segs(shapes, S, es, lambda i: grads[i], (1 << 44) + 512, dims, shift)
    assert any(len(sg) == 8 for sg in segs)
    check_copy(segs, es, shift)
    R = 2 * S
    gr = {(g, i): (1 << 40) + (g * 64 + i) * (1 << 24) + 16 * int(rng.integers(0, 8))
          for g in range(R) for i in range(len(shapes))}
    outs = {g: (1 << 46) + g * (1 << 26) + 512 * int(rng.integers(0, 8)) for g in range(R)}
    jobs, ptr = rs_copy_reduce_jobs(shapes, R, S, es, lambda g, i: gr[(g, i)], lambda g: outs[g], dims, shift)
    assert any(len(jb) == 10 for jb in jobs) or L["I"] * es < 16
    check_reduce(jobs, ptr, shift, es)


# ---------------------------------------------------------------------------
# XCD-aware chunk order (xcd_chunk in kernels.hip)
# ---------------------------------------------------------------------------

XCD_RUN = 64


def xcd_chunk(c, n, run=XCD_RUN):
    G = 8 * run
    if c >= n // G * G:
        return c
    rem = c % G
    return c - rem + (rem & 7) * run + (rem >> 3)


def grid_for(n_chunks, max_grid):
    if n_chunks < max_grid:
        return n_chunks
    return max_grid & ~7 if max_grid >= 8 else max_grid


@pytest.mark.parametrize("n", [1, 7, 8, 511, 512, 513, 1023, 1024, 1556, 6148, 12296, 24736, 100003])
def test_xcd_chunk_order_is_a_bijection(n):
    assert sorted(xcd_chunk(c, n) for c in range(n)) == list(range(n))


@pytest.mark.parametrize("n,max_grid", [(24736, 1 << 20), (5000, 1000), (5000, 1003), (100003, 4096), (9, 5)])
def test_xcd_runs_are_contiguous_per_xcd(n, max_grid):
    """Every chunk is processed exactly once over the grid-stride loop, and
    in every full group the chunks of one XCD (slot % 8 under round-robin
    dispatch) are kXcdRun consecutive chunks."""
    G = grid_for(n, max_grid)
    seen = []
    xcd_of = {}
    for b in range(G):
        slot = b
        while slot < n:
            c = xcd_chunk(slot, n)
            seen.append(c)
            xcd_of[c] = b % 8
            slot += G
    assert sorted(seen) == list(range(n))
    if G % 8 == 0 or G == n:
        full = n // (8 * XCD_RUN) * 8 * XCD_RUN
        for g0 in range(0, full, 8 * XCD_RUN):
            for x in range(8):
                run = range(g0 + x * XCD_RUN, g0 + (x + 1) * XCD_RUN)
                assert {xcd_of[c] for c in run} == {x}


@pytest.mark.parametrize("S", [2, 4, 8])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", (9, 14))
def test_misaligned_strided_blocks_cover_exactly(S, es, shift):
    """Copy blocks whose rows are not whole aligned vectors (odd slice
    sizes put every rank slice at another offset mod 16; rows of a few
    bytes; buffers at element offsets): heads, tails and realigned whole
    vectors cover every row exactly, reads stay in each row's envelope."""
    shapes = [(96, 64), (7, 40), (3,), (33, 128), (5, 24, 2), (2, 2048), (9, 8)]
    dims = [1, 1, 0, 1, 1, 1, 1]
    dims = [k if k == 0 or shapes[i][k] % S == 0 else 0 for i, k in enumerate(dims)]
    rng = np.random.default_rng(S * 11 + es + shift)
    base = 1 << 32
    ag = base + es * int(rng.integers(1, 9))
    full = {i: base + (1 << 30) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = ag_copy_out_segs(shapes, S, es, ag, lambda i: full[i], dims, shift)
    blocks = [sg for sg in segs if len(sg) == 8]
    assert any((sg[0] | sg[1]) & 15 for sg in blocks), "no misaligned block planned"
    check_copy(segs, es, shift)
    grads = {i: (1 << 40) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = rs_copy_in_segs(shapes, S, es, lambda i: grads[i], (1 << 44) + es * 5, dims, shift)
    assert any(len(sg) == 8 for sg in segs)
    check_copy(segs, es, shift)


@pytest.mark.parametrize("S", [2, 4, 8])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", (9, 13))
def test_misaligned_strided_reduce_jobs_cover_exactly(S, es, shift):
    """RS copy-reduce blocks with gradients and outputs at element offsets
    (operands shifted alike or differently, heads and tails per row)."""
    shapes = [(96, 64), (7, 40), (3,), (33, 128), (5, 24, 2), (2, 2048), (9, 8)]
    dims = [1, 1, 0, 1, 1, 1, 1]
    dims = [k if k == 0 or shapes[i][k] % S == 0 else 0 for i, k in enumerate(dims)]
    R = 2 * S
    rng = np.random.default_rng(S * 13 + es + shift)
    for same_shift in (True, False):
        off = {(g, i): es * (3 if same_shift else int(rng.integers(0, 8))) for g in range(R) for i in range(len(shapes))}
        gr = {(g, i): (1 << 40) + (g * 64 + i) * (1 << 24) + off[(g, i)] for g in range(R) for i in range(len(shapes))}
        outs = {g: (1 << 46) + g * (1 << 26) + es * int(rng.integers(1, 8)) for g in range(R)}
        jobs, ptr = rs_copy_reduce_jobs(shapes, R, S, es, lambda g, i: gr[(g, i)], lambda g: outs[g], dims, shift)
        assert any(len(jb) == 10 for jb in jobs)
        check_reduce(jobs, ptr, shift, es)


# parameters whose dim-k chunks have row pitches that are not multiples of
# 16 bytes: short rows (element-unit blocks), rows long enough for 8-byte
# units, and long rows of narrow units (one item per row)
ODD_PITCH_SHAPES = [(64, 6), (33, 12, 3), (9, 20), (1000, 6), (3, 2050, 1), (5, 8, 3), (2, 1030, 4), (7, 4, 5)]


@pytest.mark.parametrize("S", [2, 4])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shift", (9, 14))
def test_odd_pitch_blocks_cover_exactly(S, es, shift):
    """Copy blocks and RS copy-reduce blocks of rows whose pitches are not
    multiples of 16 bytes: the rows move in 8-, 4- or element-sized units
    (every unit aligned to its width), every row byte written once, reads
    inside the rows; buffers at element offsets."""
    shapes = ODD_PITCH_SHAPES
    dims = [1 if sh[1] % S == 0 else 0 for sh in shapes]
    rng = np.random.default_rng(S * 17 + es + shift)
    base = 1 << 32
    ag = base + es * int(rng.integers(0, 9))
    full = {i: base + (1 << 30) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = ag_copy_out_segs(shapes, S, es, ag, lambda i: full[i], dims, shift)
    odd = [sg for sg in segs if len(sg) == 8 and (sg[5] | sg[6]) % 16]
    assert odd, "no odd-pitch block planned"
    check_copy(segs, es, shift)
    grads = {i: (1 << 40) + i * (1 << 24) + es * int(rng.integers(0, 9)) for i in range(len(shapes))}
    segs = rs_copy_in_segs(shapes, S, es, lambda i: grads[i], (1 << 44) + es * 3, dims, shift)
    assert any(len(sg) == 8 and (sg[5] | sg[6]) % 16 for sg in segs)
    check_copy(segs, es, shift)
    R = 2 * S
    gr = {(g, i): (1 << 40) + (g * 64 + i) * (1 << 24) + es * int(rng.integers(0, 8))
          for g in range(R) for i in range(len(shapes))}
    outs = {g: (1 << 46) + g * (1 << 26) + es * int(rng.integers(0, 8)) for g in range(R)}
    jobs, ptr = rs_copy_reduce_jobs(shapes, R, S, es, lambda g, i: gr[(g, i)], lambda g: outs[g], dims, shift)
    assert any(len(jb) == 10 and (jb[7] | jb[8]) % 16 for jb in jobs)
    check_reduce(jobs, ptr, shift, es)


def test_odd_pitch_unit_widths():
    """The unit width the kernel picks for a chunk of odd-pitch rows: the
    widest of 8, 4 and the element size that divides both first-row
    addresses, both pitches and the row length."""
    def unit(es, s0, d0, sp, dp, row):
        m = s0 | d0 | sp | dp | row
        return 8 if m % 8 == 0 else 4 if m % 4 == 0 else es
    assert unit(4, 1 << 20, 8, 24, 40, 8) == 8
    assert unit(4, 1 << 20, 4, 24, 40, 8) == 4
    assert unit(2, 2, 0, 24, 40, 8) == 2
    assert unit(2, 0, 0, 36, 18, 18) == 2
    # the planner keeps long rows of narrow units one item per row
    assert not copy_block_ok(0, 2, 4100, 2050, 2050, 3, 14)
    assert copy_block_ok(0, 8, 8200, 4104, 4104, 3, 14)
    assert copy_block_ok(2, 0, 36, 18, 18, 100, 14)
    # a chunk's rows must lie within 4 GiB of its first row (32-bit offsets)
    assert not copy_block_ok(0, 0, 1 << 20 | 4, 4, 4, 100, 14) and copy_block_ok(0, 0, (1 << 18) | 4, 4, 4, 100, 14)
    assert not reduce_block_ok(8200, 4104, 4104, 3, 14) and reduce_block_ok(36, 18, 18, 100, 14)


# ---------------------------------------------------------------------------
# fold_copy_kernel: a dim-k parameter's short rows, all shard ranks at once
# ---------------------------------------------------------------------------

FOLD_FMT = "<6Q4I"  # full, run_bytes, rows, rows_per_chunk, rank0, rank_pitch, nrank, unit, gather, reserved


def _merge(iv):
    out = []
    for a, b in sorted(x for x in iv if x[0] < x[1]):
        if out and a <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], b))
        else:
            out.append((a, b))
    return out


FOLD_LDS = 18 * 1024  # kFoldLds
FOLD_LDS_MAX_UNIT = 4  # kFoldLdsMaxUnit
FOLD_UNIT_CHUNK = 16384  # kFoldUnitChunk


def fold_lds_bytes(f, r0, nr):
    """LDS bytes a fold chunk needs, 0 if it does not fit (fold_lds_bytes)."""
    full, run, S, gather = f[0], f[1], f[6], f[8]
    L = nr * run
    if gather:
        need = S * ((L + 15) // 16 + 1) * 16
    else:
        F0 = full + r0 * S * run
        need = ((F0 + L * S + 15) & ~15) - (F0 & ~15)
    return need if need <= FOLD_LDS else 0


class Recorder:
    """Memory for the emulated kernels: records every access as (lo, hi,
    item); with `mem` (a numpy uint8 array indexed by address) it also
    moves the bytes."""

    def __init__(self, mem=None):
        self.mem, self.reads, self.writes, self.item = mem, [], [], 0

    def load(self, a, n):
        self.reads.append((a, a + n, self.item))
        return bytes(self.mem[a:a + n]) if self.mem is not None else bytes(n)

    def store(self, a, data):
        self.writes.append((a, a + len(data), self.item))
        if self.mem is not None:
            self.mem[a:a + len(data)] = np.frombuffer(data, dtype=np.uint8)


def _ends(lo, hi):
    """The element runs of [lo, hi) outside its whole aligned vectors."""
    va, vb = (lo + 15) & ~15, hi & ~15
    return [(lo, va), (vb, hi)] if va < vb else [(lo, hi)]


def fold_lds_chunk(f, r0, nr, io):
    """One chunk of fold_copy_kernel's LDS path (fold_lds)."""
    full, run, S, W, gather, pitch, rank0 = f[0], f[1], f[6], f[7], f[8], f[5], f[4]
    g = 4 if W >= 4 else 2
    FR, L = S * run, nr * run
    F0, R0 = full + r0 * FR, rank0 + r0 * run
    lds = bytearray(FOLD_LDS)
    if gather:
        nb = (L + 15) // 16 + 1
        for i in range(S * nb):  # the kernel's flat block loop
            s, k = divmod(i, nb)
            a = R0 + s * pitch
            blk = (a & ~15) + 16 * k
            if blk < ((a + L + 15) & ~15):
                assert 16 * i + 16 <= FOLD_LDS
                lds[16 * i:16 * i + 16] = io.load(blk, 16)

        def src(x):  # full-side chunk byte x
            row, rem = divmod(x, FR)
            s, col = divmod(rem, run)
            o = s * nb * 16 + ((R0 + s * pitch) & 15) + row * run + col
            assert o + g <= (s + 1) * nb * 16 <= FOLD_LDS  # inside window s
            return bytes(lds[o:o + g])

        va, vb = (F0 + 15) & ~15, (F0 + nr * FR) & ~15
        for v in range(va, vb, 16):
            io.store(v, b"".join(src(v - F0 + k) for k in range(0, 16, g)))
        for lo, hi in _ends(F0, F0 + nr * FR):
            for x in range(lo, hi, g):
                io.store(x, src(x - F0))
    else:
        fa = F0 & ~15
        delta = F0 - fa
        for i in range((((F0 + nr * FR + 15) & ~15) - fa) // 16):
            assert 16 * i + 16 <= FOLD_LDS
            lds[16 * i:16 * i + 16] = io.load(fa + 16 * i, 16)
        for s in range(S):
            d = R0 + s * pitch

            def src(y):  # rank s's chunk byte y
                row, col = divmod(y, run)
                o = delta + row * FR + s * run + col
                assert o + g <= delta + nr * FR <= FOLD_LDS
                return bytes(lds[o:o + g])

            for v in range((d + 15) & ~15, (d + L) & ~15, 16):
                io.store(v, b"".join(src(v - d + k) for k in range(0, 16, g)))
            for lo, hi in _ends(d, d + L):
                for y in range(lo, hi, g):
                    io.store(y, src(y - d))


def fold_units_chunk(f, r0, nr, io):
    """One chunk of fold_copy_kernel's unit path (fold_units): unit q of a
    chunk is row q // upf, rank (q % upf) // upr, column q % upr; the full
    side is contiguous, rank s's rows dense from rank0 + s*rank_pitch."""
    full, run, S, W, gather, pitch, rank0 = f[0], f[1], f[6], f[7], f[8], f[5], f[4]
    assert nr * run < 1 << 32  # the kernel's 32-bit rank-side offsets
    upr = run // W
    upf = S * upr
    full0 = full + r0 * S * run
    for q in range(nr * upf):
        row, rem = divmod(q, upf)
        s, col = divmod(rem, upr)
        fa = full0 + q * W
        ra = rank0 + s * pitch + (r0 + row) * run + col * W
        src, dst = (ra, fa) if gather else (fa, ra)
        io.store(dst, io.load(src, W))


FLAT_CHUNK = 12288     # kFlatChunk: full-tensor bytes of a flat chunk
FLAT_MIN_RUN = 1024     # kFlatMinRun
FLAT_ADJ = 256          # kFlatAdj: LDS bytes kept for the pieces' offsets


def fold_item_chunks(rows, per, full_row, sub):
    """Chunks of a fold or fold-reduce item (fold_item_chunks)."""
    return -(-(rows * full_row) // sub) if per == 0 else -(-rows // per)


def flat_chunk(k, total, sub, run):
    """A flat chunk (flat_chunk): first byte, length, first piece, and the
    parts (piece, a, b) it meets, a and b chunk-relative."""
    X0 = k * sub
    n = min(total - X0, sub)
    p_lo = X0 // run
    off0 = X0 - p_lo * run
    pieces = (off0 + n - 1) // run + 1
    parts = []
    for q in range(pieces):
        lo, hi = q * run, (q + 1) * run
        parts.append((p_lo + q, max(lo, off0) - off0, min(hi, off0 + n) - off0))
    return X0, n, p_lo, off0, parts


def _flat_scatter(parts, delta, lds, g, dst, io, writes=None, j=None):
    """flat_scatter: every part written from LDS (chunk byte x at delta + x)."""
    for p, a, b in parts:
        d = dst(p, a)

        def src(y, a=a, d=d):
            o = delta + a + (y - d)
            assert 0 <= o and o + g <= len(lds)
            return bytes(lds[o:o + g])

        for v in range((d + 15) & ~15, (d + b - a) & ~15, 16):
            # the kernel reads the vector's 16 LDS bytes as four or five dwords
            assert ((delta + a + (v - d)) & ~3) + 20 <= FOLD_LDS
            io.store(v, b"".join(src(v + k) for k in range(0, 16, g)))
            if writes is not None:
                writes.append((v, v + 16, j, None))
        for lo, hi in _ends(d, d + b - a):
            for y in range(lo, hi, g):
                io.store(y, src(y))
                if writes is not None:
                    writes.append((y, y + g, j, None))


def fold_sub_chunk(f, k, io):
    """One flat chunk of fold_copy_kernel (fold_flat)."""
    full, run, rows, per, rank0, pitch, S, W, gather, sub = f
    assert per == 0 and sub % 16 == 0 and sub % W == 0
    g = 4 if W >= 4 else 2
    X0, n, p_lo, off0, parts = flat_chunk(k, rows * S * run, sub, run)
    assert n > 0 and 4 * len(parts) <= FLAT_ADJ
    F = full + X0

    def src_addr(p, a):
        r, s_ = divmod(p, S)
        return rank0 + s_ * pitch + r * run + (X0 + a - p * run)

    if gather:
        lds = bytearray(FOLD_LDS)
        w, adj, win = 0, {}, {}
        for q, (p, a, b) in enumerate(parts):
            ad = src_addr(p, a)
            lo, hi = ad & ~15, (ad + (b - a) + 15) & ~15
            adj[q] = w + (ad & 15) - a
            win[q] = (w, w + hi - lo)
            for blk in range(lo, hi, 16):
                assert w + 16 <= FOLD_LDS - FLAT_ADJ
                lds[w:w + 16] = io.load(blk, 16)
                w += 16

        def rd(x):
            q = (x + off0) // run
            o = adj[q] + x
            assert win[q][0] <= o and o + g <= win[q][1]  # inside piece q's window
            return bytes(lds[o:o + g])

        for v in range((F + 15) & ~15, (F + n) & ~15, 16):
            x = v - F
            q = (x + off0) // run
            if x + off0 + 16 <= (q + 1) * run:  # one piece: four or five dwords from LDS
                assert ((adj[q] + x) & ~3) + 20 <= FOLD_LDS - FLAT_ADJ + 4
            io.store(v, b"".join(rd(x + i) for i in range(0, 16, g)))
        for lo, hi in _ends(F, F + n):
            for xa in range(lo, hi, g):
                io.store(xa, rd(xa - F))
    else:
        fa = F & ~15
        nblk = (((F + n + 15) & ~15) - fa) // 16
        assert nblk * 16 <= FOLD_LDS
        lds = bytearray(nblk * 16)
        for i in range(nblk):
            lds[16 * i:16 * i + 16] = io.load(fa + 16 * i, 16)
        _flat_scatter(parts, F - fa, lds, g, src_addr, io)


def flat_fold_item(full, rank0, pitch, S, run, rows, es, gather, shift=14):
    """A flat-chunk fold item as the planner builds it (push_fold, rows too
    long for one chunk); None where the planner makes none."""
    CH = 1 << shift
    if not (S >= 2 and rows >= 2 and S * run > CH and run >= FLAT_MIN_RUN and run % 8):
        return None
    m = full | run | rank0 | pitch
    W = 16 if m % 16 == 0 else 8 if m % 8 == 0 else 4 if m % 4 == 0 else 2
    if W < es:
        return None
    return (full, run, rows, 0, rank0, pitch, S, W, int(gather), FLAT_CHUNK)


def emulate_fold(folds, CH, io=None, lds=True):
    """fold_copy_kernel over a fold table: returns the chunk prefix, the
    chunk count and the reads and writes as (lo, hi, item).  Chunk k of item
    j is full-tensor rows [k*per, ...); a chunk takes the LDS path when its
    unit and its windows allow it (lds=False: the unit path always)."""
    io = io if io is not None else Recorder()
    begin, n = [], 0
    for f in folds:
        begin.append(n)
        n += fold_item_chunks(f[2], f[3], f[6] * f[1], f[9])
    for c in range(n):
        j = find_item(begin, len(folds), c)
        f = folds[j]
        full, run, rows, per, rank0, pitch, S, W = f[:8]
        assert W in (2, 4, 8, 16) and (full | run | rank0 | pitch) % W == 0
        if per == 0:  # flat chunks
            io.item = j
            fold_sub_chunk(f, c - begin[j], io)
            continue
        assert per * S * run <= CH and per >= 1
        r0 = (c - begin[j]) * per
        nr = min(per, rows - r0)
        io.item = j
        if lds and W <= FOLD_LDS_MAX_UNIT and fold_lds_bytes(f, r0, nr):
            fold_lds_chunk(f, r0, nr, io)
        else:
            fold_units_chunk(f, r0, nr, io)
    return begin, n, io.writes, io.reads


def fold_item(full, rank0, pitch, S, run, rows, es, gather, shift=14):
    """A fold item as the planner builds it (push_fold)."""
    CH = 1 << shift
    m = full | run | rank0 | pitch
    W = 16 if m % 16 == 0 else 8 if m % 8 == 0 else 4 if m % 4 == 0 else 2
    assert W >= es
    return (full, run, rows, CH // (S * run), rank0, pitch, S, W, int(gather), 0)


@pytest.mark.parametrize("S", [2, 3, 4, 8])
@pytest.mark.parametrize("run", [2, 6, 12, 16, 24, 48, 200])
@pytest.mark.parametrize("gather", [True, False])
def test_fold_items_cover_exactly(S, run, gather):
    """Every byte of the full tensor and of every rank's rows is moved
    exactly once, from the right place, with aligned units of every width."""
    es = 2 if run % 4 else 4
    rows = 1000 + S
    rng = np.random.default_rng(S * 100 + run)
    full = (1 << 40) + es * int(rng.integers(0, 8)) * (1 if run % 16 else 8)
    pitch = rows * run + es * int(rng.integers(0, 64))
    rank0 = (1 << 44) + es * int(rng.integers(0, 8))
    ranks = [rank0 + s * pitch for s in range(S)]
    f = fold_item(full, rank0, pitch, S, run, rows, es, gather)
    _, _, writes, reads = emulate_fold([f], 1 << 14, lds=False)
    for a, b, _ in writes:
        assert b - a == f[7]
    pairs = sorted(zip(writes, reads))
    full_iv = [(full, full + rows * S * run)]
    rank_iv = _merge([(b, b + rows * run) for b in ranks])
    w_iv = [(a, b) for (a, b, _), _ in pairs]
    r_iv = [(a, b) for _, (a, b, _) in pairs]
    assert _merge(w_iv) == (full_iv if gather else rank_iv)
    assert _merge(r_iv) == (rank_iv if gather else full_iv)
    assert sum(b - a for a, b in w_iv) == rows * S * run  # each byte once
    for (wa, wb, _), (ra, rb, _) in pairs:
        fa, raddr = (wa, ra) if gather else (ra, wa)
        r, rem = divmod(fa - full, S * run)
        s, x = divmod(rem, run)
        assert raddr == ranks[s] + r * run + x


# ---------------------------------------------------------------------------
# fold_reduce_kernel: the fused RS of short dim-k rows, one shard group per item
# ---------------------------------------------------------------------------

FOLD_RED_FMT = "<3Q4I3Q"  # run_bytes, rows, rows_per_chunk, src0, dst0, nrank, unit, reserved[3]


def fold_reduce_item(src, dst, run, rows, es, shift=13, copy_shift=14):
    """A fold-reduce item and its pointers as the planner builds them
    (push_fold_reduce: reduce-sized chunks, or copy-sized ones where a
    reduce chunk would hold one full row, or kFoldUnitChunk-sized ones of at
    least two rows where the kernel never stages them); None where the
    planner keeps other jobs."""
    CH, CHX = 1 << shift, 1 << max(shift, copy_shift)
    S = len(src)
    if not fold_rows(run, rows, S, CHX, 16):
        return None
    m = run
    for a in list(src) + list(dst):
        m |= a
    W = 16 if m % 16 == 0 else 8 if m % 8 == 0 else 4 if m % 4 == 0 else 2
    if W < es:
        return None
    if W > FOLD_LDS_MAX_UNIT and S < 4:  # never staged: kFoldUnitChunk bytes, at least two rows
        per = max(2, FOLD_UNIT_CHUNK // (S * run))
    else:
        per = CH // (S * run) if 2 * S * run <= CH else CHX // (S * run)
    return (run, rows, per, 0, S, S, W, 0, 0, 0), list(src) + list(dst)


def fold_reduce_lds_ok(f, ptr, r0, nr):
    """Does a fold-reduce chunk take the LDS path (fold_reduce_lds_ok)?"""
    run, rows, per, src0, dst0, S, W = f[:7]
    if W > FOLD_LDS_MAX_UNIT and S < 4:
        return False
    a = ptr[src0]
    if any((ptr[src0 + t] ^ a) & 15 for t in range(1, S)):
        return False
    F0 = a + r0 * S * run
    return ((F0 + nr * S * run + 15) & ~15) - (F0 & ~15) <= FOLD_LDS


def _sum_bytes(blocks, dtype):
    """The elementwise reduction of equal-length byte strings holding
    `dtype` values: summed in float32 in operand order from the first,
    rounded once to dtype (the kernels' arithmetic, SUM)."""
    vals = [np.frombuffer(b, dtype=dtype).astype(np.float32) for b in blocks]
    acc = vals[0].copy()
    with np.errstate(invalid="ignore", over="ignore"):  # edge-block bytes outside the rows may be any bits
        for v in vals[1:]:
            acc = acc + v
        return acc.astype(dtype).tobytes()


def emulate_fold_reduce(items, ptr, CH, io=None, lds=True, dtype=np.float32):
    """fold_reduce_kernel over a fold-reduce table: the chunk prefix, the
    chunk count, the writes as (lo, hi, item, operand offset or None) and
    the reads as (lo, hi, item).  Chunk k of item j is full-tensor rows
    [k*per, ...).  Unit path: unit q of a chunk is row q // upf, rank
    (q % upf) // upr, column q % upr; every operand is read at the chunk's
    offset + q units, the result written to rank s's dense rows.  LDS path
    (lds=True: 2- and 4-byte units, or wider in groups of 4 ranks or more;
    operands at one offset modulo 16): the
    operands' aligned blocks over the chunk are reduced into LDS, then every
    rank's rows are written in aligned vectors and element-wise ends."""
    io = io if io is not None else Recorder()
    begin, n = [], 0
    for f in items:
        begin.append(n)
        n += fold_item_chunks(f[1], f[2], f[5] * f[0], f[7])
    writes = []
    for c in range(n):
        j = find_item(begin, len(items), c)
        f = items[j]
        run, rows, per, src0, dst0, S, W = f[:7]
        if per == 0:  # flat chunks (fold_reduce_flat)
            io.item = j
            sub = f[7]
            assert W in (2, 4, 8, 16) and run % W == 0 and sub % 16 == 0
            assert all(((ptr[src0 + t] ^ ptr[src0]) & 15) == 0 for t in range(S))
            g = 4 if W >= 4 else 2
            X0, nb_, p_lo, off0, parts = flat_chunk(c - begin[j], rows * S * run, sub, run)
            F0 = ptr[src0] + X0
            fa = F0 & ~15
            nblk = (((F0 + nb_ + 15) & ~15) - fa) // 16
            assert nblk * 16 <= FOLD_LDS
            lds_mem = bytearray(nblk * 16)
            for i in range(nblk):
                blocks = [io.load(((ptr[src0 + t] + X0) & ~15) + 16 * i, 16) for t in range(S)]
                lds_mem[16 * i:16 * i + 16] = _sum_bytes(blocks, dtype) if io.mem is not None else bytes(16)

            def dst_addr(p, a, X0=X0):
                r, s_ = divmod(p, S)
                return ptr[dst0 + s_] + r * run + (X0 + a - p * run)

            _flat_scatter(parts, F0 - fa, lds_mem, g, dst_addr, io, writes, j)
            continue
        # never staged: kFoldUnitChunk bytes or two rows
        cap = max(FOLD_UNIT_CHUNK, 2 * S * run) if W > FOLD_LDS_MAX_UNIT and S < 4 else CH
        assert W in (2, 4, 8, 16) and run % W == 0 and per >= 1 and per * S * run <= cap
        assert all(ptr[k] % W == 0 for k in range(src0, src0 + S)) and all(ptr[k] % W == 0 for k in range(dst0, dst0 + S))
        r0 = (c - begin[j]) * per
        nr = min(per, rows - r0)
        assert nr * S * run < 1 << 32  # the kernel's 32-bit unit indices and offsets
        io.item = j
        FR, off = S * run, r0 * S * run
        if lds and fold_reduce_lds_ok(f, ptr, r0, nr):
            g = 4 if W >= 4 else 2
            F0 = ptr[src0] + off
            fa = F0 & ~15
            delta = F0 - fa
            nblk = (((F0 + nr * FR + 15) & ~15) - fa) // 16
            assert nblk * 16 <= FOLD_LDS
            lds_mem = bytearray(FOLD_LDS)
            for i in range(nblk):
                blocks = [io.load(((ptr[src0 + t] + off) & ~15) + 16 * i, 16) for t in range(S)]
                lds_mem[16 * i:16 * i + 16] = _sum_bytes(blocks, dtype) if io.mem is not None else bytes(16)
            for s_ in range(S):
                d = ptr[dst0 + s_] + r0 * run

                def src(y):
                    row, col = divmod(y, run)
                    o = delta + row * FR + s_ * run + col
                    assert o + g <= nblk * 16
                    return bytes(lds_mem[o:o + g])

                L = nr * run
                for v in range((d + 15) & ~15, (d + L) & ~15, 16):
                    io.store(v, b"".join(src(v - d + k) for k in range(0, 16, g)))
                    writes.append((v, v + 16, j, None))
                for lo, hi in _ends(d, d + L):
                    for y in range(lo, hi, g):
                        io.store(y, src(y - d))
                        writes.append((y, y + g, j, None))
            continue
        upr = run // W
        upf = S * upr
        for q in range(nr * upf):
            row, rem = divmod(q, upf)
            s_, col = divmod(rem, upr)
            so = off + q * W
            blocks = [io.load(ptr[src0 + t] + so, W) for t in range(S)]
            d = ptr[dst0 + s_] + (r0 + row) * run + col * W
            io.store(d, _sum_bytes(blocks, dtype) if io.mem is not None else bytes(W))
            writes.append((d, d + W, j, so))
    return begin, n, writes, io.reads


@pytest.mark.parametrize("S", [2, 3, 4, 8])
@pytest.mark.parametrize("run", [2, 4, 6, 12, 16, 24, 48, 200])
@pytest.mark.parametrize("es", [2, 4])
def test_fold_reduce_items_cover_exactly(S, run, es):
    """Every byte of every rank's rows is written exactly once, with the
    reduction of the operands' bytes at that rank's piece of the same full
    row and column, and every operand is read whole, once per unit."""
    if run % es:
        return
    rows = 700 + 3 * S
    rng = np.random.default_rng(S * 1000 + run * 10 + es)
    src = [(1 << 40) + t * (1 << 32) + es * int(rng.integers(0, 8)) for t in range(S)]
    dst = [(1 << 44) + s * (1 << 32) + es * int(rng.integers(0, 8)) for s in range(S)]
    made = fold_reduce_item(src, dst, run, rows, es)
    if made is None:
        assert not fold_rows(run, rows, S, 1 << 14, 16)
        return
    item, ptr = made
    W = item[6]
    _, _, writes, reads = emulate_fold_reduce([item], ptr, 1 << 14, lds=False)
    assert all(b - a == W for a, b, _, _ in writes)
    w_iv = [(a, b) for a, b, _, _ in writes]
    assert _merge(w_iv) == _merge([(d, d + rows * run) for d in dst])
    assert sum(b - a for a, b in w_iv) == S * rows * run  # each byte once
    for a, _, _, so in writes:
        r, rem = divmod(so, S * run)
        s, x = divmod(rem, run)
        assert a == dst[s] + r * run + x
    for t in range(S):
        r_t = [(a, b) for a, b, _ in reads if src[t] <= a < src[t] + rows * S * run]
        assert _merge(r_t) == [(src[t], src[t] + rows * S * run)]
        assert sum(b - a for a, b in r_t) == rows * S * run


def test_fold_reduce_unit_is_the_widest_common_alignment():
    """The unit divides the row and every pointer and is at least the
    element; a 2-byte alignment with 4-byte elements keeps interleaved jobs."""
    src = [1 << 40, (1 << 40) + 4096]
    dst = [1 << 44, (1 << 44) + 4096]
    assert fold_reduce_item(src, dst, 32, 100, 4)[0][6] == 16
    assert fold_reduce_item(src, [dst[0] + 8, dst[1]], 32, 100, 4)[0][6] == 8
    assert fold_reduce_item(src, dst, 12, 100, 4)[0][6] == 4
    assert fold_reduce_item([src[0] + 2, src[1]], dst, 12, 100, 2)[0][6] == 2
    assert fold_reduce_item([src[0] + 2, src[1]], dst, 12, 100, 4) is None
    assert fold_reduce_item(src[:1], dst[:1], 32, 100, 4) is None  # one rank: no fold
    assert fold_reduce_item(src, dst, 256, 100, 4) is None  # 256-byte rows at a multiple of 16: per-rank blocks
    assert fold_reduce_item(src, dst, 264, 100, 4)[0][6] == 8  # a multiple of 8 only: folded
    assert fold_reduce_item(src, dst, 770, 100, 2)[0][2] == (1 << 13) // (2 * 770)  # 8 KiB chunks
    assert fold_reduce_item(src, dst, 2052, 100, 2)[0][2] == (1 << 14) // (2 * 2052)  # one row per 8 KiB: 16 KiB


@pytest.mark.parametrize("S", [2, 3, 4, 8])
@pytest.mark.parametrize("run", [2, 4, 6, 8, 12, 16, 24, 40, 200])
@pytest.mark.parametrize("gather", [True, False])
@pytest.mark.parametrize("shift", [9, 14, 16])
def test_fold_moves_every_byte_to_its_place(S, run, gather, shift):
    """The byte-level emulation of fold_copy_kernel (both its LDS and its
    unit path, every chunk shape, bases at every unit alignment) turns the
    source image into exactly the expected one: full row r is the S ranks'
    rows r side by side, and no other byte of memory changes."""
    es = 2 if run % 4 else 4
    rows = 37 + 5 * S
    rng = np.random.default_rng(S * 7919 + run * 31 + gather * 3 + shift)
    size = 1 << 20
    mem = rng.integers(0, 256, size, dtype=np.uint8)
    full = 4096 + es * int(rng.integers(0, 16))
    rank0 = (1 << 18) + es * int(rng.integers(0, 16))
    pitch = rows * run + es * int(rng.integers(0, 40))
    f = fold_item(full, rank0, pitch, S, run, rows, es, gather, shift=shift)
    if f[3] < 1:
        return  # S*run above the chunk: the planner makes no fold item
    before = mem.copy()
    io = Recorder(mem)
    emulate_fold([f], 1 << shift, io)
    want = before.copy()
    for r in range(rows):
        for s_ in range(S):
            fa = full + (r * S + s_) * run
            ra = rank0 + s_ * pitch + r * run
            if gather:
                want[fa:fa + run] = before[ra:ra + run]
            else:
                want[ra:ra + run] = before[fa:fa + run]
    assert np.array_equal(mem, want)
    # every byte written once, reads inside the sources' aligned blocks
    w_iv = [(a, b) for a, b, _ in io.writes]
    assert sum(b - a for a, b in w_iv) == sum(b - a for a, b in _merge(w_iv))
    src = [(full, full + rows * S * run)] if not gather else [(rank0 + s_ * pitch, rank0 + s_ * pitch + rows * run)
                                                             for s_ in range(S)]
    env = _merge([(a & ~15, (b + 15) & ~15) for a, b in src])
    for a, b, _ in io.reads:
        assert any(x <= a and b <= y for x, y in env), (a, b)


@pytest.mark.parametrize("S", [2, 3, 4, 8])
@pytest.mark.parametrize("run", [2, 4, 6, 8, 12, 16, 40, 770, 2052])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
@pytest.mark.parametrize("same_offset", [True, False])
def test_fold_reduce_moves_sums_to_their_place(S, run, dtype, same_offset):
    """The byte-level emulation of fold_reduce_kernel (LDS path when the
    operands share their offset modulo 16, else the unit path) writes, for
    every rank s and row r, the sum over the group of the gradients' piece
    s of full row r, and changes no other byte."""
    es = np.dtype(dtype).itemsize
    if run % es:
        return
    rows = 29 + 7 * S if run < 256 else 9
    rng = np.random.default_rng(S * 131 + run * 7 + es + same_offset)
    n_el = rows * S * run // es
    span = (n_el * es + 64 + 4095) & ~4095  # per operand, and per destination region
    mem = rng.integers(0, 256, 4096 + 2 * S * span, dtype=np.uint8)
    src, dst = [], []
    for t in range(S):
        a = 4096 + t * span + (0 if same_offset else es * t) + 16 * int(rng.integers(0, 4))
        mem[a:a + n_el * es] = np.frombuffer(rng.integers(-50, 50, n_el).astype(dtype).tobytes(), np.uint8)
        src.append(a)
    for s_ in range(S):
        dst.append(4096 + (S + s_) * span + es * int(rng.integers(0, 16)))
    made = fold_reduce_item(src, dst, run, rows, es)
    if made is None:
        return
    item, ptr = made
    before = mem.copy()
    io = Recorder(mem)
    emulate_fold_reduce([item], ptr, 1 << 14, io, dtype=dtype)
    want = before.copy()
    for r in range(rows):
        for s_ in range(S):
            o = (r * S + s_) * run
            blocks = [bytes(before[a + o:a + o + run]) for a in src]
            d = dst[s_] + r * run
            want[d:d + run] = np.frombuffer(_sum_bytes(blocks, dtype), np.uint8)
    assert np.array_equal(mem, want)
    env = _merge([(a & ~15, (a + n_el * es + 15) & ~15) for a in src])
    for a, b, _ in io.reads:
        assert any(x <= a and b <= y for x, y in env), (a, b)


# ---------------------------------------------------------------------------
# flat chunks: dim-k rows too long for one chunk
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S", [2, 3, 4])
@pytest.mark.parametrize("run", [1028, 2052, 4100, 8196, 6150])
@pytest.mark.parametrize("gather", [True, False])
def test_flat_chunk_fold_moves_every_byte_to_its_place(S, run, gather):
    """Fold items of long rows (the S pieces of a full row exceed a chunk)
    are cut into flat chunks of the full tensor; their byte-level emulation turns the
    source image into exactly the expected one, writes every byte once and
    reads only the aligned blocks of the sources."""
    es = 2 if run % 4 else 4
    rows = 5
    rng = np.random.default_rng(S * 7 + run + gather)
    size = 1 << 21
    mem = rng.integers(0, 256, size, dtype=np.uint8)
    full = 4096 + es * int(rng.integers(0, 16))
    rank0 = (1 << 20) + es * int(rng.integers(0, 16))
    pitch = rows * run + es * int(rng.integers(0, 40))
    f = flat_fold_item(full, rank0, pitch, S, run, rows, es, gather)
    if f is None:
        assert S * run <= 1 << 14 or run % 8 == 0
        return
    before = mem.copy()
    io = Recorder(mem)
    emulate_fold([f], 1 << 14, io)
    want = before.copy()
    for r in range(rows):
        for s_ in range(S):
            fa = full + (r * S + s_) * run
            ra = rank0 + s_ * pitch + r * run
            if gather:
                want[fa:fa + run] = before[ra:ra + run]
            else:
                want[ra:ra + run] = before[fa:fa + run]
    assert np.array_equal(mem, want)
    w_iv = [(a, b) for a, b, _ in io.writes]
    assert sum(b - a for a, b in w_iv) == sum(b - a for a, b in _merge(w_iv)) == rows * S * run
    src = [(full, full + rows * S * run)] if not gather else [(rank0 + s_ * pitch, rank0 + s_ * pitch + rows * run)
                                                             for s_ in range(S)]
    env = _merge([(a & ~15, (b + 15) & ~15) for a, b in src])
    for a, b, _ in io.reads:
        assert any(x <= a and b <= y for x, y in env), (a, b)


@pytest.mark.parametrize("S", [2, 4])
@pytest.mark.parametrize("run", [4100, 8196])
@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_flat_chunk_fold_reduce_moves_sums_to_their_place(S, run, dtype):
    """Fold-reduce items of long rows (flat chunks): every rank's rows get
    the group's sum of their pieces, every byte once; no other byte changes."""
    es = np.dtype(dtype).itemsize
    rows = 4
    rng = np.random.default_rng(S * 13 + run + es)
    n_el = rows * S * run // es
    span = (n_el * es + 64 + 4095) & ~4095
    mem = rng.integers(0, 256, 4096 + 2 * S * span, dtype=np.uint8)
    src, dst = [], []
    for t in range(S):
        a = 4096 + t * span + 16 * int(rng.integers(0, 4))
        mem[a:a + n_el * es] = np.frombuffer(rng.integers(-50, 50, n_el).astype(dtype).tobytes(), np.uint8)
        src.append(a)
    for s_ in range(S):
        dst.append(4096 + (S + s_) * span + es * int(rng.integers(0, 16)))
    m = run
    for a in src + dst:
        m |= a
    W = 16 if m % 16 == 0 else 8 if m % 8 == 0 else 4 if m % 4 == 0 else 2
    item = (run, rows, 0, 0, S, S, W, FLAT_CHUNK, 0, 0)
    ptr = src + dst
    before = mem.copy()
    io = Recorder(mem)
    _, _, writes, reads = emulate_fold_reduce([item], ptr, 1 << 14, io, dtype=dtype)
    want = before.copy()
    for r in range(rows):
        for s_ in range(S):
            o = (r * S + s_) * run
            blocks = [bytes(before[a + o:a + o + run]) for a in src]
            d = dst[s_] + r * run
            want[d:d + run] = np.frombuffer(_sum_bytes(blocks, dtype), np.uint8)
    assert np.array_equal(mem, want)
    w_iv = [(a, b) for a, b, _, _ in writes]
    assert sum(b - a for a, b in w_iv) == sum(b - a for a, b in _merge(w_iv)) == rows * S * run
    env = _merge([(a & ~15, (a + n_el * es + 15) & ~15) for a in src])
    for a, b, _ in reads:
        assert any(x <= a and b <= y for x, y in env), (a, b)
