"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's formulas: they compare it with
hand-derived values of the pages' examples (tests/golden), with torch.chunk
(the library routine that implements the same ceil-chunk split), with
brute-force forward maps on tiny inputs, with exact integer sums, with a
float64 error bound, and with the group lists the pages print.  The
planted-mistake tests at the end show that a plausible slip in the oracle
fails at least one pin.
"""

import itertools

import numpy as np
import pytest
import torch

import oracle as O
from oracle import fsdp_oracle as F

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------
# pin helpers: each returns a list of failure strings (empty = pinned)
# ---------------------------------------------------------------------------

def pin_golden_dim0(golden):
    bad = []
    for c in golden["dim0"]:
        lay = O.bucket_layout([tuple(c["shape"])], c["shard_size"])
        got = (lay.chunk_rows[0], lay.row_off[0], lay.row_len[0], lay.padded[0])
        want = (c["chunk_rows"], c["row_off"], c["row_len"], c["padded"])
        if got != want:
            bad.append(f"{c['shape']} S={c['shard_size']}: {got} != {want}")
    for b in golden["buckets"]:
        lay = O.bucket_layout([tuple(s) for s in b["shapes"]], b["shard_size"])
        if (lay.in_off, lay.I) != (b["in_off"], b["I"]):
            bad.append(f"bucket {b['shapes']}: {(lay.in_off, lay.I)}")
    return bad


def pin_torch_chunk(max_n0=40, max_s=9):
    """Non-empty shards equal torch.chunk's pieces, in order; the rest are empty."""
    bad = []
    for n0 in range(0, max_n0 + 1):
        x = torch.arange(n0 * 3).reshape(n0, 3)
        for S in range(1, max_s + 1):
            lay = O.bucket_layout([(n0, 3)], S)
            shards = O.shard_params([x.numpy()], lay)
            pieces = [p.numpy() for p in torch.chunk(x, S, dim=0)] if n0 > 0 else []
            nonempty = [sh[0] for sh in shards if sh[0].shape[0] > 0]
            if len(nonempty) != len(pieces) or any(
                    not np.array_equal(a, b) for a, b in zip(nonempty, pieces)):
                bad.append(f"n0={n0} S={S}")
            # empty shards all come after the non-empty ones
            lens = [sh[0].shape[0] for sh in shards]
            if lens != sorted(lens, reverse=True):
                bad.append(f"n0={n0} S={S}: lengths {lens} not non-increasing")
            if lay.chunk_rows[0] != (pieces[0].shape[0] if pieces else 0):
                bad.append(f"n0={n0} S={S}: chunk rows {lay.chunk_rows[0]}")
    return bad


def forward_map_ag(params, lay):
    """Brute force: every element (r, c) of parameter i goes to the unique
    rank whose rows contain r, at its row-within-shard; everything else 0."""
    S, I = lay.S, lay.I
    want = [None] * (S * I)
    for i, x in enumerate(params):
        x2 = x.reshape(x.shape[0], lay.inner[i])
        for r in range(x2.shape[0]):
            owners = [s for s in range(S) if lay.row_off[i][s] <= r < lay.row_off[i][s] + lay.row_len[i][s]]
            assert len(owners) == 1
            s = owners[0]
            for c in range(x2.shape[1]):
                pos = s * I + lay.in_off[i] + (r - lay.row_off[i][s]) * lay.inner[i] + c
                assert want[pos] is None
                want[pos] = x2[r, c]
    return want


def pin_ag_bruteforce(dtype=np.float32, max_s=9):
    bad = []
    for S in range(1, max_s + 1):
        for inner in (1, 2, 3, 5, 8):
            for n0 in range(0, 3 * S + 3):
                shape = (n0,) if inner == 1 else (n0, inner)
                x = (RNG.standard_normal(shape) * 100).astype(np.float32)
                if dtype == np.uint16:
                    x = x.view(np.uint32).astype(np.uint16)  # arbitrary bit patterns
                lay = O.bucket_layout([shape], S)
                ag = O.ag_copy_in(O.shard_params([x], lay), lay, x.dtype)
                want = forward_map_ag([x], lay)
                for p, w in enumerate(want):
                    v = ag[p]
                    if (w is None and v != 0) or (w is not None and v != w):
                        bad.append(f"S={S} shape={shape} pos={p}")
                        break
                full = O.ag_copy_out(O.all_gather(ag), lay)[0]
                if full.shape != x.shape or not np.array_equal(full.view(np.uint8), x.view(np.uint8)):
                    bad.append(f"roundtrip S={S} shape={shape}")
    return bad


def pin_ag_multiparam():
    """all_gather(shard(x)) == x for mixed buckets, and every padding element is 0."""
    bad = []
    shape_pool = [(7, 8), (5, 3), (16,), (3,), (1, 5), (0, 2), (9,), (2, 2, 3), (13, 1)]
    for S in (1, 2, 3, 4, 5, 8):
        for k in range(4):
            idx = RNG.choice(len(shape_pool), size=4, replace=True)
            shapes = [shape_pool[j] for j in idx]
            xs = [(RNG.standard_normal(sh) + 3).astype(np.float32) for sh in shapes]  # nonzero
            lay = O.bucket_layout(shapes, S)
            ag = O.ag_copy_in(O.shard_params(xs, lay), lay, np.float32)
            outs = O.ag_copy_out(O.all_gather(ag), lay)
            if any(not np.array_equal(a, b) for a, b in zip(outs, xs)):
                bad.append(f"roundtrip {shapes} S={S}")
            n_data = sum(x.size for x in xs)
            if int(np.count_nonzero(ag)) != n_data or ag.size != S * sum(lay.padded):
                bad.append(f"padding {shapes} S={S}")
            want = forward_map_ag(xs, lay)
            got_zero = [p for p, w in enumerate(want) if w is None]
            if np.any(ag[got_zero] != 0):
                bad.append(f"pad positions {shapes} S={S}")
    return bad


def textbook_rs(grads_int, shapes, members, s, S):
    """Exact reduce-scatter: chunk s (torch.chunk) of the int64 sum over members."""
    out = []
    for i, sh in enumerate(shapes):
        tot = sum(torch.as_tensor(grads_int[m][i]).to(torch.int64) for m in members)
        pieces = torch.chunk(tot, S, dim=0) if sh[0] > 0 else []
        out.append(pieces[s] if s < len(pieces) else torch.zeros((0,) + tuple(sh[1:]), dtype=torch.int64))
    return out


def _fold_operands(n_ops, n, seed):
    """n_ops float32 arrays of n values over twelve decades (sums of them are
    not exact, so their bits depend on the order of the additions), with
    every operand -0.0 at the first four positions (only a fold that starts
    from the first operand keeps -0.0 there)."""
    rng = np.random.default_rng(seed)
    ops = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6, n)).astype(np.float32) for _ in range(n_ops)]
    for x in ops:
        x[:4] = np.float32(-0.0)
    return ops


def _left_fold(ops):
    """NumPy's float32 add.accumulate over the operands in the listed order:
    out[k] = out[k-1] + ops[k], the sequential fold by the ufunc's definition."""
    return np.add.accumulate(np.stack(ops), axis=0, dtype=np.float32)[-1]


def pin_fold_order(R, S, op, n=2048, seed=7):
    """The fixed rank order: every RS and fused-AR output is, bit for bit,
    the ascending-rank left fold of its group's operands in float32 (a
    different routine from the oracle's loop), then for AVG one float32
    division by the group size.  Catches a reversed or tree-shaped order and
    a fold started from +0.0."""
    bad = []
    D = R // S
    I = n
    rs_in = _fold_operands(R, S * I, seed)
    outs = O.rs_reduce(rs_in, I, R, S, op)
    for g in range(R):
        d, s = divmod(g, S)
        want = _left_fold([rs_in[d * S + t][s * I:(s + 1) * I] for t in range(S)])
        if op == O.AVG:
            want = np.divide(want, np.float32(S), dtype=np.float32)
        if not np.array_equal(outs[g].view(np.int32), want.view(np.int32)):
            bad.append(f"RS fold order R={R} S={S} {op} g={g}")
    fused = _fold_operands(R, I, seed + 1)
    outs = O.fused_ar(fused, R, S, op)
    for g in range(R):
        s = g % S
        want = _left_fold([fused[d * S + s] for d in range(D)])
        if op == O.AVG:
            want = np.divide(want, np.float32(D), dtype=np.float32)
        if not np.array_equal(outs[g].view(np.int32), want.view(np.int32)):
            bad.append(f"AR fold order R={R} S={S} {op} g={g}")
    return bad


def pin_rs_exact(R, S, op, shapes, bf16=False):
    """Integer-valued gradients in [-8, 8]: every partial sum is exact in
    float32 and in bfloat16 (|sum| <= 64 < 2**8), whatever the order."""
    bad = []
    D = R // S
    gi = [[RNG.integers(-8, 9, size=sh).astype(np.float32) for sh in shapes] for _ in range(R)]
    lay = O.bucket_layout(shapes, S)
    if bf16:
        gb = [[torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16) for x in row]
              for row in gi]
        rs_in = [O.rs_copy_in(gb[g], lay, np.uint16) for g in range(R)]
        outs = [O.bf16_to_f32(o) for o in O.rs_reduce(rs_in, lay.I, R, S, op)]
    else:
        rs_in = [O.rs_copy_in(gi[g], lay) for g in range(R)]
        outs = O.rs_reduce(rs_in, lay.I, R, S, op)
    for g in range(R):
        d, s = divmod(g, S)
        members = list(range(d * S, d * S + S))
        want = textbook_rs(gi, shapes, members, s, S)
        for i in range(len(shapes)):
            got = O.sharded_grad(outs[g], lay, i, s)
            w = want[i].to(torch.float64).numpy() / (S if op == O.AVG else 1)
            if got.shape != w.shape or not np.array_equal(got.astype(np.float64), w):
                bad.append(f"RS R={R} S={S} {op} g={g} param={i}")
        # padding of the RS output is zero (a zero-padded input reduces to zero)
        mask = np.ones(lay.I, bool)
        for i in range(len(shapes)):
            a = lay.in_off[i]
            mask[a:a + lay.row_len[i][s] * lay.inner[i]] = False
        if np.any(outs[g][mask] != 0):
            bad.append(f"RS padding g={g}")
    return bad


def pin_end_to_end_exact(R, S, op, shapes, buckets=None):
    """After RS then AR, rank (d, s) holds chunk s of the sum over all R ranks
    (SUM) or that sum over R (AVG; exact for power-of-two S and D)."""
    bad = []
    gi = [[RNG.integers(-8, 9, size=sh).astype(np.float32) for sh in shapes] for _ in range(R)]
    buckets = buckets or [shapes]
    res, fused, offs, lays = O.reduce_grads_fused(gi, buckets, R, S, op)
    for g in range(R):
        s = g % S
        want = textbook_rs(gi, shapes, list(range(R)), s, S)
        for i in range(len(shapes)):
            w = want[i].to(torch.float64).numpy() / (R if op == O.AVG else 1)
            got = res[g][i].astype(np.float64)
            if got.shape != w.shape or not np.array_equal(got, w):
                bad.append(f"e2e R={R} S={S} {op} g={g} param={i}")
    return bad


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------

def test_golden_dim0_and_bucket(golden):
    assert pin_golden_dim0(golden) == []


def test_chunk_matches_torch_chunk():
    assert pin_torch_chunk() == []


def test_chunk_differs_from_array_split():
    # np.array_split balances the remainder over the first ranks (2,1,1,1);
    # the pages' fixed-size chunking gives (2,2,1,0).
    _, _, lens = O.dim0_chunk(5, 4)
    assert lens == [2, 2, 1, 0]
    assert [len(a) for a in np.array_split(np.arange(5), 4)] == [2, 1, 1, 1]


def test_chunk_invariants():
    for n0, S in itertools.product(range(0, 70), range(1, 17)):
        chunk, offs, lens = O.dim0_chunk(n0, S)
        assert sum(lens) == n0
        assert all(0 <= n <= chunk for n in lens)
        assert offs[0] == 0 and all(offs[s + 1] == offs[s] + lens[s] for s in range(S - 1))
        partial = [n for n in lens if 0 < n < chunk]
        assert len(partial) <= 1
        assert chunk * S >= n0 and (chunk - 1) * S < n0 or n0 == 0
        if n0 % S == 0:  # even parameter: no padding at all
            assert chunk * S == n0 and all(n == chunk for n in lens)


def test_ag_bruteforce_fp32():
    assert pin_ag_bruteforce(np.float32, max_s=9) == []


def test_ag_bruteforce_bf16_bits():
    assert pin_ag_bruteforce(np.uint16, max_s=5) == []


def test_ag_multiparam_roundtrip_and_padding():
    assert pin_ag_multiparam() == []


def test_single_parameter_gather_prefix_is_the_parameter():
    """Zero-copy AG ('option 2' of the Hyper PR write-up): in a one-parameter
    bucket the first N elements of the gathered buffer are the full
    parameter, because fixed-size chunking leaves every padding element
    after the last data row.  Brute force over shapes and shard counts."""
    for S in range(1, 10):
        for n0 in range(0, 3 * S + 4):
            for inner in (1, 3):
                shape = (n0, inner)
                x = (RNG.standard_normal(shape) + 5).astype(np.float32)
                lay = O.bucket_layout([shape], S)
                ag = O.ag_copy_in(O.shard_params([x], lay), lay, np.float32)
                assert np.array_equal(ag[:x.size], x.reshape(-1))
                assert not np.any(ag[x.size:])  # the rest is padding


@pytest.mark.parametrize("R,S", [(4, 4), (8, 4), (8, 8), (8, 2), (6, 3)])
@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_rs_exact_integer_sums(R, S, op):
    if op == O.AVG and S & (S - 1):
        pytest.skip("division by a non-power-of-two is not exact")
    assert pin_rs_exact(R, S, op, [(7, 8), (5, 3), (16,), (3,), (11, 2)]) == []


@pytest.mark.parametrize("R,S", [(4, 4), (8, 4), (8, 8), (8, 2), (6, 3)])
@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_rs_exact_integer_sums_bf16(R, S, op):
    if op == O.AVG and S & (S - 1):
        pytest.skip("division by a non-power-of-two is not exact")
    assert pin_rs_exact(R, S, op, [(7, 8), (5, 3), (16,), (3,), (11, 2)], bf16=True) == []


def _bf16_special_values():
    rng = np.random.default_rng(77)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(2000) * 1e-40).astype(np.float32),          # denormals
            np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 3.3895314e38, -3.3895314e38,
                      3.4028235e38, 1.0, -1.0, 1e-45, -1e-45], dtype=np.float32)]
    # exact ties: a kept part with each parity and the dropped half exactly 0x8000
    top = rng.integers(0, 0x7F7F, size=2000).astype(np.uint32)
    vals.append(((top << 16) | 0x8000).view(np.float32))
    vals.append(((top << 16) | 0x7FFF).view(np.float32))
    vals.append(((top << 16) | 0x8001).view(np.float32))
    return np.concatenate(vals)


def test_bf16_conversions_match_torch():
    x = _bf16_special_values()
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f32_to_bf16(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0)
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_to_f32(bits).view(np.uint32), back.view(np.uint32))


def pin_bf16_round_once():
    """bf16 RS = round_to_bf16(float32 ordered sum of the widened operands),
    checked against torch's float32 arithmetic and its bf16 rounding."""
    bad = []
    R, S = 8, 4
    shapes = [(33, 7), (10,)]
    lay = O.bucket_layout(shapes, S)
    gen = torch.Generator().manual_seed(5)
    gi = [[torch.randn(sh, generator=gen).to(torch.bfloat16) for sh in shapes] for _ in range(R)]
    rs_in = [O.rs_copy_in([t.view(torch.int16).numpy().view(np.uint16) for t in gi[g]], lay, np.uint16)
             for g in range(R)]
    for op in (O.SUM, O.AVG):
        outs = O.rs_reduce(rs_in, lay.I, R, S, op)
        for g in range(R):
            d, s = divmod(g, S)
            acc = torch.from_numpy(rs_in[d * S][s * lay.I:(s + 1) * lay.I].view(np.int16)).view(torch.bfloat16).float()
            for t in range(1, S):
                acc = acc + torch.from_numpy(rs_in[d * S + t][s * lay.I:(s + 1) * lay.I].view(np.int16)).view(torch.bfloat16).float()
            if op == O.AVG:
                acc = acc / S
            want = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            if not np.array_equal(outs[g], want):
                bad.append(f"bf16 RS {op} rank {g}")
    return bad


def test_bf16_reductions_round_once():
    assert pin_bf16_round_once() == []


def pin_f16_round_once():
    """fp16 RS = round_to_fp16(float32 ordered sum of the widened operands),
    checked against torch's float32 arithmetic and its fp16 rounding, with
    sums that overflow fp16 and results in its denormal range."""
    bad = []
    R, S = 8, 4
    shapes = [(33, 7), (10,)]
    lay = O.bucket_layout(shapes, S)
    gen = torch.Generator().manual_seed(6)
    scale = [1.0, 3e4, 1e-5]  # ordinary, overflowing, denormal results
    gi = [[(torch.randn(sh, generator=gen) * scale[(g + i) % 3]).half() for i, sh in enumerate(shapes)]
          for g in range(R)]
    rs_in = [O.rs_copy_in([t.numpy() for t in gi[g]], lay, np.float16) for g in range(R)]
    with np.errstate(all="ignore"):
        for op in (O.SUM, O.AVG):
            outs = O.rs_reduce(rs_in, lay.I, R, S, op)
            for g in range(R):
                d, s = divmod(g, S)
                acc = torch.from_numpy(rs_in[d * S][s * lay.I:(s + 1) * lay.I]).float()
                for t in range(1, S):
                    acc = acc + torch.from_numpy(rs_in[d * S + t][s * lay.I:(s + 1) * lay.I]).float()
                if op == O.AVG:
                    acc = acc / S
                want = acc.half().numpy()
                if outs[g].dtype != np.float16 or not np.array_equal(outs[g].view(np.uint16), want.view(np.uint16)):
                    bad.append(f"fp16 RS {op} rank {g}")
    return bad


def test_f16_reductions_round_once():
    assert pin_f16_round_once() == []


def test_f16_conversion_matches_torch():
    x = _bf16_special_values()
    x = np.concatenate([x, np.array([65504.0, 65519.99, 65520.0, 7e4, -7e4, 6e-8, 3e-8, 2.98e-8], np.float32)])
    # exact fp16 ties in the normal range: 13 dropped bits equal to 0x1000
    top = np.random.default_rng(3).integers(0, 0x0F00, size=4000).astype(np.uint32)
    x = np.concatenate([x, (((top << 13) | 0x1000) + 0x38000000).astype(np.uint32).view(np.float32)])
    with np.errstate(all="ignore"):
        got = O.fsdp_oracle._store(x, np.zeros(1, np.float16))
    want = torch.from_numpy(x.copy()).half().numpy()
    nan = np.isnan(x)
    assert np.array_equal(got[~nan].view(np.uint16), want[~nan].view(np.uint16))
    assert np.all(np.isnan(got[nan]))


def pin_avg_correctly_rounded():
    """AVG over a group of 3 or 6 (not a power of two) on integer-valued
    gradients: the sum is exact, so the result must be the exact quotient
    rounded once to float32 (the quotient of an integer by 3 is never a
    float32 tie, so rounding the float64 quotient is rounding the exact
    one)."""
    from fractions import Fraction
    bad = []
    for R, S in ((6, 3), (6, 6), (12, 3)):
        shapes = [(7, 8), (5, 3), (40,)]
        lay = O.bucket_layout(shapes, S)
        gi = [[RNG.integers(-9, 10, size=sh).astype(np.float32) for sh in shapes] for _ in range(R)]
        rs_in = [O.rs_copy_in(gi[g], lay) for g in range(R)]
        outs = O.rs_reduce(rs_in, lay.I, R, S, O.AVG)
        for g in range(R):
            d, s = divmod(g, S)
            tot = sum(rs_in[m][s * lay.I:(s + 1) * lay.I].astype(np.int64) for m in range(d * S, d * S + S))
            want = np.array([float(Fraction(int(v), S)) for v in tot], dtype=np.float64).astype(np.float32)
            if not np.array_equal(outs[g].view(np.uint32), want.view(np.uint32)):
                bad.append(f"AVG/{S} rank {g}")
    return bad


def test_avg_over_non_power_of_two_is_correctly_rounded():
    assert pin_avg_correctly_rounded() == []


@pytest.mark.parametrize("R,S", [(8, 4), (8, 1), (4, 4), (8, 2), (2, 1)])
@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_end_to_end_exact_integer_sums(R, S, op):
    shapes = [(7, 8), (5, 3), (16,), (3,), (9, 4)]
    assert pin_end_to_end_exact(R, S, op, shapes) == []
    # the same result with one bucket per parameter (several fused segments)
    assert pin_end_to_end_exact(R, S, op, shapes, buckets=[[s] for s in shapes]) == []


@pytest.mark.parametrize("R,S", [(8, 8), (8, 4), (8, 2), (6, 3), (8, 1)])
@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_reductions_are_the_ascending_rank_fold(R, S, op):
    assert pin_fold_order(R, S, op) == []


def test_fold_order_inputs_tell_orders_apart():
    """The pin's inputs are sensitive: the reversed fold and a pairwise tree
    give other bits at many positions, and a fold from +0.0 loses -0.0."""
    ops = _fold_operands(8, 2048, 7)
    fwd = _left_fold(ops)
    assert np.count_nonzero(fwd.view(np.int32) != _left_fold(ops[::-1]).view(np.int32)) > 100
    tree = ((ops[0] + ops[1]) + (ops[2] + ops[3])) + ((ops[4] + ops[5]) + (ops[6] + ops[7]))
    assert np.count_nonzero(fwd.view(np.int32) != tree.view(np.int32)) > 100
    assert np.all(np.signbit(fwd[:4])) and not np.any(np.signbit(np.float32(0.0) + fwd[:4]))


def test_float64_error_bound():
    """Non-integer float32 sums: within the float32 rounding bound of the
    exact (float64) result, whatever the summation order."""
    shapes = [(33, 7), (10,), (5, 3)]
    for R, S in ((8, 4), (8, 8), (16, 16)):
        gi = [[RNG.standard_normal(sh).astype(np.float32) for sh in shapes] for _ in range(R)]
        lay = O.bucket_layout(shapes, S)
        rs_in = [O.rs_copy_in(gi[g], lay) for g in range(R)]
        for op in (O.SUM, O.AVG):
            outs = O.rs_reduce(rs_in, lay.I, R, S, op)
            for g in range(R):
                d, s = divmod(g, S)
                xs = np.stack([rs_in[m][s * lay.I:(s + 1) * lay.I].astype(np.float64)
                               for m in range(d * S, d * S + S)])
                exact = xs.sum(0) / (S if op == O.AVG else 1)
                bound = (S - 1) * 2.0 ** -24 * np.abs(xs).sum(0) / (S if op == O.AVG else 1) \
                    + 2.0 ** -24 * np.abs(exact) + 1e-45
                assert np.all(np.abs(outs[g].astype(np.float64) - exact) <= bound)


def test_avg_is_sum_divided_by_replicate_size():
    R, S = 8, 2
    D = R // S
    fused = [RNG.standard_normal(640).astype(np.float32) for _ in range(R)]
    a = O.fused_ar(fused, R, S, O.AVG)
    b = O.fused_ar(fused, R, S, O.SUM)
    for g in range(R):
        assert np.array_equal(a[g].view(np.uint32), (b[g] / np.float32(D)).view(np.uint32))
        assert np.array_equal(a[g], a[g % S])  # every replica holds the result


@pytest.mark.parametrize("R,S", [(8, 4), (8, 1), (4, 4), (8, 2), (6, 2)])
@pytest.mark.parametrize("op", [O.SUM, O.AVG])
def test_fused_equals_nonfused_bitwise(R, S, op):
    shapes = [(7, 8), (5, 3), (16,), (3,), (130,), (9, 4)]
    gi = [[RNG.standard_normal(sh).astype(np.float32) for sh in shapes] for _ in range(R)]
    nf = O.reduce_grads_nonfused(gi, shapes, R, S, op)
    for buckets in ([shapes], [shapes[:2], shapes[2:]], [[s] for s in shapes]):
        fu, fused, offs, _ = O.reduce_grads_fused(gi, buckets, R, S, op)
        for g in range(R):
            for i in range(len(shapes)):
                assert fu[g][i].shape == nf[g][i].shape
                assert np.array_equal(fu[g][i].view(np.uint32), nf[g][i].view(np.uint32))
        for o in offs:
            assert (o * 4) % 512 == 0
        assert (fused[0].size * 4) % 512 == 0


def test_group_lists_and_decision_matrix(golden):
    for c in golden["groups"]:
        assert O.group_sizes(c["rank_size"], c["shard_size"]) == (c["shard_size"], c["dp_size"])
        got = [[k, g] for k, g in O.grad_sync_plan(c["rank_size"], c["shard_size"])]
        assert got == c["calls"], c["why"]
    # every rank is in exactly one shard group and one replicate group, and
    # a shard group and a replicate group meet in exactly one rank
    for R, S in ((8, 4), (8, 2), (16, 4), (6, 3)):
        sg, rg = O.shard_groups(R, S), O.replicate_groups(R, S)
        assert sorted(sum(sg, [])) == list(range(R)) == sorted(sum(rg, []))
        assert all(len(set(a) & set(b)) == 1 for a in sg for b in rg)


def pin_fused_layout(golden):
    return ["fused " + c["why"] for c in golden["fused"]
            if list(O.fused_layout(c["seg_numel"], c["elem_bytes"])) != [c["offsets"], c["F"]]]


def test_fused_layout_golden(golden):
    assert pin_fused_layout(golden) == []
    sizes = [int(v) for v in RNG.integers(0, 3000, size=200)]
    offs, Fn = O.fused_layout(sizes)
    end = 0
    for o, n in zip(offs, sizes):
        assert o * 4 % 512 == 0 and o >= end and o * 4 - end * 4 < 512
        end = o + n
    assert Fn * 4 % 512 == 0 and Fn >= end and (Fn - end) * 4 < 512


def test_oracle_rejects():
    with pytest.raises(NotImplementedError):  # uneven on a non-zero dim
        O.bucket_layout([(4, 3)], 2, shard_dim=1)
    with pytest.raises(ValueError):  # no such dim
        O.bucket_layout([(4,)], 2, shard_dim=1)
    with pytest.raises(ValueError):
        O.bucket_layout([()], 2)
    with pytest.raises(ValueError):
        O.group_sizes(8, 3)
    with pytest.raises(ValueError):
        O.group_sizes(8, 0)


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin
# ---------------------------------------------------------------------------

def _floor_chunk(n0, S):
    chunk = max(n0 // S, 1) if n0 else 0
    offs = [min(s * chunk, n0) for s in range(S)]
    lens = [min(chunk, n0 - o) if s < S - 1 else n0 - o for s, o in enumerate(offs)]
    return chunk, offs, lens


def _array_split_chunk(n0, S):
    lens = [len(a) for a in np.array_split(np.arange(n0), S)]
    offs = list(np.cumsum([0] + lens[:-1]))
    return max(lens), [int(o) for o in offs], lens


def _head_padding_copy_in(shards, lay, dtype):
    ag = np.zeros(lay.S * lay.I, dtype=dtype)
    for s in range(lay.S):
        for i in range(len(lay.shapes)):
            flat = np.ascontiguousarray(shards[s][i]).reshape(-1)
            end = s * lay.I + lay.in_off[i] + lay.padded[i]
            ag[end - flat.size:end] = flat
    return ag


_ORIG_RS_REDUCE = F.rs_reduce
_ORIG_BUCKET_LAYOUT = F.bucket_layout


def _avg_over_rank_size(rs_in, I, R, S, op):
    outs = _ORIG_RS_REDUCE(rs_in, I, R, S, F.SUM)
    return [o / np.float32(R) for o in outs] if op == F.AVG else outs


def _drop_last_operand(operands):
    acc = np.array(operands[0], dtype=np.float32, copy=True)
    for x in operands[1:-1]:
        acc = acc + x
    return acc


def _transposed_replicate_groups(R, S):
    _, D = F.group_sizes(R, S)
    return [[s * D + d for d in range(D)] for s in range(S)]


def _unpadded_bucket_layout(shapes, S, shard_dim=0):
    lay = _ORIG_BUCKET_LAYOUT(shapes, S, shard_dim)
    off = 0
    for i, sh in enumerate(lay.shapes):
        lay.in_off[i] = off
        off += sh[0] * lay.inner[i] // S if sh[0] >= S else lay.padded[i]
    return lay


def _truncating_bf16(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _avg_by_reciprocal(acc, op, n):
    return acc * np.float32(1.0 / n) if op == F.AVG else acc


def _round_each_add(operands):
    bf = operands[0].dtype == np.uint16
    acc = np.array(F._as_f32(operands[0]), dtype=np.float32, copy=True)
    for x in operands[1:]:
        acc = acc + F._as_f32(x)
        if bf:
            acc = F.bf16_to_f32(F.f32_to_bf16(acc))
    return acc


def _f16_round_each_add(operands):
    f16 = operands[0].dtype == np.float16
    acc = np.array(F._as_f32(operands[0]), dtype=np.float32, copy=True)
    for x in operands[1:]:
        acc = acc + F._as_f32(x)
        if f16:
            acc = acc.astype(np.float16).astype(np.float32)
    return acc


_ORIG_STORE = F._store


def _f16_truncating_store(acc, like):
    if like.dtype == np.float16:
        # drop the 13 low mantissa bits (round toward zero in magnitude)
        b = np.asarray(acc, np.float32).view(np.uint32) & np.uint32(0xFFFFE000)
        return b.view(np.float32).astype(np.float16)
    return _ORIG_STORE(acc, like)


def _chunk_on_dim0(x, lay, i, s):
    a, n = lay.row_off[i][s], lay.row_len[i][s]
    return x[a:a + n]


def _fused_align_256(seg_numel, elem_bytes=4, align_bytes=512):
    return _ORIG_FUSED_LAYOUT(seg_numel, elem_bytes, 256)


_ORIG_FUSED_LAYOUT = F.fused_layout
_ORIG_RS_COPY_IN = F.rs_copy_in


def _rs_copy_in_pad_one(grads, lay, dtype=np.float32):
    buf = _ORIG_RS_COPY_IN(grads, lay, dtype)
    data = np.zeros(buf.size, bool)
    for i in range(len(lay.shapes)):
        for s in range(lay.S):
            a = s * lay.I + lay.in_off[i]
            data[a:a + lay.row_len[i][s] * lay.inner[i] * lay.outer[i]] = True
    buf[~data] = 1
    return buf


def _replicate_major_shard_groups(R, S):
    # the shard group of replicate d read as ranks d, D + d, 2D + d, ...
    _, D = F.group_sizes(R, S)
    return [[s * D + d for s in range(S)] for d in range(D)]


def _rs_avg_over_dp_size(rs_in, I, R, S, op):
    outs = _ORIG_RS_REDUCE(rs_in, I, R, S, F.SUM)
    return [o / np.float32(R // S) for o in outs] if op == F.AVG else outs


def _rs_slice_at_replicate_index(rs_in, I, R, S, op):
    # every rank of shard group d keeps slice d instead of its own slice s
    out = [None] * R
    for d, group in enumerate(F.shard_groups(R, S)):
        for g in group:
            operands = [rs_in[m][d * I:(d + 1) * I] for m in group]
            out[g] = F._store(F._scale(F._ordered_sum(operands), op, S), rs_in[group[0]])
    return out


_ORIG_FUSED_AR = F.fused_ar


def _descending_sum(operands):
    return _ORIG_ORDERED_SUM(list(operands)[::-1])


def _pairwise_sum(operands):
    ops = [F._as_f32(x).astype(np.float32) for x in operands]
    while len(ops) > 1:
        ops = [ops[k] + ops[k + 1] if k + 1 < len(ops) else ops[k] for k in range(0, len(ops), 2)]
    return ops[0]


def _zero_start_sum(operands):
    acc = np.zeros_like(F._as_f32(operands[0]), dtype=np.float32)
    for x in operands:
        acc = acc + F._as_f32(x)
    return acc


_ORIG_ORDERED_SUM = F._ordered_sum


def _ar_avg_over_shard_size(fused, R, S, op):
    outs = _ORIG_FUSED_AR(fused, R, S, F.SUM)
    return [o / np.float32(S) for o in outs] if op == F.AVG else outs


MUTANTS = {
    "bf16_truncation": ("f32_to_bf16", _truncating_bf16),
    "floor_chunk": ("dim0_chunk", _floor_chunk),
    "array_split": ("dim0_chunk", _array_split_chunk),
    "head_padding": ("ag_copy_in", _head_padding_copy_in),
    "avg_over_R": ("rs_reduce", _avg_over_rank_size),
    "dropped_term": ("_ordered_sum", _drop_last_operand),
    "rank_mapping": ("replicate_groups", _transposed_replicate_groups),
    "offset_by_actual": ("bucket_layout", _unpadded_bucket_layout),
    "avg_by_reciprocal": ("_scale", _avg_by_reciprocal),
    "bf16_round_each_add": ("_ordered_sum", _round_each_add),
    "chunk_on_dim0": ("_chunk", _chunk_on_dim0),
    "fused_align_256": ("fused_layout", _fused_align_256),
    "rs_padding_not_zero": ("rs_copy_in", _rs_copy_in_pad_one),
    "f16_round_each_add": ("_ordered_sum", _f16_round_each_add),
    "f16_truncating_store": ("_store", _f16_truncating_store),
    "rs_groups_replicate_major": ("shard_groups", _replicate_major_shard_groups),
    "rs_avg_over_dp_size": ("rs_reduce", _rs_avg_over_dp_size),
    "rs_slice_at_replicate_index": ("rs_reduce", _rs_slice_at_replicate_index),
    "ar_avg_over_shard_size": ("fused_ar", _ar_avg_over_shard_size),
    "descending_rank_order": ("_ordered_sum", _descending_sum),
    "pairwise_tree_sum": ("_ordered_sum", _pairwise_sum),
    "fold_from_zero": ("_ordered_sum", _zero_start_sum),
}


def _bf16_pin():
    x = _bf16_special_values()
    ok = ~np.isnan(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bool(np.array_equal(O.f32_to_bf16(x)[ok], want[ok]))


def _groups_pin(golden):
    return ["groups %s" % c["why"] for c in golden["groups"]
            if [[k, g] for k, g in O.grad_sync_plan(c["rank_size"], c["shard_size"])] != c["calls"]]


def _all_pins(golden):
    """Run every pin; a pin that raises counts as failed (and is named)."""
    pins = [
        lambda: pin_golden_dim0(golden),
        lambda: pin_torch_chunk(max_n0=12, max_s=5),
        lambda: pin_ag_bruteforce(np.float32, max_s=4),
        pin_ag_multiparam,
        lambda: pin_rs_exact(8, 4, O.AVG, [(7, 8), (5, 3), (16,)]),
        lambda: pin_rs_exact(8, 4, O.SUM, [(7, 8), (5, 3), (16,)]),
        lambda: pin_end_to_end_exact(8, 4, O.SUM, [(7, 8), (5, 3), (16,)]),
        lambda: pin_end_to_end_exact(8, 4, O.AVG, [(7, 8), (5, 3), (16,)]),
        lambda: _groups_pin(golden),
        lambda: [] if _bf16_pin() else ["bf16 rounding"],
        pin_bf16_round_once,
        pin_f16_round_once,
        pin_avg_correctly_rounded,
        pin_nonzero_dims,
        lambda: pin_fused_layout(golden),
        lambda: pin_fold_order(8, 4, O.SUM, n=256),
        lambda: pin_fold_order(8, 2, O.AVG, n=256),
    ]
    bad = []
    for k, pin in enumerate(pins):
        try:
            bad += pin()
        except Exception as e:
            bad.append(f"pin {k} raised {e!r}")
    return bad


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, golden, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(F, name, fn)
    if hasattr(O, name):  # the package re-exports most names
        monkeypatch.setattr(O, name, fn)
    bad = _all_pins(golden)
    # caught by a value check, not only by something raising
    assert [b for b in bad if " raised " not in b], \
        f"planted mistake {mutant} ({name}) passed every value pin: {bad}"


def test_unmutated_oracle_passes_all_pins(golden):
    assert _all_pins(golden) == []


# ---------------------------------------------------------------------------
# non-zero shard dims (divisible only)
# ---------------------------------------------------------------------------

MIXED = [((6, 8), 1), ((4, 12, 3), 1), ((5, 3, 8), 2), ((7, 3), 0), ((16,), 0), ((2, 0, 4), 2)]


def pin_nonzero_dims():
    """Chunks along a non-zero dim equal torch.chunk along that dim, sit
    contiguously in their slice region, and gather back to the parameter."""
    bad = []
    for S in (1, 2, 4):
        shapes = [sh for sh, k in MIXED]
        dims = [k for sh, k in MIXED]
        lay = O.bucket_layout(shapes, S, shard_dims=dims)
        xs = [(RNG.standard_normal(sh) + 3).astype(np.float32) for sh in shapes]
        shards = O.shard_params(xs, lay)
        for i, (x, k) in enumerate(zip(xs, dims)):
            if k == 0:
                continue
            pieces = torch.chunk(torch.from_numpy(x), S, dim=k)
            for s in range(S):
                if not np.array_equal(shards[s][i], pieces[s].numpy()):
                    bad.append(f"dim-{k} chunk S={S} param {i} rank {s}")
            if lay.padded[i] * S != x.size:  # even: no padding
                bad.append(f"dim-{k} padding S={S} param {i}")
        ag = O.ag_copy_in(shards, lay, np.float32)
        outs = O.ag_copy_out(O.all_gather(ag), lay)
        if not all(np.array_equal(a, b) for a, b in zip(outs, xs)):
            bad.append(f"dim-k round trip S={S}")
        # slice s, region i = rank s's chunk, contiguous
        for s in range(S):
            for i in range(len(shapes)):
                region = ag[s * lay.I + lay.in_off[i]: s * lay.I + lay.in_off[i] + shards[s][i].size]
                if not np.array_equal(region, shards[s][i].reshape(-1)):
                    bad.append(f"dim-k region S={S} param {i} rank {s}")
    return bad


def test_nonzero_shard_dim_matches_torch_chunk_and_roundtrips():
    assert pin_nonzero_dims() == []


def test_nonzero_shard_dim_rejects_uneven():
    with pytest.raises(NotImplementedError):
        O.bucket_layout([(6, 7)], 2, shard_dims=[1])
    with pytest.raises(ValueError):
        O.bucket_layout([(6,)], 2, shard_dims=[1])


@pytest.mark.parametrize("R,S", [(8, 4), (4, 2), (8, 8)])
def test_nonzero_shard_dim_exact_reduce_scatter(R, S):
    shapes = [((6, 8), 1), ((4, 8, 3), 1), ((5, 3, 8), 2), ((7, 3), 0)]
    lay = O.bucket_layout([sh for sh, _ in shapes], S, shard_dims=[k for _, k in shapes])
    gi = [[RNG.integers(-8, 9, size=sh).astype(np.float32) for sh, _ in shapes] for _ in range(R)]
    rs_in = [O.rs_copy_in(gi[g], lay) for g in range(R)]
    outs = O.rs_reduce(rs_in, lay.I, R, S, O.SUM)
    for g in range(R):
        d, s = divmod(g, S)
        for i, (sh, k) in enumerate(shapes):
            tot = sum(torch.from_numpy(gi[m][i]).to(torch.int64) for m in range(d * S, d * S + S))
            pieces = torch.chunk(tot, S, dim=k) if sh[k] else ()
            empty = list(sh)
            empty[k] = 0
            want = pieces[s] if s < len(pieces) else torch.zeros(empty, dtype=torch.int64)
            got = O.sharded_grad(outs[g], lay, i, s)
            assert got.shape == tuple(want.shape) and np.array_equal(got.astype(np.int64), want.numpy())
