"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

The layout and group queries run on the host only, so they are compared
with the oracle here.  Invalid arguments to the device entry points are
rejected before any HIP call, so those error paths are exercised here too,
with fake addresses that are never dereferenced.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsdp_flat.h")

hp = pytest.importorskip("hsdp_parameter_gradient_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hp.lib_path()):
        pytest.fail("libfsdpflat.so is not built (run __graft_entry__.build())")
    return hp.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fsdp_\w+)\s*\(", text)))


def test_header_declares_the_five_ops_and_queries():
    names = declared_functions()
    for n in ("fsdp_ag_copy_in", "fsdp_ag_copy_out", "fsdp_rs_copy_in", "fsdp_rs_reduce",
              "fsdp_rs_copy_reduce", "fsdp_fused_ar", "fsdp_bucket_layout", "fsdp_fused_layout", "fsdp_group_ranks",
              "fsdp_last_error", "fsdp_release_cache", "fsdp_time_next_launch", "fsdp_cache_info",
              "fsdp_rs_copy_reduce_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", hp.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(fsdp_\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(L, n)


SHAPE_SETS = [
    [(7, 8), (5, 3), (16,)],
    [(3072, 1024), (1024, 1024), (4096, 1024), (1024, 4096), (1024,), (1024,)],
    [(4097, 4096), (11009, 4096), (32001, 4096), (5, 64), (3,)],
    [(0, 4), (1,), (2, 3, 4), (9,), (13, 1, 2)],
    [],
]


@pytest.mark.parametrize("shapes", SHAPE_SETS)
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8, 16])
def test_bucket_layout_matches_oracle(L, shapes, S):
    got = hp.fsdp_bucket_layout(shapes, S)
    want = O.bucket_layout(shapes, S)
    assert got.I == want.I
    assert got.padded == want.padded
    assert got.in_off == want.in_off
    assert got.row_off == want.row_off
    assert got.row_len == want.row_len


@pytest.mark.parametrize("S", [1, 2, 4])
def test_bucket_layout_nonzero_shard_dims_match_oracle(L, S):
    shapes = [(6, 8), (4, 12, 3), (5, 3, 8), (7, 3), (16,), (2, 0, 4), (3, 4, 4)]
    dims = [1, 1, 2, 0, 0, 2, 2]
    got = hp.fsdp_bucket_layout(shapes, S, shard_dims=dims)
    want = O.bucket_layout(shapes, S, shard_dims=dims)
    assert (got.I, got.padded, got.in_off, got.row_off, got.row_len) == \
        (want.I, want.padded, want.in_off, want.row_off, want.row_len)


def test_fused_layout_matches_oracle(L, golden):
    for c in golden["fused"]:
        assert hp.fsdp_fused_layout(c["seg_numel"], c["elem_bytes"]) == (c["offsets"], c["F"])
    rng = np.random.default_rng(7)
    for _ in range(20):
        sizes = [int(v) for v in rng.integers(0, 5000, size=int(rng.integers(0, 300)))]
        assert hp.fsdp_fused_layout(sizes, 4) == O.fused_layout(sizes, 4)
        assert hp.fsdp_fused_layout(sizes, 2) == O.fused_layout(sizes, 2)


def test_group_ranks_match_oracle(L, golden):
    for R, S in [(8, 4), (8, 1), (8, 8), (1, 1), (16, 4), (6, 2), (12, 3)]:
        rs, ar = hp.fsdp_group_ranks(R, S)
        plan = dict((k, g) for k, g in O.grad_sync_plan(R, S))
        assert rs == plan.get("RS", [])
        assert ar == plan.get("AR", [])
    for c in golden["groups"]:
        rs, ar = hp.fsdp_group_ranks(c["rank_size"], c["shard_size"])
        want = dict((k, g) for k, g in c["calls"])
        assert rs == want.get("RS", []) and ar == want.get("AR", [])


def test_query_errors(L):
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([(4, 3)], 2, shard_dim=1)
    assert e.value.code == 2 and "divisible" in e.value.message
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([(4,)], 2, shard_dim=1)
    assert e.value.code == 1
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([()], 2)
    assert e.value.code == 1
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([(4,)], 0)
    assert e.value.code == 1
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([(-1, 2)], 2)
    assert e.value.code == 1
    with pytest.raises(hp.FSDPError) as e:
        hp.fsdp_bucket_layout([(1 << 40, 1 << 30)], 2)
    assert e.value.code == 1
    with pytest.raises(hp.FSDPError):
        hp.fsdp_group_ranks(8, 3)
    with pytest.raises(hp.FSDPError):
        hp.fsdp_fused_layout([4, -1])
    with pytest.raises(hp.FSDPError):
        hp.fsdp_fused_layout([4], 8)


# --- device entry points: argument errors caught before any HIP call -------

def _bucket(shapes, shard_dim=0):
    from hsdp_parameter_gradient_amd._binding import _BucketArg
    return _BucketArg(shapes, shard_dim)


def _ptrs(vals):
    return (ctypes.c_void_p * max(len(vals), 1))(*[v or None for v in vals])


BASE = 1 << 40  # fake, never dereferenced


def test_device_entry_points_reject_bad_arguments(L):
    shapes = [(7, 8), (5, 3), (16,)]
    S, P = 4, 3
    lay = O.bucket_layout(shapes, S)
    b = _bucket(shapes)
    shards = _ptrs([BASE + 0x100000 * (k + 1) for k in range(S * P)])
    ag = ctypes.c_void_p(BASE)
    # shard_dim != 0
    b1 = _bucket(shapes, shard_dim=1)
    assert L.fsdp_ag_copy_in(b1.ref, S, 0, shards, ag, None) == 2
    # unknown dtype
    assert L.fsdp_ag_copy_in(b.ref, S, 7, shards, ag, None) == 2
    # NULL output with bytes to write
    assert L.fsdp_ag_copy_in(b.ref, S, 0, shards, None, None) == 1
    # misaligned output
    assert L.fsdp_ag_copy_in(b.ref, S, 0, shards, ctypes.c_void_p(BASE + 2), None) == 3
    # a source inside the output buffer
    bad = _ptrs([BASE + 64] + [BASE + 0x100000 * (k + 1) for k in range(1, S * P)])
    assert L.fsdp_ag_copy_in(b.ref, S, 0, bad, ag, None) == 5
    assert "overlap" in hp.fsdp_last_error()
    # NULL shard pointer that should hold rows (rank 0 of param 0 holds 2 rows)
    nul = _ptrs([0] + [BASE + 0x100000 * (k + 1) for k in range(1, S * P)])
    assert L.fsdp_ag_copy_in(b.ref, S, 0, nul, ag, None) == 1
    # copy-out: two full outputs overlap
    full = _ptrs([BASE + 0x200000, BASE + 0x200000 + 8, BASE + 0x300000])
    assert L.fsdp_ag_copy_out(b.ref, S, 0, ag, full, None) == 5
    # rs_copy_in: rank_size not a multiple of shard_size
    grads = _ptrs([BASE + 0x100000 * (k + 1) for k in range(6 * P)])
    rs_in = _ptrs([BASE + 0x10000000 * (g + 1) for g in range(6)])
    assert L.fsdp_rs_copy_in(b.ref, 6, S, 0, grads, rs_in, None) == 1
    # rs_reduce: dp_size inconsistent, op unknown, dtype not a reduction dtype, output aliasing input
    rs8 = _ptrs([BASE + 0x10000000 * (g + 1) for g in range(8)])
    out8 = _ptrs([BASE + 0x1000000 * (g + 1) for g in range(8)])
    assert L.fsdp_rs_reduce(b.ref, 8, S, 3, 0, 0, rs8, out8, None) == 1
    assert L.fsdp_rs_reduce(b.ref, 8, S, 2, 9, 0, rs8, out8, None) == 1
    assert L.fsdp_rs_reduce(b.ref, 8, S, 2, 0, 5, rs8, out8, None) == 2
    alias = _ptrs([BASE + 0x10000000 * (g + 1) + 4 * lay.I for g in range(8)])
    assert L.fsdp_rs_reduce(b.ref, 8, S, 2, 0, 0, rs8, alias, None) == 5
    # rs_copy_reduce: an unknown dtype; an output inside a gradient
    g8 = _ptrs([BASE + 0x100000 * (k + 1) for k in range(8 * P)])
    assert L.fsdp_rs_copy_reduce(b.ref, 8, S, 2, 0, 5, g8, out8, None) == 2
    inside = _ptrs([BASE + 0x100000 + 8] + [BASE + 0x10000000 * (g + 1) for g in range(1, 8)])
    assert L.fsdp_rs_copy_reduce(b.ref, 8, S, 2, 0, 0, g8, inside, None) == 5
    assert L.fsdp_rs_copy_reduce(b.ref, 8, S, 3, 0, 0, g8, out8, None) == 1
    # the variant that allocates nothing validates the same way
    assert L.fsdp_rs_copy_reduce_noalloc(b.ref, 8, S, 2, 0, 5, g8, out8, None) == 2
    assert L.fsdp_rs_copy_reduce_noalloc(b.ref, 8, S, 2, 0, 0, g8, inside, None) == 5
    assert L.fsdp_rs_copy_reduce_noalloc(b.ref, 8, S, 3, 0, 0, g8, out8, None) == 1
    # fused_ar: base not 512-byte aligned, an unknown dtype
    segs = (ctypes.c_int64 * 2)(100, 3)
    f8 = _ptrs([BASE + 0x100000 * g + 256 for g in range(8)])
    assert L.fsdp_fused_ar(2, segs, 8, 4, 2, 1, 0, f8, None) == 3
    f8a = _ptrs([BASE + 0x100000 * g for g in range(8)])
    assert L.fsdp_fused_ar(2, segs, 8, 4, 2, 1, 5, f8a, None) == 2
    ovl = _ptrs([BASE + 512 * g for g in range(8)])
    assert L.fsdp_fused_ar(2, segs, 8, 4, 2, 1, 0, ovl, None) == 5


def test_binding_checks_buffer_sizes():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4)
    with pytest.raises(ValueError):  # host tensors are refused before any C call
        hp.fsdp_ag_copy_in([(4,)], 1, [x], x)


def test_binding_refuses_unknown_ops():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4)
    with pytest.raises(ValueError, match="reduce op"):
        hp.fsdp_fused_ar([4], 2, 1, 2, "max", [x, x])
    # the valid ops get past the op check to the buffer checks
    from hsdp_parameter_gradient_amd import _binding as B
    assert (B._op_code("sum"), B._op_code("avg")) == (0, 1)
    for op in ("sum", "avg"):
        with pytest.raises(ValueError, match="device tensor"):
            hp.fsdp_fused_ar([4], 2, 1, 2, op, [x, x])


def test_binding_checks_shard_dims_length():
    """One shard dim per parameter: a shorter or longer list is refused
    (the C side reads exactly n_params entries)."""
    for dims in ([1], [0, 1, 0]):
        with pytest.raises(ValueError, match="shard_dims"):
            hp.fsdp_bucket_layout([(4, 8), (6, 8)], 2, shard_dims=dims)
    assert hp.fsdp_bucket_layout([(4, 8), (6, 8)], 2, shard_dims=[1, 0]).I == 4 * 4 + 3 * 8


def test_plain_c_consumer_of_the_header(tmp_path):
    """A C program that includes only include/fsdp_flat.h, links the library
    and calls the host-only entry points (and two argument errors) gets the
    hand-derived values."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no C compiler")
    lib = hp.lib_path()
    if not os.path.exists(lib):
        pytest.fail("libfsdpflat.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "c_abi_host")
    src = os.path.join(ROOT, "tests", "c_abi_host.c")
    libdir = os.path.dirname(lib)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src, "-o", exe,
                        "-L", libdir, "-lfsdpflat", "-Wl,-rpath," + libdir], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_flat_bucket_and_group_need_bind():
    """Steps before bind() and mismatched bind() lists are refused with a
    clear error (the checks run on the host, before any device call)."""
    torch = pytest.importorskip("torch")
    fb = hp.FlatBucket.__new__(hp.FlatBucket)
    fb._calls = None
    with pytest.raises(RuntimeError, match="bind"):
        fb.run("ag_copy_in")
    grp = hp.FusedGroup.__new__(hp.FusedGroup)
    grp.buckets, grp._ar = [object(), object()], None
    with pytest.raises(ValueError, match="bind"):
        grp.bind([[]], [[], []])
    with pytest.raises(RuntimeError, match="bind"):
        grp.step()
    with pytest.raises(RuntimeError, match="bind"):
        grp.graph()
    grp._ar = object()
    with pytest.raises(ValueError, match="n_streams"):
        grp.graph(n_streams=0)


def test_shared_fused_buffers_each_bucket_ar_covers_its_own_segment():
    """Buckets sharing a fused buffer (FusedGroup): each bucket's own fused_ar
    step covers its segment and the zero gap after it, on a 512-byte
    boundary, and nothing else; the segments' AR ranges are disjoint and
    together cover the whole buffer (host tensors: no device call)."""
    torch = pytest.importorskip("torch")
    buckets = [[(7, 8), (5, 3)], [(16,)], [(1000, 3)], [(3,)]]
    for R, S, dt in ((8, 4, torch.float32), (4, 2, torch.bfloat16)):
        grp = hp.FusedGroup(buckets, R, S, torch.float32, grad_dtype=dt, device="cpu")
        es = dt.itemsize
        F = grp.fused[0].numel()
        spans = []
        for fb in grp.buckets:
            I = fb.layout.I
            for g in range(R):
                v = fb.ar_buffers[g]
                off = (v.data_ptr() - grp.fused[g].data_ptr()) // es
                assert v.untyped_storage().data_ptr() == grp.fused[g].untyped_storage().data_ptr()
                assert (off * es) % 512 == 0 and off == fb.fused_off
                assert (v.numel() * es) % 512 == 0 and I <= v.numel() < I + 512 // es
                assert fb.rs_out[g].data_ptr() == v.data_ptr() and fb.rs_out[g].numel() == I
            spans.append((fb.fused_off, fb.fused_off + fb.ar_numel))
        spans.sort()
        assert spans[0][0] == 0 and spans[-1][1] == F
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:])), spans


def test_noalloc_refuses_tables_beyond_its_scratch(L):
    """fsdp_rs_copy_reduce_noalloc plans on the host first: a call whose
    descriptor tables exceed the 1 MiB scratch array is refused with
    FSDP_EINVAL and a message naming the sizes, before any HIP call (so it
    runs here, without a GPU, on fake addresses)."""
    P, R, S = 2000, 8, 8
    b = hp._binding._BucketArg([(8,)] * P)
    g = _ptrs([BASE + 0x1000 * (k + 1) for k in range(R * P)])
    out = _ptrs([BASE + 0x40000000 + 0x100000 * (k + 1) for k in range(R)])
    assert L.fsdp_rs_copy_reduce_noalloc(b.ref, R, S, 1, 0, 0, g, out, None) == 1
    msg = hp.fsdp_last_error()
    assert "scratch" in msg and "1048576" in msg, msg


def test_time_next_launch_arguments(L):
    """Both events or neither: one NULL handle is FSDP_EINVAL (no HIP call)."""
    assert L.fsdp_time_next_launch(None, None) == 0
    assert L.fsdp_time_next_launch(ctypes.c_void_p(0x1000), None) == 1
    assert L.fsdp_time_next_launch(None, ctypes.c_void_p(0x1000)) == 1
    assert "both events" in hp.fsdp_last_error()
    assert L.fsdp_time_next_launch(None, None) == 0


def test_cache_info_without_a_gpu(L):
    """Nothing is cached without a GPU; NULL outputs are allowed."""
    hp.fsdp_release_cache()
    assert hp.fsdp_cache_info() == {"plans": 0, "pinned": 0, "table_bytes": 0}
    assert L.fsdp_cache_info(None, None, None) == 0
