"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer,
and the tables it really builds against the CPU emulation of the kernels.

fsdp_flat.cpp (validation, layout, descriptor-table construction, plan
cache) is built with g++ -fsanitize=address,undefined and the table hook,
without the device kernels, and driven by tests/host_sanitizer_driver.cpp
over ragged, empty, non-zero-dim and misaligned buckets.  With no GPU
visible every call plans in full and then fails its upload (FSDP_EHIP), so
any out-of-bounds access, overflow or leak in the planner is reported; the
hook dumps every planned table, and the kernels' indexing (emulated in
tests/test_kernel_indexing.py) is run over each one: every destination byte
written exactly once with the right source, nothing outside, every read
inside its source envelope.  CPU only.
"""

import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import test_kernel_indexing as KI

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hsdp_parameter_gradient_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the ROCm runtime library")
    exe = str(tmp_path_factory.mktemp("drv") / "host_sanitizer_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-DFSDP_TABLE_HOOK", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fsdp_flat.cpp"), os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _run(exe, extra_env=None, args=()):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    env.update(extra_env or {})
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=env)
    if r.stdout.strip() == "skip":
        pytest.skip("a GPU is visible: the driver needs the uploads to fail")
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-4000:]


def test_planner_under_asan_and_ubsan(driver):
    _run(driver)


def test_exceptions_do_not_cross_the_c_abi(driver):
    """An exception thrown while a call is planned (planted in the table
    hook: bad_alloc, length_error, another std::exception) comes back as
    FSDP_ENOMEM / FSDP_ENOMEM / FSDP_EINVAL from copies and reductions, and
    the following calls plan normally (no leak under LeakSanitizer)."""
    _run(driver, args=("throw",))


def _records(path):
    data = open(path, "rb").read()
    pos = 0
    while pos < len(data):
        kind, elt, a, b = struct.unpack_from("<4I", data, pos)
        n_chunks, nbytes = struct.unpack_from("<2Q", data, pos + 16)
        pos += 32
        yield kind, elt, a, b, n_chunks, data[pos:pos + nbytes]
        pos += nbytes


def _merge(iv):
    out = []
    for a, b in sorted(x for x in iv if x[0] < x[1]):
        if out and a <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], b))
        else:
            out.append((a, b))
    return out


def _inside(iv, allowed):
    """Every interval of iv lies inside one interval of allowed (merged)."""
    import bisect
    starts = [a for a, _ in allowed]
    for a, b in iv:
        k = bisect.bisect_right(starts, a) - 1
        if k < 0 or b > allowed[k][1]:
            return (a, b)
    return None


TUNINGS = {
    "default": {},
    # the smallest and a large chunk size the tuning accepts (copy and reduce chunks)
    "chunks_512B": {"FSDP_COPY_CHUNK_SHIFT": "9", "FSDP_REDUCE_CHUNK_SHIFT": "9"},
    "chunks_1MiB": {"FSDP_COPY_CHUNK_SHIFT": "20", "FSDP_REDUCE_CHUNK_SHIFT": "20"},
}


@pytest.mark.parametrize("tuning", list(TUNINGS))
def test_planner_tables_pass_the_kernel_emulation(driver, tmp_path, tuning):
    """Every table the planner builds, run through the emulated kernels,
    writes exactly its call's output buffers (every byte once) and reads
    only inside the aligned envelopes of its call's inputs; at the default
    chunk sizes and at the extremes the tuning overrides allow."""
    dump = str(tmp_path / "tables.bin")
    _run(driver, {"FSDP_DUMP_TABLES": dump, **TUNINGS[tuning]})
    counts = _check_tables(dump)
    # the driver's buckets produce copy, reduce, fold and fold-reduce tables,
    # strided blocks included
    assert counts[0] > 100 and counts[1] > 100 and counts["blocks"] > (50 if tuning == "default" else 0), counts
    assert counts[3] > (10 if tuning != "chunks_512B" else 0), counts
    assert counts[4] > (10 if tuning != "chunks_512B" else 0), counts
    # long rows at per-row alignments: fold and fold-reduce items of flat chunks
    assert tuning != "default" or counts["flat_chunks"] > 10, counts


def test_random_bucket_tables_pass_the_kernel_emulation(driver, tmp_path):
    """The seeded random buckets that test_gpu_random.py runs on the GPU
    (ragged and zero dims, shard dims 1 and 2, group sizes up to 32, every
    buffer at its own element offset), planned by the real planner and run
    through the emulated kernels: exact writes, reads inside the inputs."""
    import bucket_cases as BC
    cases = tmp_path / "cases.txt"
    cases.write_text("\n".join(BC.case_line(c) for c in BC.random_cases(BC_SEED, BC_COUNT)) + "\n")
    dump = str(tmp_path / "tables.bin")
    _run(driver, {"FSDP_DUMP_TABLES": dump}, args=("cases", str(cases)))
    counts = _check_tables(dump)
    assert counts[0] > 2 * BC_COUNT and counts[1] > 2 * BC_COUNT, counts


BC_SEED, BC_COUNT = 20261202, 40  # the cases of test_gpu_random.py (its SEED, COUNT)
if os.environ.get("FSDP_RANDOM_CASES"):  # a longer sweep, as in test_gpu_random.py
    BC_SEED, BC_COUNT = (int(x) for x in os.environ["FSDP_RANDOM_CASES"].split(":"))


def _check_tables(dump):
    """Run every dumped table through the emulated kernels; per call (the
    tables between two span records), the writes of all its tables together
    cover exactly the call's outputs, each byte once, and every read lies in
    the aligned envelope of the call's inputs."""
    counts = {0: 0, 1: 0, 3: 0, 4: 0, "blocks": 0, "flat_chunks": 0}
    state = {"outs": None, "ins": None, "w": [], "tables": 0}

    def finish():
        if state["tables"]:
            w = state["w"]
            assert _merge(w) == state["outs"], "the call's writes do not cover exactly its outputs"
            assert sum(b - a for a, b in w) == sum(b - a for a, b in state["outs"]), "a byte written twice"
        state["w"], state["tables"] = [], 0

    for kind, elt, a, b, n_chunks, blob in _records(dump):
        words = np.frombuffer(blob[:len(blob) // 8 * 8], dtype=np.uint64)  # a copy table ends in 32-bit words
        if kind == 2:  # the next call's output and input spans
            finish()
            sp = [(int(words[2 * k]), int(words[2 * k]) + int(words[2 * k + 1])) for k in range(a + b)]
            state["outs"], state["ins"] = _merge(sp[:a]), _merge(sp[a:])
            continue
        n, shift = a, b
        begin = [int(v) for v in words[:n]]
        if kind == 0:
            recs = words[n:n + 8 * n].reshape(n, 8)
            segs = [tuple(int(v) for v in r) for r in recs]
            # the planner's chunk prefix is the one the kernel indexes
            want, c = [], 0
            for sg in segs:
                want.append(c)
                c += KI.item_chunks(sg[1], sg[3], sg[4], sg[7], shift)
            assert begin == want and c == n_chunks
            # item_of maps every chunk to its item, as the prefix does
            assert len(blob) == 72 * n + 4 * n_chunks
            item_of = np.frombuffer(blob[72 * n:], dtype=np.uint32)
            assert np.array_equal(item_of, np.repeat(np.arange(n, dtype=np.uint32), np.diff(want + [c])))
            writes, reads = KI.check_copy(segs, elt, shift)
            w_iv = [(w[0], w[1]) for w in writes]
            r_iv = [(r[0], r[1]) for r in reads]
            counts["blocks"] += sum(sg[4] > 1 for sg in segs)
        elif kind == 3:
            raw = blob[8 * n:8 * n + 64 * n]
            assert len(blob) == 8 * n + 64 * n
            folds = [struct.unpack_from(KI.FOLD_FMT, raw, 64 * k) for k in range(n)]
            counts["flat_chunks"] += sum(f[3] == 0 for f in folds)
            fbegin, c, writes, reads = KI.emulate_fold(folds, 1 << shift)
            assert begin == fbegin and c == n_chunks
            w_iv = [(w[0], w[1]) for w in writes]
            r_iv = [(r[0], r[1]) for r in reads]
            # within a table every byte is written once
            assert sum(y - x for x, y in w_iv) == sum(y - x for x, y in _merge(w_iv))
        elif kind == 4:
            raw = blob[8 * n:8 * n + 64 * n]
            items = [struct.unpack_from(KI.FOLD_RED_FMT, raw, 64 * k) for k in range(n)]
            counts["flat_chunks"] += sum(f[2] == 0 for f in items)
            ptr = [int(v) for v in np.frombuffer(blob[8 * n + 64 * n:], dtype=np.uint64)]
            fbegin, c, writes, reads = KI.emulate_fold_reduce(items, ptr, 1 << shift)
            assert begin == fbegin and c == n_chunks
            w_iv = [(w[0], w[1]) for w in writes]
            r_iv = [(r[0], r[1]) for r in reads]
            assert sum(y - x for x, y in w_iv) == sum(y - x for x, y in _merge(w_iv))
        else:
            raw = blob[8 * n:8 * n + 64 * n]
            jobs = [struct.unpack_from("<2Q4I4Q", raw, 64 * k) for k in range(n)]
            ptr = [int(v) for v in np.frombuffer(blob[8 * n + 64 * n:], dtype=np.uint64)]
            want, c = [], 0
            for jb in jobs:
                want.append(c)
                c += KI.item_chunks(ptr[jb[4]], jb[0], jb[6], jb[9], shift)
            assert begin == want and c == n_chunks
            es = 4 if elt == 0 else 2
            writes, reads = KI.check_reduce(jobs, ptr, shift, es)
            w_iv = [(w[0], w[1]) for w in writes]
            r_iv = [(r[0], r[1]) for r in reads]
            counts["blocks"] += sum(jb[6] > 1 for jb in jobs)
        state["w"].extend(_merge(w_iv))
        state["tables"] += 1
        # an input's envelope: from the 128-byte line of its first byte (the
        # reduction's line-phase rotation reads there; a line never spans two
        # pages) to the 16-byte block of its last byte
        env = _merge([(x & ~127, (y + 15) & ~15) for x, y in state["ins"]])
        bad = _inside(r_iv, env)
        assert bad is None, f"read {bad} outside the inputs' aligned envelopes"
        counts[kind] += 1
    finish()
    return counts
