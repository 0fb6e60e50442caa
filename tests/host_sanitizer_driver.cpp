// Host-side driver for a sanitizer build of the planner (fsdp_flat.cpp built
// with g++ -fsanitize=address,undefined, without the device kernels).
//
// With no GPU visible, every call runs its validation and builds its
// descriptor table; the upload then fails (no device) and the call returns
// FSDP_EHIP, so the planner's table construction runs in full under the
// sanitizers.  Calls that are rejected earlier must return the documented
// error code.  The device kernels are replaced by launchers that must never
// be reached.  Buffers are fake addresses that are never dereferenced.
//
// Prints "ok" (exit 0), "skip" (exit 0) when a GPU is visible, or the
// failed checks (exit 1).
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <stdexcept>
#include <utility>
#include <vector>

#include "fsdp_flat.h"

int fsdp_launch_seg_copy(int, const void*, uint32_t, uint64_t, uint32_t, uint32_t, int, void*, void*, void*) {
  std::fprintf(stderr, "seg_copy launcher reached without a device\n");
  std::abort();
}
int fsdp_launch_reduce(int, const void*, uint32_t, uint32_t, uint64_t, uint32_t, uint32_t, int, int, void*, void*,
                       void*) {
  std::fprintf(stderr, "reduce launcher reached without a device\n");
  std::abort();
}
int fsdp_launch_fold(const void*, uint32_t, uint64_t, uint32_t, int, int, void*, void*, void*) {
  std::fprintf(stderr, "fold launcher reached without a device\n");
  std::abort();
}
int fsdp_launch_fold_reduce(int, const void*, uint32_t, uint32_t, uint64_t, uint32_t, int, int, int, void*, void*,
                            void*) {
  std::fprintf(stderr, "fold-reduce launcher reached without a device\n");
  std::abort();
}

int fsdp_scratch_ptr(void** out) {
  *out = nullptr;
  return (int)hipErrorNoDevice;  // no device here: the call stops after planning
}
int fsdp_scratch_write(void*, const void*, size_t, size_t, void*) {
  std::fprintf(stderr, "scratch writer reached without a device\n");
  std::abort();
}

// Set by the "throw" mode: the hook then throws the given exception kind
// (1 bad_alloc, 2 length_error, 3 runtime_error), as an allocation inside
// the planner would.
int g_hook_throw = 0;

// With FSDP_TABLE_HOOK, every planned table is appended to the file named
// by FSDP_DUMP_TABLES (if set): a 32-byte header (kind: 0 copy, 1 reduce,
// 3 fold copy, 4 fold reduce; elt, n_items, shift, n_chunks, table bytes)
// and the table itself.
void fsdp_table_hook(int reduce, int elt, uint32_t n_items, uint64_t n_chunks, uint32_t shift,
                     const std::vector<uint8_t>& table) {
  if (g_hook_throw == 1) throw std::bad_alloc();
  if (g_hook_throw == 2) throw std::length_error("table");
  if (g_hook_throw == 3) throw std::runtime_error("planted");
  const char* path = std::getenv("FSDP_DUMP_TABLES");
  if (!path) return;
  FILE* f = std::fopen(path, "ab");
  if (!f) return;
  const uint32_t h32[4] = {(uint32_t)reduce, (uint32_t)elt, n_items, shift};
  const uint64_t h64[2] = {n_chunks, (uint64_t)table.size()};
  std::fwrite(h32, sizeof h32, 1, f);
  std::fwrite(h64, sizeof h64, 1, f);
  std::fwrite(table.data(), 1, table.size(), f);
  std::fclose(f);
}

// Before each device call the driver appends the call's output and input
// byte spans (a record with reduce = 2), so each dumped table can be
// checked against what its call must write and may read.
void dump_io(const std::vector<std::pair<uint64_t, uint64_t>>& outs,
             const std::vector<std::pair<uint64_t, uint64_t>>& ins) {
  const char* path = std::getenv("FSDP_DUMP_TABLES");
  if (!path) return;
  FILE* f = std::fopen(path, "ab");
  if (!f) return;
  std::vector<uint64_t> body;
  for (auto& o : outs) body.insert(body.end(), {o.first, o.second});
  for (auto& i : ins) body.insert(body.end(), {i.first, i.second});
  const uint32_t h32[4] = {2u, 0u, (uint32_t)outs.size(), (uint32_t)ins.size()};
  const uint64_t h64[2] = {0, (uint64_t)(body.size() * 8)};
  std::fwrite(h32, sizeof h32, 1, f);
  std::fwrite(h64, sizeof h64, 1, f);
  std::fwrite(body.data(), 8, body.size(), f);
  std::fclose(f);
}

namespace {

int failures = 0;

using Spans = std::vector<std::pair<uint64_t, uint64_t>>;
uint64_t A(const void* p) { return reinterpret_cast<uint64_t>(p); }

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want, fsdp_last_error());
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// Fake, disjoint, 512-byte-aligned buffers (plus an element offset).  With
// vary set, a non-zero offset (one element) becomes 1..7 elements, changing
// from buffer to buffer.
bool g_vary_offsets = false;

struct Fake {
  uint64_t next = uint64_t(1) << 40;
  uint64_t count = 0;
  void* get(uint64_t bytes, uint64_t offset = 0) {
    if (g_vary_offsets && offset) offset *= 1 + (count++ % 7);
    void* p = reinterpret_cast<void*>(next + offset);
    next += (bytes + offset + 4096 + 511) / 512 * 512;
    return p;
  }
};

struct Case {
  std::vector<std::vector<int64_t>> shapes;
  std::vector<int32_t> dims;  // empty: all 0
};

int64_t numel(const std::vector<int64_t>& s) {
  int64_t n = 1;
  for (int64_t d : s) n *= d;
  return n;
}

void run_case(const Case& c, int32_t S, int32_t R, int32_t es, bool misalign) {
  const int32_t P = (int32_t)c.shapes.size();
  std::vector<int32_t> ndim;
  std::vector<int64_t> shape;
  for (const auto& s : c.shapes) {
    ndim.push_back((int32_t)s.size());
    shape.insert(shape.end(), s.begin(), s.end());
  }
  fsdp_bucket_t b = {P, ndim.data(), shape.data(), 0, c.dims.empty() ? nullptr : c.dims.data()};
  int64_t I = 0;
  if (fsdp_bucket_layout(&b, S, &I, nullptr, nullptr, nullptr, nullptr) != FSDP_OK) {
    std::fprintf(stderr, "layout failed: %s\n", fsdp_last_error());
    ++failures;
    return;
  }
  std::vector<int64_t> row_len((size_t)P * S);
  fsdp_bucket_layout(&b, S, nullptr, nullptr, nullptr, nullptr, row_len.data());
  const int32_t dtype = es == 4 ? FSDP_F32 : misalign ? FSDP_F16 : FSDP_BF16;
  const int32_t D = R / S;
  Fake f;
  const uint64_t off = misalign ? (uint64_t)es : 0;
  // the layout's total bytes of chunk s of parameter i
  auto chunk_bytes = [&](int32_t i, int32_t s) {
    const auto& sh = c.shapes[(size_t)i];
    const int32_t k = c.dims.empty() ? 0 : c.dims[(size_t)i];
    return numel(sh) / (sh[(size_t)k] ? sh[(size_t)k] : 1) * row_len[(size_t)i * S + s] * es;
  };
  const bool work = I > 0;
  const int want = work ? FSDP_EHIP : FSDP_OK;

  std::vector<const void*> shards;
  Spans shard_sp;
  for (int32_t s = 0; s < S; ++s)
    for (int32_t i = 0; i < P; ++i) {
      const uint64_t nb = (uint64_t)chunk_bytes(i, s);
      shards.push_back(f.get(nb, off));
      shard_sp.push_back({A(shards.back()), nb});
    }
  void* ag = f.get((uint64_t)(S * I * es), off);
  const Spans ag_sp = {{A(ag), (uint64_t)(S * I * es)}};
  dump_io(ag_sp, shard_sp);
  EXPECT(fsdp_ag_copy_in(&b, S, dtype, shards.data(), ag, nullptr), want);
  std::vector<void*> full;
  Spans full_sp;
  bool any_full = false;
  for (int32_t i = 0; i < P; ++i) {
    const uint64_t nb = (uint64_t)(numel(c.shapes[(size_t)i]) * es);
    full.push_back(f.get(nb, off));
    full_sp.push_back({A(full.back()), nb});
    any_full = any_full || nb > 0;
  }
  dump_io(full_sp, ag_sp);
  EXPECT(fsdp_ag_copy_out(&b, S, dtype, ag, full.data(), nullptr), any_full ? FSDP_EHIP : FSDP_OK);

  std::vector<const void*> grads;
  Spans grad_sp;
  for (int32_t g = 0; g < R; ++g)
    for (int32_t i = 0; i < P; ++i) {
      const uint64_t nb = (uint64_t)(numel(c.shapes[(size_t)i]) * es);
      grads.push_back(f.get(nb, off));
      grad_sp.push_back({A(grads.back()), nb});
    }
  std::vector<void*> rs_in, rs_out;
  Spans in_sp, out_sp;
  for (int32_t g = 0; g < R; ++g) {
    rs_in.push_back(f.get((uint64_t)(S * I * es), off));
    rs_out.push_back(f.get((uint64_t)(I * es), off));
    in_sp.push_back({A(rs_in.back()), (uint64_t)(S * I * es)});
    out_sp.push_back({A(rs_out.back()), (uint64_t)(I * es)});
  }
  dump_io(in_sp, grad_sp);
  EXPECT(fsdp_rs_copy_in(&b, R, S, dtype, grads.data(), rs_in.data(), nullptr), want);
  const void* const* rs_in_c = rs_in.data();
  dump_io(out_sp, in_sp);
  EXPECT(fsdp_rs_reduce(&b, R, S, D, FSDP_AVG, dtype, rs_in_c, rs_out.data(), nullptr), want);
  dump_io(out_sp, grad_sp);
  EXPECT(fsdp_rs_copy_reduce(&b, R, S, D, FSDP_SUM, dtype, grads.data(), rs_out.data(), nullptr), want);
  // the variant that allocates nothing plans the same tables, then stops at
  // the scratch array's address (no device), or refuses tables too large
  // for the scratch array
  dump_io(out_sp, grad_sp);
  {
    const int rc = fsdp_rs_copy_reduce_noalloc(&b, R, S, D, FSDP_SUM, dtype, grads.data(), rs_out.data(), nullptr);
    const bool big = rc == FSDP_EINVAL && std::strstr(fsdp_last_error(), "scratch");
    if (!(rc == want || (work && big))) expect(rc, want, "fsdp_rs_copy_reduce_noalloc", __LINE__);
  }

  // fused buffers: this bucket's RS output plus two more segments
  const int64_t segs[3] = {I, 3, 1000};
  int64_t F = 0;
  fsdp_fused_layout(3, segs, es, nullptr, &F);
  std::vector<void*> fused;
  Spans fused_sp;
  for (int32_t g = 0; g < R; ++g) {
    fused.push_back(f.get((uint64_t)(F * es)));
    fused_sp.push_back({A(fused.back()), (uint64_t)(F * es)});
  }
  dump_io(fused_sp, fused_sp);
  EXPECT(fsdp_fused_ar(3, segs, R, S, D, FSDP_AVG, dtype, fused.data(), nullptr), D > 1 ? FSDP_EHIP : FSDP_OK);

  // argument errors, caught before planning
  EXPECT(fsdp_rs_reduce(&b, R, S, D + 1, FSDP_AVG, dtype, rs_in_c, rs_out.data(), nullptr), FSDP_EINVAL);
  EXPECT(fsdp_rs_copy_reduce(&b, R, S, D, 7, dtype, grads.data(), rs_out.data(), nullptr), FSDP_EINVAL);
  EXPECT(fsdp_ag_copy_in(&b, S, 9, shards.data(), ag, nullptr), FSDP_ENOTIMPL);
  if (work) {
    // an output inside an input
    std::vector<void*> bad(rs_out);
    bad[0] = const_cast<void*>(rs_in_c[0]);
    EXPECT(fsdp_rs_reduce(&b, R, S, D, FSDP_SUM, dtype, rs_in_c, bad.data(), nullptr), FSDP_EOVERLAP);
  }
}

}  // namespace

// An exception thrown while a call is planned must come back as a status
// code (FSDP_ENOMEM for allocation failures, FSDP_EINVAL otherwise), for
// copies and reductions alike, and the next call must work normally.
void run_throw_mode() {
  const std::vector<int64_t> shape = {7, 8, 5, 3, 16};
  const int32_t ndim[3] = {2, 2, 1};
  fsdp_bucket_t b = {3, ndim, shape.data(), 0, nullptr};
  const int32_t S = 4;
  int64_t I = 0;
  fsdp_bucket_layout(&b, S, &I, nullptr, nullptr, nullptr, nullptr);
  std::vector<int64_t> row_len(3 * S);
  fsdp_bucket_layout(&b, S, nullptr, nullptr, nullptr, nullptr, row_len.data());
  Fake f;
  std::vector<const void*> shards;
  const int64_t inner[3] = {8, 3, 1};
  for (int32_t s = 0; s < S; ++s)
    for (int32_t i = 0; i < 3; ++i) shards.push_back(f.get((uint64_t)(row_len[(size_t)i * S + s] * inner[i] * 4)));
  void* ag = f.get((uint64_t)(S * I * 4));
  std::vector<void*> fused;
  const int64_t seg[1] = {I};
  int64_t F = 0;
  fsdp_fused_layout(1, seg, 4, nullptr, &F);
  for (int g = 0; g < 2; ++g) fused.push_back(f.get((uint64_t)(F * 4)));
  const int want[4] = {FSDP_EHIP, FSDP_ENOMEM, FSDP_ENOMEM, FSDP_EINVAL};
  for (int kind = 1; kind <= 3; ++kind) {
    g_hook_throw = kind;
    EXPECT(fsdp_ag_copy_in(&b, S, FSDP_F32, shards.data(), ag, nullptr), want[kind]);
    if (kind == 3 && !std::strstr(fsdp_last_error(), "planted")) {
      std::fprintf(stderr, "message does not carry the exception's text: %s\n", fsdp_last_error());
      ++failures;
    }
    EXPECT(fsdp_fused_ar(1, seg, 2, 1, 2, FSDP_AVG, FSDP_F32, fused.data(), nullptr), want[kind]);
  }
  g_hook_throw = 0;  // and the library works on
  EXPECT(fsdp_ag_copy_in(&b, S, FSDP_F32, shards.data(), ag, nullptr), want[0]);
  EXPECT(fsdp_fused_ar(1, seg, 2, 1, 2, FSDP_AVG, FSDP_F32, fused.data(), nullptr), want[0]);
}

int main(int argc, char** argv) {
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
    std::printf("skip\n");
    return 0;
  }
  if (argc > 2 && std::strcmp(argv[1], "cases") == 0) {
    // one case per line: S R es misaligned P, then per parameter ndim, its
    // dims and its shard dim
    FILE* f = std::fopen(argv[2], "r");
    if (!f) {
      std::fprintf(stderr, "cannot open %s\n", argv[2]);
      return 1;
    }
    g_vary_offsets = true;
    int S, R, es, mis, P, n_cases = 0;
    while (std::fscanf(f, "%d %d %d %d %d", &S, &R, &es, &mis, &P) == 5) {
      Case c;
      for (int i = 0; i < P; ++i) {
        int nd = 0, k = 0;
        if (std::fscanf(f, "%d", &nd) != 1) return 1;
        std::vector<int64_t> sh((size_t)nd);
        for (int d = 0; d < nd; ++d) {
          long long v = 0;
          if (std::fscanf(f, "%lld", &v) != 1) return 1;
          sh[(size_t)d] = v;
        }
        if (std::fscanf(f, "%d", &k) != 1) return 1;
        c.shapes.push_back(sh);
        c.dims.push_back(k);
      }
      run_case(c, S, R, es, mis != 0);
      ++n_cases;
    }
    std::fclose(f);
    fsdp_release_cache();
    if (failures || n_cases == 0) {
      std::fprintf(stderr, "%d checks failed over %d cases\n", failures, n_cases);
      return 1;
    }
    std::printf("ok\n");
    return 0;
  }
  if (argc > 1 && std::strcmp(argv[1], "throw") == 0) {
    run_throw_mode();
    if (failures) {
      std::fprintf(stderr, "%d checks failed\n", failures);
      return 1;
    }
    std::printf("ok\n");
    return 0;
  }
  const std::vector<Case> cases = {
      {{{7, 8}, {5, 3}, {16}}, {}},
      {{{0, 4}, {1}, {2, 3, 4}, {9}, {13, 1, 2}}, {}},
      {{{4097, 8}, {1009, 8}, {5, 64}, {3}}, {}},
      {{{6, 8}, {4, 16, 3}, {5, 3, 8}, {7, 3}, {16}, {64, 1024}, {3, 4, 8}}, {1, 1, 2, 0, 0, 1, 2}},
      {{{96, 64}, {7, 40}, {3}, {33, 128}, {5, 24, 2}, {2, 2048}, {9, 8}}, {1, 1, 0, 1, 1, 1, 1}},
      // row pitches that are not multiples of 16 bytes (unit-wise blocks)
      {{{64, 6}, {33, 12, 3}, {9, 20}, {1000, 6}, {3, 2050, 1}, {5, 8, 3}, {2, 1030, 4}, {7, 4, 5}},
       {1, 1, 1, 1, 1, 1, 1, 1}},
      {{{33, 4, 3}, {9, 12}, {7, 4, 5}, {100, 12}, {5}}, {1, 1, 1, 1, 0}},
      // rows too long for one chunk at per-row alignments (flat chunks)
      {{{3, 4098}, {9, 8}}, {1, 0}},
      {{{5, 8248}, {7, 16}}, {1, 1}},
      {{}, {}},
  };
  for (size_t ci = 0; ci < cases.size(); ++ci) {
    for (int32_t S : {1, 2, 4, 8}) {
      const Case& c = cases[ci];
      bool divisible = true;
      for (size_t i = 0; i < c.dims.size(); ++i)
        if (c.dims[i] != 0 && c.shapes[i][(size_t)c.dims[i]] % S) divisible = false;
      if (!divisible) continue;
      for (int32_t es : {2, 4})
        for (bool mis : {false, true}) {
          run_case(c, S, S, es, mis);
          run_case(c, S, 2 * S, es, mis);
        }
    }
  }
  fsdp_release_cache();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
