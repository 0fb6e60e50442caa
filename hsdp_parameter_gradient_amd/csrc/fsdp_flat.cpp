// Host side of the FSDP/HSDP flat-buffer library: argument validation, the
// dim-0 layout planner, descriptor-table construction and caching, and the
// extern "C" entry points declared in include/fsdp_flat.h.
//
// Layout rules implemented here (cited by page title and section):
//   FSDP dim-0 non-uniform sharding RFC (mindspore/hyper-parallel issue
//   319) 6.4: chunk = ceil(N0 / S); rank s holds rows starting at
//   min(s*chunk, N0), at most chunk of them, clamped to N0; the
//   communication storage of every rank has chunk rows (zero padded at the
//   tail); fused offsets advance by the padded element count.
//   Hyper communication-overlap PR #758 write-up (mindspore/hyper-parallel
//   issue 184) 2.1: the AG send buffer is this rank's slice of the AG
//   output; RS outputs are written as views into a 512-byte-aligned fused
//   buffer that one all-reduce covers.
//   FullyShard multi-dimensional RFC (yide12/hyper-parallel issue 1) 2.2.2
//   and 2.2.5: dp_size = rank_size / shard_size; RS when shard_size > 1,
//   AR when dp_size > 1.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <list>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <unordered_map>
#include <vector>

#include "fsdp_flat.h"
#include "plan.hpp"
#include "tuning.hpp"

#ifdef FSDP_TABLE_HOOK
// Test builds only (the host sanitizer driver): every planned table is
// handed to this function before its upload (reduce: 0 copy, 1 reduce,
// 3 fold copy, 4 fold reduce; elt: element bytes of a copy, dtype code of a
// reduction), so the tables the planner really builds can be checked
// against an emulation of the kernels.
void fsdp_table_hook(int reduce, int elt, uint32_t n_items, uint64_t n_chunks, uint32_t shift,
                     const std::vector<uint8_t>& table);
#endif

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_err = buf;
  } catch (...) {  // no memory for the message: the code still stands
    g_err.clear();
  }
  return code;
}

int ok() {
  g_err.clear();
  return FSDP_OK;
}

constexpr int64_t kMaxBytes = int64_t(1) << 60;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_mul_overflow(a, b, out) && *out <= kMaxBytes;
}
bool add_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_add_overflow(a, b, out) && *out <= kMaxBytes;
}

// Per parameter i sharded on dim k: outer = product of the dims before k,
// dk = dim k, inner = product of the dims after k; rank s holds rows
// [row_off, row_off + row_len) along k, i.e. outer runs of row_len*inner
// elements; its region in a rank slice is padded = outer*chunk*inner.
struct Layout {
  int32_t P = 0;
  int32_t S = 1;
  int64_t I = 0;
  std::vector<int64_t> chunk, inner, outer, dk, padded, in_off, numel;
  std::vector<int64_t> row_off, row_len;  // [i*S + s]
};

int make_layout(const fsdp_bucket_t* b, int32_t S, Layout* L) {
  if (!b) return fail(FSDP_EINVAL, "bucket is NULL");
  if (S < 1) return fail(FSDP_EINVAL, "shard_size %d < 1", S);
  if (b->n_params < 0) return fail(FSDP_EINVAL, "n_params %d < 0", b->n_params);
  if (b->n_params > 0 && (!b->ndim || !b->shape))
    return fail(FSDP_EINVAL, "ndim / shape arrays are NULL");
  L->P = b->n_params;
  L->S = S;
  for (auto* v : {&L->chunk, &L->inner, &L->outer, &L->dk, &L->padded, &L->in_off, &L->numel})
    v->resize(L->P);
  L->row_off.resize((size_t)L->P * S);
  L->row_len.resize((size_t)L->P * S);
  int64_t off = 0;
  size_t pos = 0;
  for (int32_t i = 0; i < L->P; ++i) {
    const int32_t nd = b->ndim[i];
    if (nd < 1) return fail(FSDP_EINVAL, "param %d: ndim %d < 1 (a 0-d tensor has no dim to shard)", i, nd);
    const int64_t* sh = b->shape + pos;
    pos += (size_t)nd;
    const int32_t k = b->shard_dims ? b->shard_dims[i] : b->shard_dim;
    if (k < 0 || k >= nd) return fail(FSDP_EINVAL, "param %d: shard dim %d outside [0, %d)", i, k, nd);
    int64_t outer = 1, inner = 1;
    for (int32_t d = 0; d < nd; ++d) {
      if (sh[d] < 0) return fail(FSDP_EINVAL, "param %d: negative dim %lld", i, (long long)sh[d]);
      if (d < k && !mul_ok(outer, sh[d], &outer)) return fail(FSDP_EINVAL, "param %d: size overflow", i);
      if (d > k && !mul_ok(inner, sh[d], &inner)) return fail(FSDP_EINVAL, "param %d: size overflow", i);
    }
    const int64_t n0 = sh[k];
    int64_t chunk;
    if (k == 0) {
      chunk = n0 / S + (n0 % S != 0);
    } else {
      if (n0 % S)
        return fail(FSDP_ENOTIMPL, "param %d: dim %d of size %lld is not divisible by shard_size %d "
                    "(only dim 0 may be uneven)", i, k, (long long)n0, S);
      chunk = n0 / S;
    }
    int64_t padded, numel, t;
    if (!mul_ok(outer, chunk, &t) || !mul_ok(t, inner, &padded) || !mul_ok(outer, n0, &t) ||
        !mul_ok(t, inner, &numel))
      return fail(FSDP_EINVAL, "param %d: size overflow", i);
    L->chunk[i] = chunk;
    L->inner[i] = inner;
    L->outer[i] = outer;
    L->dk[i] = n0;
    L->padded[i] = padded;
    L->numel[i] = numel;
    L->in_off[i] = off;
    for (int32_t s = 0; s < S; ++s) {
      const int64_t start = std::min<int64_t>((int64_t)s * chunk, n0);
      L->row_off[(size_t)i * S + s] = start;
      L->row_len[(size_t)i * S + s] = std::min<int64_t>(chunk, n0 - start);
    }
    if (!add_ok(off, padded, &off)) return fail(FSDP_EINVAL, "bucket size overflow");
  }
  L->I = off;
  int64_t tmp;
  if (!mul_ok(L->I, S, &tmp) || !mul_ok(tmp, 4, &tmp)) return fail(FSDP_EINVAL, "bucket size overflow");
  return FSDP_OK;
}

int elem_size(int32_t dtype) {
  switch (dtype) {
    case FSDP_F32: return 4;
    case FSDP_BF16: return 2;
    case FSDP_F16: return 2;
    default: return 0;
  }
}

// Element size of a reduction dtype: fp32, or bf16 / fp16 (summed in fp32).
int reduce_elem_size(int32_t dtype) {
  return dtype == FSDP_F32 ? 4 : (dtype == FSDP_BF16 || dtype == FSDP_F16) ? 2 : 0;
}

int check_groups(int32_t R, int32_t S) {
  if (R < 1 || S < 1) return fail(FSDP_EINVAL, "rank_size %d / shard_size %d must be >= 1", R, S);
  if (R % S != 0) return fail(FSDP_EINVAL, "rank_size %d is not a multiple of shard_size %d", R, S);
  return FSDP_OK;
}

// ---------------------------------------------------------------------------
// pointer checks
// ---------------------------------------------------------------------------

struct Span {
  uint64_t a, b;  // [a, b)
  int id;
};

int check_ptr(const void* p, int64_t nbytes, uint64_t align, const char* what, long idx) {
  if (nbytes == 0) return FSDP_OK;
  if (!p) return fail(FSDP_EINVAL, "%s[%ld] is NULL but holds %lld bytes", what, idx, (long long)nbytes);
  if ((uint64_t)p % align)
    return fail(FSDP_EALIGN, "%s[%ld] = %p is not %llu-byte aligned", what, idx, p, (unsigned long long)align);
  return FSDP_OK;
}

// Outputs must be pairwise disjoint and disjoint from every input.
int check_overlap(std::vector<Span> outs, const std::vector<Span>& ins) {
  outs.erase(std::remove_if(outs.begin(), outs.end(), [](const Span& s) { return s.a == s.b; }), outs.end());
  std::sort(outs.begin(), outs.end(), [](const Span& x, const Span& y) { return x.a < y.a; });
  for (size_t k = 1; k < outs.size(); ++k)
    if (outs[k].a < outs[k - 1].b)
      return fail(FSDP_EOVERLAP, "output buffers %d and %d overlap", outs[k - 1].id, outs[k].id);
  for (const Span& in : ins) {
    if (in.a == in.b) continue;
    // first output whose end is beyond in.a
    auto it = std::upper_bound(outs.begin(), outs.end(), in.a,
                               [](uint64_t v, const Span& s) { return v < s.b; });
    if (it != outs.end() && it->a < in.b)
      return fail(FSDP_EOVERLAP, "input buffer %d overlaps output buffer %d", in.id, it->id);
  }
  return FSDP_OK;
}

// ---------------------------------------------------------------------------
// plan cache: per call signature, the call's descriptor table in device
// memory and its launch parameters.  A repeated call (same entry point,
// arguments, shapes and pointers, same device) skips validation, planning
// and the upload: its result depends on nothing else.
// ---------------------------------------------------------------------------

// Everything a call's result depends on, as 64-bit words.
class Key {
 public:
  explicit Key(uint64_t entry) {
    int device = 0;
    ok_ = hipGetDevice(&device) == hipSuccess;
    w_.push_back(entry);
    w_.push_back((uint64_t)device);
  }
  void add(int64_t v) { w_.push_back((uint64_t)v); }
  // false if the bucket's arrays cannot be read (validation then reports it)
  bool bucket(const fsdp_bucket_t* b) {
    if (!b || b->n_params < 0 || (b->n_params > 0 && (!b->ndim || !b->shape))) return ok_ = false;
    add(b->n_params);
    add(b->shard_dim);
    add(b->shard_dims ? 1 : 0);
    size_t nshape = 0;
    for (int32_t i = 0; i < b->n_params; ++i) {
      if (b->ndim[i] < 0) return ok_ = false;
      add(b->ndim[i]);
      nshape += (size_t)b->ndim[i];
    }
    for (size_t k = 0; k < nshape; ++k) add(b->shape[k]);
    if (b->shard_dims)
      for (int32_t i = 0; i < b->n_params; ++i) add(b->shard_dims[i]);
    return ok_;
  }
  bool ptrs(const void* const* p, int64_t n) {
    if (n < 0 || (n > 0 && !p)) return ok_ = false;
    for (int64_t k = 0; k < n; ++k) w_.push_back((uint64_t)p[k]);
    return ok_;
  }
  bool valid() const { return ok_; }
  uint64_t hash() const {
    uint64_t h = 1469598103934665603ull;
    for (uint64_t x : w_) {
      h ^= x;
      h *= 0x9E3779B97F4A7C15ull;
      h ^= h >> 29;
    }
    return h;
  }
  bool operator==(const Key& o) const { return w_ == o.w_; }

 private:
  std::vector<uint64_t> w_;
  bool ok_ = true;
};

enum : uint64_t { kAgCopyIn = 1, kAgCopyOut, kRsCopyIn, kRsReduce, kRsCopyReduce, kFusedAr };

// A prepared launch.
struct Plan {
  bool launch = false;  // false: nothing to enqueue
  bool reduce = false;  // seg_copy_kernel or reduce_kernel
  void* dev = nullptr;  // the descriptor table (owned by the cache entry)
  size_t bytes = 0;
  uint32_t n_items = 0;
  uint64_t n_chunks = 0;
  uint32_t shift = 0;
  int es = 0;  // copies: element bytes; reductions: the dtype code
  uint32_t nsrc = 0;
  int avg = 0;
  int nts = 0;
  // a second launch for the call's fold items (fold_copy_kernel, or
  // fold_reduce_kernel with the dtype code, operand count and op), if any
  void* fold_dev = nullptr;
  size_t fold_bytes = 0;
  uint32_t fold_items = 0;
  uint64_t fold_chunks = 0;
  int fold_nts = 0;
  bool fold_reduce = false;
  bool fold_narrow = false;  // every fold item's unit is 2 or 4 bytes
  int fold_elt = 0;
  uint32_t fold_nsrc = 0;
  int fold_avg = 0;
  int device = 0;  // the device whose memory holds the tables

  size_t table_bytes() const { return bytes + fold_bytes; }
  void free_tables() const {
    if (dev) (void)hipFree(dev);
    if (fold_dev) (void)hipFree(fold_dev);
  }
};

struct Entry {
  Key key;
  uint64_t hash;
  Plan plan;
  // launched into a stream capture: a HIP graph holds the table's address,
  // so the plan is never evicted (only fsdp_release_cache frees it)
  bool pinned = false;
};

constexpr size_t kMaxEntries = 256;
constexpr size_t kMaxTableBytes = size_t(256) << 20;

std::mutex g_mu;
std::list<Entry> g_lru;  // front = most recent
std::unordered_map<uint64_t, std::vector<std::list<Entry>::iterator>> g_index;
size_t g_table_bytes = 0;

void drop_entry(std::list<Entry>::iterator it) {
  auto& v = g_index[it->hash];
  v.erase(std::remove(v.begin(), v.end(), it), v.end());
  if (v.empty()) g_index.erase(it->hash);
  it->plan.free_tables();
  g_table_bytes -= it->plan.table_bytes();
  g_lru.erase(it);
}

// Is `stream` being captured into a HIP graph?
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

// Events the calling thread's next kernel launch records at its start and
// end (fsdp_time_next_launch); taken by that launch.
thread_local void* g_time_start = nullptr;
thread_local void* g_time_stop = nullptr;

int enqueue(const Plan& p, hipStream_t stream) {
  if (!p.launch && !p.fold_dev) return ok();
  const uint32_t max_grid = fsdp::tuning().max_grid;
  // a pending timing request spans the whole call: the first kernel records
  // the start event, the last one the stop event (not in a launch into a
  // graph capture: the request then waits for the next launch outside one)
  void* t0 = nullptr;
  void* t1 = nullptr;
  if (g_time_start && !capturing(stream)) {
    t0 = g_time_start;
    t1 = g_time_stop;
    g_time_start = g_time_stop = nullptr;
  }
  if (p.launch) {
    void* stop = p.fold_dev ? nullptr : t1;  // a fold launch follows: it records the stop
    int he = p.reduce ? fsdp_launch_reduce(p.es, p.dev, p.n_items, p.nsrc, p.n_chunks, p.shift, max_grid, p.avg,
                                           p.nts, stream, t0, stop)
                      : fsdp_launch_seg_copy(p.es, p.dev, p.n_items, p.n_chunks, p.shift, max_grid, p.nts, stream,
                                             t0, stop);
    if (he != hipSuccess)
      return fail(FSDP_EHIP, "%s launch: %s", p.reduce ? "reduce" : "seg_copy", hipGetErrorString((hipError_t)he));
    t0 = nullptr;
  }
  if (p.fold_dev) {
    int he = p.fold_reduce ? fsdp_launch_fold_reduce(p.fold_elt, p.fold_dev, p.fold_items, p.fold_nsrc,
                                                     p.fold_chunks, max_grid, p.fold_narrow, p.fold_avg,
                                                     p.fold_nts, stream, t0, t1)
                           : fsdp_launch_fold(p.fold_dev, p.fold_items, p.fold_chunks, max_grid, p.fold_narrow,
                                              p.fold_nts, stream, t0, t1);
    if (he != hipSuccess)
      return fail(FSDP_EHIP, "%s launch: %s", p.fold_reduce ? "fold_reduce" : "fold_copy",
                  hipGetErrorString((hipError_t)he));
  }
  return ok();
}

// Launch the cached plan of `key`, if there is one.
bool launch_cached(const Key& key, hipStream_t stream, int* rc) {
  if (!key.valid()) return false;
  const uint64_t h = key.hash();
  std::lock_guard<std::mutex> lock(g_mu);
  auto found = g_index.find(h);
  if (found == g_index.end()) return false;
  for (auto it : found->second) {
    if (it->key == key) {
      g_lru.splice(g_lru.begin(), g_lru, it);
      if (!it->pinned && capturing(stream)) it->pinned = true;
      *rc = enqueue(it->plan, stream);
      return true;
    }
  }
  return false;
}

// Synchronize every device that holds a cached table (the key's second
// word is the device), then make the caller's device current again.
hipError_t sync_cached_devices() {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  std::vector<int> devs;
  for (const Entry& en : g_lru)
    if ((en.plan.dev || en.plan.fold_dev) && std::find(devs.begin(), devs.end(), en.plan.device) == devs.end())
      devs.push_back(en.plan.device);
  if (std::find(devs.begin(), devs.end(), cur) == devs.end()) devs.push_back(cur);
  for (int d : devs) {
    if ((e = hipSetDevice(d)) != hipSuccess) break;
    if ((e = hipDeviceSynchronize()) != hipSuccess) break;
  }
  const hipError_t r = hipSetDevice(cur);
  return e != hipSuccess ? e : r;
}

// Keep `plan` under `key` (evicting old plans first if needed) and launch it.
int store_and_launch(Key&& key, Plan&& plan, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  const size_t nb = plan.table_bytes();
  if (g_lru.size() >= kMaxEntries || g_table_bytes + nb > kMaxTableBytes) {
    // tables still in use by queued kernels must outlive them: wait for
    // every device that owns a cached table, not only the current one
    hipError_t e = sync_cached_devices();
    if (e != hipSuccess) {
      plan.free_tables();
      return fail(FSDP_EHIP, "device synchronize before evicting plans: %s", hipGetErrorString(e));
    }
    // least recent first; plans held by captured graphs stay
    for (auto it = g_lru.end();
         it != g_lru.begin() && (g_lru.size() >= kMaxEntries / 2 || g_table_bytes + nb > kMaxTableBytes / 2);) {
      auto victim = std::prev(it);
      if (victim->pinned)
        it = victim;
      else
        drop_entry(victim);
    }
  }
  const uint64_t h = key.hash();
  // the tables must not leak if the host bookkeeping cannot grow
  try {
    g_lru.push_front(Entry{std::move(key), h, plan});
  } catch (...) {
    plan.free_tables();
    throw;
  }
  try {
    g_index[h].push_back(g_lru.begin());
  } catch (...) {
    g_lru.pop_front();
    plan.free_tables();
    throw;
  }
  g_table_bytes += nb;
  return enqueue(g_lru.front().plan, stream);
}

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------

template <typename T>
void append(std::vector<uint8_t>& t, const T* p, size_t n) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(p);
  t.insert(t.end(), b, b + n * sizeof(T));
}

enum class Reuse { kReadNext, kFinal };

// Nontemporal stores for this output?  (the policy of fsdp::Tuning::cached_store_max)
bool stream_stores(Reuse reuse, uint64_t out_bytes) {
  return reuse == Reuse::kFinal || out_bytes > fsdp::tuning().cached_store_max;
}

// Upload a table (blocking copy into fresh device memory, so it is complete
// before anything is enqueued on any stream).
int upload_table(const std::vector<uint8_t>& table, void** dev, size_t* bytes, int* device) {
  hipError_t e = hipGetDevice(device);
  if (e != hipSuccess) return fail(FSDP_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  e = hipMalloc(dev, table.size());
  if (e != hipSuccess) {
    *dev = nullptr;
    return fail(FSDP_EHIP, "hipMalloc(%zu) for a descriptor table: %s", table.size(), hipGetErrorString(e));
  }
  if ((e = hipMemcpy(*dev, table.data(), table.size(), hipMemcpyHostToDevice)) != hipSuccess) {
    (void)hipFree(*dev);
    *dev = nullptr;
    return fail(FSDP_EHIP, "upload of a descriptor table: %s", hipGetErrorString(e));
  }
  *bytes = table.size();
  return FSDP_OK;
}

int upload(const std::vector<uint8_t>& table, Plan* p) { return upload_table(table, &p->dev, &p->bytes, &p->device); }

// Strided blocks: `rows` runs of row_bytes, row r from src + r*src_pitch to
// dst + r*dst_pitch.  The kernels move whole rows per chunk.  Pitches that
// are multiples of 16 keep every row at the alignment of the first (16-byte
// vectors); other pitches are moved in 8-, 4- or element-sized units, which
// beats one item (one workgroup) per row for short rows and for 8-byte
// units.  Rows longer than a chunk, and long rows of narrow units, go one
// item per row.
constexpr uint64_t kShortRow = 1024;

bool vector_rows(uint64_t src_pitch, uint64_t dst_pitch) { return src_pitch % 16 == 0 && dst_pitch % 16 == 0; }

bool rows_fit(uint64_t row_bytes, uint64_t rows, uint32_t shift) {
  return rows >= 2 && row_bytes > 0 && row_bytes <= (uint64_t(1) << shift);
}

// Rows per chunk of a strided copy block: as many whole rows as a chunk
// holds, or, for unit-wise rows, the fewest that fill it (one row may cross
// the chunk size).  Measured on MI355X, 4,120-byte rows of 8-byte units over
// 2 ranks ((20000, 1030, 4) fp16 sharded on dim 1): four rows per 16 KiB
// chunk instead of three, RS copy-in 132 -> 115 us, AG copy-out 63 -> 60 us;
// twice the chunk size was slower than both.
uint64_t block_rows_per_chunk(uint64_t src_pitch, uint64_t dst_pitch, uint64_t row_bytes, uint32_t shift) {
  const uint64_t CH = uint64_t(1) << shift;
  return vector_rows(src_pitch, dst_pitch) ? CH / row_bytes : (CH + row_bytes - 1) / row_bytes;
}

bool copy_block_ok(uint64_t src, uint64_t dst, uint64_t src_pitch, uint64_t dst_pitch, uint64_t row_bytes,
                   uint64_t rows, uint32_t shift) {
  if (!rows_fit(row_bytes, rows, shift)) return false;
  if (vector_rows(src_pitch, dst_pitch)) return true;
  // unit-wise rows: a chunk's rows lie within 4 GiB of its first row (the
  // kernel's offsets are 32-bit)
  const uint64_t per = block_rows_per_chunk(src_pitch, dst_pitch, row_bytes, shift);
  if (per * std::max(src_pitch, dst_pitch) >= (uint64_t(1) << 32)) return false;
  return row_bytes <= kShortRow || ((src | dst | src_pitch | dst_pitch | row_bytes) & 7u) == 0;
}

// The reduction kernel moves rows of other pitches element by element.
bool reduce_block_ok(uint64_t src_pitch, uint64_t dst_pitch, uint64_t row_bytes, uint64_t rows, uint32_t shift) {
  return rows_fit(row_bytes, rows, shift) && (vector_rows(src_pitch, dst_pitch) || row_bytes <= kShortRow);
}

void push_rows(std::vector<fsdp::CopySeg>& segs, uint64_t src, uint64_t dst, uint64_t row_bytes, uint64_t rows,
               uint64_t src_pitch, uint64_t dst_pitch) {
  if (row_bytes == 0 || rows == 0) return;
  const uint32_t shift = fsdp::tuning().copy_shift;
  if (copy_block_ok(src, dst, src_pitch, dst_pitch, row_bytes, rows, shift)) {
    fsdp::CopySeg sg{src, dst, row_bytes, row_bytes};
    sg.rows = rows;
    sg.src_pitch = src_pitch;
    sg.dst_pitch = dst_pitch;
    sg.rows_per_chunk = block_rows_per_chunk(src_pitch, dst_pitch, row_bytes, shift);
    segs.push_back(sg);
    return;
  }
  for (uint64_t r = 0; r < rows; ++r)
    segs.push_back({src + r * src_pitch, dst + r * dst_pitch, row_bytes, row_bytes});
}

// Short rows of dim-k chunks: every cache line of the full tensor holds
// pieces of several shard ranks' rows.  The S ranks' items for the same rows
// are emitted next to each other, one item per chunk of rows, so that the
// XCD-aware chunk order runs them back to back on one XCD, whose L2 then
// merges the partial-line reads and writes.
constexpr uint64_t kInterleaveRow = 256;

bool interleave_rows(uint64_t row_bytes, uint64_t rows) {
  return row_bytes > 0 && row_bytes < kInterleaveRow && rows >= 2;
}

// Dim-k chunk rows that the fold kernels take, over S ranks: short rows,
// or longer ones that are not a multiple of m bytes (each rank's rows then
// sit at their own alignment, which the fold absorbs), when the S pieces of
// a full-tensor row fit a chunk of CH bytes.  Copies use m = 8 (unit-wise
// blocks of 8-byte units are as fast), the RS copy-reduce m = 16 (its rows
// at other pitches go element by element or one job per row).  Measured on
// MI355X for the long ones against one item (or job) per row or unit-wise
// blocks: (30000, 2050, 1) bf16 over 2 ranks AG copy-out / RS copy-in / RS
// copy-reduce 156 / 324 / 276 -> 54 / 97 / 85 us; (20000, 1540) bf16 over 4
// ranks 42 / 109 / 111 -> 30 / 94 / 59 us; (20000, 1030, 4) fp16 over 2
// ranks (8-byte units) RS copy-reduce 205 -> 109 us.
bool fold_rows(uint64_t row_bytes, uint64_t rows, uint64_t S, uint64_t CH, uint64_t m) {
  if (S < 2 || rows < 2 || row_bytes == 0 || S * row_bytes > CH) return false;
  return row_bytes < kInterleaveRow || row_bytes % m != 0;
}

// Dim-k chunk rows too long for the S pieces of a full-tensor row to fit one
// chunk, at per-row alignments (not a multiple of m bytes): the full tensor
// is cut into flat chunks of kFlatChunk bytes whatever rows they cross
// (rows_per_chunk 0 in the fold items), staged through LDS so that both
// sides move aligned vectors.  Pieces of at least kFlatMinRun bytes keep the
// pieces meeting one chunk few (plan.hpp).
using fsdp::kFlatChunk;
using fsdp::kFlatMinRun;

bool long_rows(uint64_t row_bytes, uint64_t rows, uint64_t S, uint64_t CH, uint64_t m) {
  return S >= 2 && rows >= 2 && S * row_bytes > CH && row_bytes >= kFlatMinRun && row_bytes % m != 0 &&
         S * row_bytes <= (uint64_t(1) << 31);
}

// The S ranks' rows of one parameter: base[s] = (first source row, first
// destination row) of rank s; the same row length, row count and pitches.
void push_rows_interleaved(std::vector<fsdp::CopySeg>& segs, const std::vector<std::pair<uint64_t, uint64_t>>& base,
                           uint64_t row_bytes, uint64_t rows, uint64_t src_pitch, uint64_t dst_pitch) {
  const uint64_t per = (uint64_t(1) << fsdp::tuning().copy_shift) / row_bytes;
  for (uint64_t r0 = 0; r0 < rows; r0 += per) {
    const uint64_t nr = std::min(per, rows - r0);
    for (const auto& b : base)
      push_rows(segs, b.first + r0 * src_pitch, b.second + r0 * dst_pitch, row_bytes, nr, src_pitch, dst_pitch);
  }
}

// A fold item for one parameter over all S ranks (rank s's first row at
// rank0 + s*rank_pitch), when its dim-k chunk rows are short and the S
// pieces of a full-tensor row fit a chunk; false otherwise.  The access
// width is the widest of 16, 8, 4 and 2 bytes that divides the row length,
// both bases and the rank pitch.  Measured on MI355X against the ranks'
// interleaved blocks: gathering (AG copy-out) is faster at every width
// (up to 2.9x); scattering (RS copy-in) is faster with 8- and 16-byte
// units (up to 1.5x) and, staged through LDS, with 2- and 4-byte ones (up
// to 2.4x).
bool push_fold(std::vector<fsdp::FoldSeg>& folds, uint64_t full, uint64_t rank0, uint64_t rank_pitch, int32_t S,
               uint64_t row_bytes, uint64_t rows, int es, bool gather) {
  const uint64_t CH = uint64_t(1) << fsdp::tuning().copy_shift;
  const bool whole = fold_rows(row_bytes, rows, (uint64_t)S, CH, 8);
  if (!whole && !long_rows(row_bytes, rows, (uint64_t)S, CH, 8)) return false;
  const uint64_t m = full | row_bytes | rank0 | rank_pitch;
  const uint32_t unit = (m & 15u) == 0 ? 16u : (m & 7u) == 0 ? 8u : (m & 3u) == 0 ? 4u : 2u;
  if (unit < (uint32_t)es) return false;
  fsdp::FoldSeg f{};
  f.full = full;
  f.run_bytes = row_bytes;
  f.rows = rows;
  f.rows_per_chunk = whole ? CH / ((uint64_t)S * row_bytes) : 0;  // 0: flat chunks
  f.reserved = whole ? 0u : (uint32_t)kFlatChunk;
  f.rank0 = rank0;
  f.rank_pitch = rank_pitch;
  f.nrank = (uint32_t)S;
  f.unit = unit;
  f.gather = gather ? 1u : 0u;
  folds.push_back(f);
  return true;
}

// A fold-reduce item for one parameter over one shard group (operand t's
// full gradient at src[t], rank s's rows at dst[s]), when its dim-k chunk
// rows are short and the S pieces of a full-tensor row fit a reduce chunk;
// false otherwise.  The access width is the widest of 16, 8, 4 and 2 bytes
// that divides the row length and every pointer, and at least the element.
// Largest chunk of a fold-reduce item: the reduce chunk, or the copy chunk
// when that is larger (the fold's LDS staging holds either).
uint64_t fold_reduce_max_chunk() {
  const fsdp::Tuning& tu = fsdp::tuning();
  return uint64_t(1) << std::max(tu.reduce_shift, tu.copy_shift);
}

bool push_fold_reduce(std::vector<fsdp::FoldRed>& items, std::vector<uint64_t>& ptrs, const std::vector<uint64_t>& src,
                      const std::vector<uint64_t>& dst, uint64_t row_bytes, uint64_t rows, int es) {
  const uint64_t CH = uint64_t(1) << fsdp::tuning().reduce_shift;
  const uint64_t CHX = fold_reduce_max_chunk();
  const uint64_t S = src.size();
  if (dst.size() != S) return false;
  const bool whole = fold_rows(row_bytes, rows, S, CHX, 16);
  // flat chunks are staged through LDS block by block, which needs every
  // operand at the same address modulo 16
  bool same16 = true;
  for (uint64_t a : src) same16 = same16 && ((a ^ src[0]) & 15u) == 0;
  if (!whole && !(same16 && long_rows(row_bytes, rows, S, CHX, 16))) return false;
  uint64_t m = row_bytes;
  for (uint64_t a : src) m |= a;
  for (uint64_t a : dst) m |= a;
  const uint32_t unit = (m & 15u) == 0 ? 16u : (m & 7u) == 0 ? 8u : (m & 3u) == 0 ? 4u : 2u;
  if (unit < (uint32_t)es) return false;
  fsdp::FoldRed f{};
  f.run_bytes = row_bytes;
  f.rows = rows;
  // reduce-sized chunks, or larger ones where a reduce chunk would hold
  // one full row and leave most of itself empty (measured on MI355X:
  // (30000, 2050, 1) bf16 over 2 ranks 85 -> 67 us; short rows lose 2-4 %
  // with the larger chunks); where the kernel never stages the chunks
  // through LDS, kFoldUnitChunk bytes and at least two rows (measured on
  // MI355X, RS copy-reduce over 2 ranks against reduce-sized chunks:
  // (20000, 1030, 4) fp16 110 -> 84 us, short rows of 8 to 128 bytes 6-15 %
  // faster; 32 KiB chunks were 3-10 % slower than 16 KiB on short rows);
  // 0: flat chunks of kFlatChunk bytes
  const bool units_only = unit > fsdp::kFoldLdsMaxUnit && S < 4;
  f.rows_per_chunk = !whole        ? 0
                     : units_only ? std::max<uint64_t>(2, fsdp::kFoldUnitChunk / (S * row_bytes))
                     : 2 * S * row_bytes <= CH ? CH / (S * row_bytes)
                                               : CHX / (S * row_bytes);
  f.reserved[0] = whole ? 0 : kFlatChunk;
  f.src0 = (uint32_t)ptrs.size();
  ptrs.insert(ptrs.end(), src.begin(), src.end());
  f.dst0 = (uint32_t)ptrs.size();
  ptrs.insert(ptrs.end(), dst.begin(), dst.end());
  f.nrank = (uint32_t)S;
  f.unit = unit;
  items.push_back(f);
  return true;
}

// Output bytes of a call's fold items.
uint64_t fold_out_bytes(const std::vector<fsdp::FoldSeg>& folds) {
  uint64_t n = 0;
  for (const auto& f : folds) n += f.rows * f.nrank * f.run_bytes;
  return n;
}

// Plan the segmented copy over `segs` into *table (uploaded by the caller;
// other_out: the output bytes of the call's other launch, for the store
// policy).
int plan_copy(std::vector<fsdp::CopySeg>& segs, int es, Reuse reuse, uint64_t other_out, Plan* p,
              std::vector<uint8_t>* table) {
  // the chunk prefix and the per-chunk item map need every item non-empty
  segs.erase(std::remove_if(segs.begin(), segs.end(), [](const fsdp::CopySeg& sg) { return sg.total_bytes == 0; }),
             segs.end());
  if (segs.empty()) return FSDP_OK;
  if (segs.size() > 0xffffffffu) return fail(FSDP_EINVAL, "too many segments");
  const fsdp::Tuning& tu = fsdp::tuning();
  std::vector<uint64_t> begin(segs.size());
  uint64_t n = 0, out_bytes = 0;
  for (size_t k = 0; k < segs.size(); ++k) {
    begin[k] = n;
    n += fsdp::item_chunks(segs[k].dst, segs[k].total_bytes, segs[k].rows, segs[k].rows_per_chunk, tu.copy_shift);
    out_bytes += segs[k].total_bytes * segs[k].rows;
  }
  // the kernel indexes chunks and its grid with 32-bit integers
  if (n >= (uint64_t(1) << 31)) return fail(FSDP_EINVAL, "too many copy chunks (%llu)", (unsigned long long)n);
  // item_of[c]: the item of chunk c (the kernel's one-load item lookup)
  std::vector<uint32_t> item_of(n);
  for (size_t k = 0; k < segs.size(); ++k) {
    const uint64_t e = k + 1 < segs.size() ? begin[k + 1] : n;
    std::fill(item_of.begin() + begin[k], item_of.begin() + e, (uint32_t)k);
  }
  table->reserve(begin.size() * 8 + segs.size() * sizeof(fsdp::CopySeg) + item_of.size() * 4);
  append(*table, begin.data(), begin.size());
  append(*table, segs.data(), segs.size());
  append(*table, item_of.data(), item_of.size());
#ifdef FSDP_TABLE_HOOK
  fsdp_table_hook(0, es, (uint32_t)segs.size(), n, tu.copy_shift, *table);
#endif
  p->launch = true;
  p->reduce = false;
  p->n_items = (uint32_t)segs.size();
  p->n_chunks = n;
  p->shift = tu.copy_shift;
  p->es = es;
  p->nts = stream_stores(reuse, out_bytes + other_out);
  return FSDP_OK;
}

// Chunks of a fold or fold-reduce item: whole full rows per chunk, or with
// rows_per_chunk 0 flat chunks of sub bytes of the whole full tensor.
uint64_t fold_item_chunks(uint64_t rows, uint64_t rows_per_chunk, uint64_t full_row, uint64_t sub) {
  if (rows_per_chunk == 0) return (rows * full_row + sub - 1) / sub;
  return (rows + rows_per_chunk - 1) / rows_per_chunk;
}

// Plan the fold items of a copy (a launch of its own) into *table.
int plan_fold(const std::vector<fsdp::FoldSeg>& folds, int es, Reuse reuse, uint64_t other_out, Plan* p,
              std::vector<uint8_t>* table) {
  (void)es;  // element bytes: only the test builds' table hook reports them
  if (folds.empty()) return FSDP_OK;
  if (folds.size() > 0xffffffffu) return fail(FSDP_EINVAL, "too many fold items");
  std::vector<uint64_t> begin(folds.size());
  uint64_t n = 0;
  for (size_t k = 0; k < folds.size(); ++k) {
    begin[k] = n;
    n += fold_item_chunks(folds[k].rows, folds[k].rows_per_chunk, folds[k].nrank * folds[k].run_bytes,
                     folds[k].reserved);
  }
  append(*table, begin.data(), begin.size());
  append(*table, folds.data(), folds.size());
#ifdef FSDP_TABLE_HOOK
  fsdp_table_hook(3, es, (uint32_t)folds.size(), n, fsdp::tuning().copy_shift, *table);
#endif
  p->fold_items = (uint32_t)folds.size();
  p->fold_chunks = n;
  p->fold_nts = stream_stores(reuse, fold_out_bytes(folds) + other_out);
  p->fold_narrow = std::all_of(folds.begin(), folds.end(), [](const fsdp::FoldSeg& f) { return f.unit <= 4; });
  return FSDP_OK;
}

// Plan the reduction over `jobs` (every job with the same operand count)
// into *table (uploaded by the caller; other_out: the output bytes of the
// call's other launch, for the store policy).
int plan_reduce(std::vector<fsdp::RedJob>& jobs, std::vector<uint64_t>& ptrs, int dtype, int avg, Reuse reuse,
                uint64_t other_out, Plan* p, std::vector<uint8_t>* table) {
  jobs.erase(std::remove_if(jobs.begin(), jobs.end(), [](const fsdp::RedJob& jb) { return jb.nbytes == 0; }),
             jobs.end());
  if (jobs.empty()) return FSDP_OK;
  if (jobs.size() > 0xffffffffu || ptrs.size() > 0xffffffffu) return fail(FSDP_EINVAL, "too many jobs");
  const fsdp::Tuning& tu = fsdp::tuning();
  std::vector<uint64_t> begin(jobs.size());
  uint64_t n = 0, out_bytes = 0;
  for (size_t k = 0; k < jobs.size(); ++k) {
    begin[k] = n;
    n += fsdp::item_chunks(ptrs[jobs[k].dst0], jobs[k].nbytes, jobs[k].rows, jobs[k].rows_per_chunk,
                           tu.reduce_shift);
    out_bytes += jobs[k].nbytes * jobs[k].ndst * jobs[k].rows;
  }
  append(*table, begin.data(), begin.size());
  append(*table, jobs.data(), jobs.size());
  append(*table, ptrs.data(), ptrs.size());
#ifdef FSDP_TABLE_HOOK
  fsdp_table_hook(1, dtype, (uint32_t)jobs.size(), n, tu.reduce_shift, *table);
#endif
  p->launch = true;
  p->reduce = true;
  p->n_items = (uint32_t)jobs.size();
  p->n_chunks = n;
  p->shift = tu.reduce_shift;
  p->es = dtype;
  p->nsrc = jobs[0].nsrc;
  p->avg = avg;
  p->nts = stream_stores(reuse, out_bytes + other_out);
  return FSDP_OK;
}

// Output bytes of a call's fold-reduce items.
uint64_t fold_reduce_out_bytes(const std::vector<fsdp::FoldRed>& items) {
  uint64_t n = 0;
  for (const auto& f : items) n += f.rows * f.nrank * f.run_bytes;
  return n;
}

// Plan the fold-reduce items of a reduction (a launch of its own; every
// item with the same operand count) into *table.
int plan_fold_reduce(const std::vector<fsdp::FoldRed>& items, const std::vector<uint64_t>& ptrs, int dtype, int avg,
                     Reuse reuse, uint64_t other_out, Plan* p, std::vector<uint8_t>* table) {
  if (items.empty()) return FSDP_OK;
  if (items.size() > 0xffffffffu || ptrs.size() > 0xffffffffu) return fail(FSDP_EINVAL, "too many fold items");
  std::vector<uint64_t> begin(items.size());
  uint64_t n = 0;
  for (size_t k = 0; k < items.size(); ++k) {
    begin[k] = n;
    n += fold_item_chunks(items[k].rows, items[k].rows_per_chunk, items[k].nrank * items[k].run_bytes,
                     items[k].reserved[0]);
  }
  append(*table, begin.data(), begin.size());
  append(*table, items.data(), items.size());
  append(*table, ptrs.data(), ptrs.size());
#ifdef FSDP_TABLE_HOOK
  fsdp_table_hook(4, dtype, (uint32_t)items.size(), n,
                  std::max(fsdp::tuning().reduce_shift, fsdp::tuning().copy_shift), *table);
#endif
  p->fold_items = (uint32_t)items.size();
  p->fold_chunks = n;
  p->fold_nts = stream_stores(reuse, fold_reduce_out_bytes(items) + other_out);
  p->fold_reduce = true;
  p->fold_narrow = std::all_of(items.begin(), items.end(), [](const fsdp::FoldRed& f) { return f.unit <= 4; });
  p->fold_elt = dtype;
  p->fold_nsrc = items[0].nrank;
  p->fold_avg = avg;
  return FSDP_OK;
}

// A call without a cached plan allocates and uploads its tables (and may
// evict, which synchronizes devices): refused while its stream is being
// captured, before anything could invalidate the capture.
int check_not_capturing(hipStream_t stream) {
  if (capturing(stream))
    return fail(FSDP_EINVAL, "the first call of a signature cannot be captured into a graph: "
                "issue it once outside the capture");
  return FSDP_OK;
}

// Finish a validated call: plan it, cache the plan and launch it.
int run_copy(Key&& key, std::vector<fsdp::CopySeg>& segs, int es, Reuse reuse, hipStream_t stream,
             const std::vector<fsdp::FoldSeg>& folds = {}) {
  if (int rc = check_not_capturing(stream)) return rc;
  uint64_t seg_out = 0;
  for (const auto& sg : segs) seg_out += sg.total_bytes * sg.rows;
  Plan p;
  std::vector<uint8_t> seg_table, fold_table;
  int rc = plan_copy(segs, es, reuse, fold_out_bytes(folds), &p, &seg_table);
  if (!rc) rc = plan_fold(folds, es, reuse, seg_out, &p, &fold_table);
  // both tables are built before either is uploaded
  if (!rc && !seg_table.empty()) rc = upload(seg_table, &p);
  if (!rc && !fold_table.empty()) rc = upload_table(fold_table, &p.fold_dev, &p.fold_bytes, &p.device);
  if (rc) {
    p.free_tables();
    return rc;
  }
  return store_and_launch(std::move(key), std::move(p), stream);
}

int run_reduce(Key&& key, std::vector<fsdp::RedJob>& jobs, std::vector<uint64_t>& ptrs, int dtype, int avg,
               Reuse reuse, hipStream_t stream, const std::vector<fsdp::FoldRed>& folds = {},
               const std::vector<uint64_t>& fold_ptrs = {}) {
  if (int rc = check_not_capturing(stream)) return rc;
  uint64_t job_out = 0;
  for (const auto& jb : jobs) job_out += jb.nbytes * jb.ndst * jb.rows;
  Plan p;
  std::vector<uint8_t> job_table, fold_table;
  int rc = plan_reduce(jobs, ptrs, dtype, avg, reuse, fold_reduce_out_bytes(folds), &p, &job_table);
  if (!rc) rc = plan_fold_reduce(folds, fold_ptrs, dtype, avg, reuse, job_out, &p, &fold_table);
  // both tables are built before either is uploaded
  if (!rc && !job_table.empty()) rc = upload(job_table, &p);
  if (!rc && !fold_table.empty()) rc = upload_table(fold_table, &p.fold_dev, &p.fold_bytes, &p.device);
  if (rc) {
    p.free_tables();
    return rc;
  }
  return store_and_launch(std::move(key), std::move(p), stream);
}

}  // namespace

// ===========================================================================
// entry points (wrapped below for the C ABI)
// ===========================================================================

namespace {

int bucket_layout_impl(const fsdp_bucket_t* bucket, int32_t shard_size, int64_t* slice_numel,
                       int64_t* padded, int64_t* in_off, int64_t* row_off, int64_t* row_len) {
  Layout L;
  int rc = make_layout(bucket, shard_size, &L);
  if (rc) return rc;
  if (slice_numel) *slice_numel = L.I;
  if (padded) std::copy(L.padded.begin(), L.padded.end(), padded);
  if (in_off) std::copy(L.in_off.begin(), L.in_off.end(), in_off);
  if (row_off) std::copy(L.row_off.begin(), L.row_off.end(), row_off);
  if (row_len) std::copy(L.row_len.begin(), L.row_len.end(), row_len);
  return ok();
}

int fused_layout_impl(int32_t n_seg, const int64_t* seg_numel, int32_t elem_bytes, int64_t* seg_off,
                      int64_t* fused_numel) {
  if (n_seg < 0) return fail(FSDP_EINVAL, "n_seg %d < 0", n_seg);
  if (n_seg > 0 && !seg_numel) return fail(FSDP_EINVAL, "seg_numel is NULL");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(FSDP_EINVAL, "elem_bytes %d not in {2, 4}", elem_bytes);
  const int64_t A = FSDP_FUSED_ALIGN_BYTES;
  int64_t end = 0;
  for (int32_t j = 0; j < n_seg; ++j) {
    if (seg_numel[j] < 0) return fail(FSDP_EINVAL, "segment %d: negative size", j);
    const int64_t start = (end + A - 1) / A * A;
    int64_t nb;
    if (!mul_ok(seg_numel[j], elem_bytes, &nb) || !add_ok(start, nb, &end))
      return fail(FSDP_EINVAL, "fused buffer size overflow");
    if (seg_off) seg_off[j] = start / elem_bytes;
  }
  if (fused_numel) *fused_numel = (end + A - 1) / A * A / elem_bytes;
  return ok();
}

int group_ranks_impl(int32_t rank_size, int32_t shard_size, int32_t* n_rs_groups, int32_t* rs_ranks,
                     int32_t* n_ar_groups, int32_t* ar_ranks) {
  int rc = check_groups(rank_size, shard_size);
  if (rc) return rc;
  const int32_t S = shard_size, D = rank_size / shard_size;
  if (n_rs_groups) *n_rs_groups = S > 1 ? D : 0;
  if (n_ar_groups) *n_ar_groups = D > 1 ? S : 0;
  if (rs_ranks && S > 1)
    for (int32_t d = 0; d < D; ++d)
      for (int32_t s = 0; s < S; ++s) rs_ranks[d * S + s] = d * S + s;
  if (ar_ranks && D > 1)
    for (int32_t s = 0; s < S; ++s)
      for (int32_t d = 0; d < D; ++d) ar_ranks[s * D + d] = d * S + s;
  return ok();
}

int ag_copy_in_impl(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype,
                    const void* const* shards, void* ag, void* stream) {
  Key key(kAgCopyIn);
  if (key.bucket(bucket)) {
    key.add(shard_size);
    key.add(dtype);
    key.add((int64_t)ag);
    key.ptrs(shards, (int64_t)shard_size * bucket->n_params);
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  Layout L;
  if ((rc = make_layout(bucket, shard_size, &L))) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "dtype %d is not supported", dtype);
  const int32_t S = L.S, P = L.P;
  const int64_t ag_bytes = (int64_t)S * L.I * es;
  if ((rc = check_ptr(ag, ag_bytes, es, "ag", 0))) return rc;
  if (S * (int64_t)P > 0 && !shards) return fail(FSDP_EINVAL, "shards array is NULL");
  std::vector<Span> ins;
  std::vector<fsdp::CopySeg> segs;
  segs.reserve((size_t)S * P);
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t i = 0; i < P; ++i) {
      const int64_t nb = L.outer[i] * L.row_len[(size_t)i * S + s] * L.inner[i] * es;
      const void* p = shards[(size_t)s * P + i];
      if ((rc = check_ptr(p, nb, es, "shards", (long)s * P + i))) return rc;
      ins.push_back({(uint64_t)p, (uint64_t)p + (uint64_t)nb, s * P + i});
      const int64_t total = L.padded[i] * es;
      if (total == 0) continue;
      segs.push_back({nb ? (uint64_t)p : 0, (uint64_t)ag + (uint64_t)((s * L.I + L.in_off[i]) * es),
                      (uint64_t)nb, (uint64_t)total});
    }
  }
  if ((rc = check_overlap({{(uint64_t)ag, (uint64_t)ag + (uint64_t)ag_bytes, -1}}, ins))) return rc;
  return run_copy(std::move(key), segs, es, Reuse::kReadNext, static_cast<hipStream_t>(stream));
}

int ag_copy_out_impl(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype, const void* ag,
                     void* const* full, void* stream) {
  Key key(kAgCopyOut);
  if (key.bucket(bucket)) {
    key.add(shard_size);
    key.add(dtype);
    key.add((int64_t)ag);
    key.ptrs(full, bucket->n_params);
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  Layout L;
  if ((rc = make_layout(bucket, shard_size, &L))) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "dtype %d is not supported", dtype);
  const int32_t S = L.S, P = L.P;
  const int64_t ag_bytes = (int64_t)S * L.I * es;
  if ((rc = check_ptr(ag, ag_bytes, es, "ag", 0))) return rc;
  if (P > 0 && !full) return fail(FSDP_EINVAL, "full array is NULL");
  std::vector<Span> outs;
  std::vector<fsdp::CopySeg> segs;
  std::vector<fsdp::FoldSeg> folds;
  for (int32_t i = 0; i < P; ++i) {
    const int64_t nb = L.numel[i] * es;
    if ((rc = check_ptr(full[i], nb, es, "full", i))) return rc;
    outs.push_back({(uint64_t)full[i], (uint64_t)full[i] + (uint64_t)nb, i});
    // rank s's chunk: outer runs of row_len*inner elements, dense in the
    // slice, at stride dk*inner in the full parameter
    auto src_of = [&](int32_t s) { return (uint64_t)ag + (uint64_t)((s * L.I + L.in_off[i]) * es); };
    auto dst_of = [&](int32_t s) {
      return (uint64_t)full[i] + (uint64_t)(L.row_off[(size_t)i * S + s] * L.inner[i] * es);
    };
    const uint64_t pitch = (uint64_t)(L.dk[i] * L.inner[i] * es);
    // a dim-k chunk (every rank the same run): all ranks' pieces of whole
    // full rows in one fold item where its rows allow it, else short rows
    // as the ranks' blocks interleaved per chunk of rows
    const uint64_t row = (uint64_t)(L.row_len[(size_t)i * S] * L.inner[i] * es);
    if (L.outer[i] > 1 &&
        push_fold(folds, (uint64_t)full[i], src_of(0), (uint64_t)(L.I * es), S, row, (uint64_t)L.outer[i], es, true))
      continue;
    if (L.outer[i] > 1 && interleave_rows(row, (uint64_t)L.outer[i])) {
      std::vector<std::pair<uint64_t, uint64_t>> base;
      for (int32_t s = 0; s < S; ++s) base.push_back({src_of(s), dst_of(s)});
      push_rows_interleaved(segs, base, row, (uint64_t)L.outer[i], row, pitch);
      continue;
    }
    for (int32_t s = 0; s < S; ++s) {
      const int64_t run = L.row_len[(size_t)i * S + s] * L.inner[i];
      push_rows(segs, src_of(s), dst_of(s), (uint64_t)(run * es), (uint64_t)L.outer[i], (uint64_t)(run * es), pitch);
    }
  }
  if ((rc = check_overlap(outs, {{(uint64_t)ag, (uint64_t)ag + (uint64_t)ag_bytes, -1}}))) return rc;
  return run_copy(std::move(key), segs, es, Reuse::kFinal, static_cast<hipStream_t>(stream), folds);
}

int rs_copy_in_impl(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dtype,
                    const void* const* grads, void* const* rs_in, void* stream) {
  Key key(kRsCopyIn);
  if (key.bucket(bucket)) {
    key.add(rank_size);
    key.add(shard_size);
    key.add(dtype);
    key.ptrs(grads, (int64_t)rank_size * bucket->n_params);
    key.ptrs(rs_in, rank_size);
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  if ((rc = check_groups(rank_size, shard_size))) return rc;
  Layout L;
  if ((rc = make_layout(bucket, shard_size, &L))) return rc;
  const int es = elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "dtype %d is not supported", dtype);
  const int32_t R = rank_size, S = L.S, P = L.P;
  const int64_t buf_bytes = (int64_t)S * L.I * es;
  if (!rs_in) return fail(FSDP_EINVAL, "rs_in array is NULL");
  if ((int64_t)R * P > 0 && !grads) return fail(FSDP_EINVAL, "grads array is NULL");
  std::vector<Span> outs, ins;
  std::vector<fsdp::CopySeg> segs;
  segs.reserve((size_t)R * S * P);
  for (int32_t g = 0; g < R; ++g) {
    if ((rc = check_ptr(rs_in[g], buf_bytes, es, "rs_in", g))) return rc;
    outs.push_back({(uint64_t)rs_in[g], (uint64_t)rs_in[g] + (uint64_t)buf_bytes, g});
    for (int32_t i = 0; i < P; ++i) {
      const void* gp = grads[(size_t)g * P + i];
      if ((rc = check_ptr(gp, L.numel[i] * es, es, "grads", (long)g * P + i))) return rc;
      ins.push_back({(uint64_t)gp, (uint64_t)gp + (uint64_t)(L.numel[i] * es), g * P + i});
    }
  }
  for (int32_t g = 0; g < R; ++g) {
    for (int32_t s = 0; s < S; ++s) {
      for (int32_t i = 0; i < P; ++i) {
        if (L.padded[i] == 0) continue;
        // outer runs of row_len*inner elements from the gradient (stride
        // dk*inner), dense in the slice, then the zero tail (a dim-0 chunk's
        // padding rows; outer is 1 there)
        const int64_t run = L.row_len[(size_t)i * S + s] * L.inner[i];
        const uint64_t src = (uint64_t)grads[(size_t)g * P + i] +
                             (uint64_t)(L.row_off[(size_t)i * S + s] * L.inner[i] * es);
        const uint64_t d0 = (uint64_t)rs_in[g] + (uint64_t)((s * L.I + L.in_off[i]) * es);
        const int64_t data = L.outer[i] * run;  // elements; the tail is padded - data
        if (L.outer[i] == 1) {
          segs.push_back({run ? src : 0, d0, (uint64_t)(run * es), (uint64_t)(L.padded[i] * es)});
          continue;
        }
        if (interleave_rows((uint64_t)(run * es), (uint64_t)L.outer[i]) ||
            fold_rows((uint64_t)(run * es), (uint64_t)L.outer[i], (uint64_t)S, uint64_t(1) << fsdp::tuning().copy_shift, 8) ||
            long_rows((uint64_t)(run * es), (uint64_t)L.outer[i], (uint64_t)S, uint64_t(1) << fsdp::tuning().copy_shift, 8))
          continue;  // below
        push_rows(segs, src, d0, (uint64_t)(run * es), (uint64_t)L.outer[i], (uint64_t)(L.dk[i] * L.inner[i] * es),
                  (uint64_t)(run * es));
        if (L.padded[i] > data)
          segs.push_back({0, d0 + (uint64_t)(data * es), 0, (uint64_t)((L.padded[i] - data) * es)});
      }
    }
  }
  // dim-k chunks (every rank the same run, no padding) whose rows the fold
  // takes, or short ones: all ranks' pieces of whole full gradient rows in
  // one fold item, else short rows as the S ranks' blocks of the same rows
  // next to each other, longer ones as each rank's block
  std::vector<fsdp::FoldSeg> folds;
  const uint64_t CHC = uint64_t(1) << fsdp::tuning().copy_shift;
  for (int32_t g = 0; g < R; ++g) {
    for (int32_t i = 0; i < P; ++i) {
      const uint64_t row = (uint64_t)(L.row_len[(size_t)i * S] * L.inner[i] * es);
      const uint64_t rows = (uint64_t)L.outer[i];
      if (L.padded[i] == 0 || L.outer[i] == 1 ||
          !(interleave_rows(row, rows) || fold_rows(row, rows, S, CHC, 8) || long_rows(row, rows, S, CHC, 8)))
        continue;
      auto rank_of = [&](int32_t s) { return (uint64_t)rs_in[g] + (uint64_t)((s * L.I + L.in_off[i]) * es); };
      auto grad_of = [&](int32_t s) {
        return (uint64_t)grads[(size_t)g * P + i] + (uint64_t)(L.row_off[(size_t)i * S + s] * L.inner[i] * es);
      };
      const uint64_t pitch = (uint64_t)(L.dk[i] * L.inner[i] * es);
      if (push_fold(folds, (uint64_t)grads[(size_t)g * P + i], rank_of(0), (uint64_t)(L.I * es), S, row, rows, es,
                    false))
        continue;
      if (interleave_rows(row, rows)) {
        std::vector<std::pair<uint64_t, uint64_t>> base;
        for (int32_t s = 0; s < S; ++s) base.push_back({grad_of(s), rank_of(s)});
        push_rows_interleaved(segs, base, row, rows, pitch, row);
        continue;
      }
      for (int32_t s = 0; s < S; ++s) push_rows(segs, grad_of(s), rank_of(s), row, rows, pitch, row);
    }
  }
  if ((rc = check_overlap(outs, ins))) return rc;
  return run_copy(std::move(key), segs, es, Reuse::kReadNext, static_cast<hipStream_t>(stream), folds);
}

int rs_reduce_impl(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dp_size,
                   int32_t op, int32_t dtype, const void* const* rs_in, void* const* rs_out, void* stream) {
  Key key(kRsReduce);
  if (key.bucket(bucket)) {
    for (int64_t v : {(int64_t)rank_size, (int64_t)shard_size, (int64_t)dp_size, (int64_t)op, (int64_t)dtype})
      key.add(v);
    key.ptrs(rs_in, rank_size);
    key.ptrs(rs_out, rank_size);
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  if ((rc = check_groups(rank_size, shard_size))) return rc;
  if (dp_size != rank_size / shard_size)
    return fail(FSDP_EINVAL, "dp_size %d != rank_size / shard_size = %d", dp_size, rank_size / shard_size);
  if (op != FSDP_SUM && op != FSDP_AVG) return fail(FSDP_EINVAL, "reduce op %d", op);
  const int es = reduce_elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "rs_reduce takes fp32, bf16 or fp16 (dtype %d)", dtype);
  Layout L;
  if ((rc = make_layout(bucket, shard_size, &L))) return rc;
  const int32_t R = rank_size, S = shard_size;
  const int64_t in_bytes = (int64_t)S * L.I * es, out_bytes = L.I * es;
  if (!rs_in || !rs_out) return fail(FSDP_EINVAL, "rs_in / rs_out array is NULL");
  std::vector<Span> outs, ins;
  for (int32_t g = 0; g < R; ++g) {
    if ((rc = check_ptr(rs_in[g], in_bytes, es, "rs_in", g))) return rc;
    if ((rc = check_ptr(rs_out[g], out_bytes, es, "rs_out", g))) return rc;
    ins.push_back({(uint64_t)rs_in[g], (uint64_t)rs_in[g] + (uint64_t)in_bytes, g});
    outs.push_back({(uint64_t)rs_out[g], (uint64_t)rs_out[g] + (uint64_t)out_bytes, g});
  }
  if ((rc = check_overlap(outs, ins))) return rc;
  if (out_bytes == 0) return ok();
  std::vector<fsdp::RedJob> jobs;
  std::vector<uint64_t> ptrs;
  for (int32_t g = 0; g < R; ++g) {
    const int32_t d = g / S, s = g % S;
    fsdp::RedJob jb;
    jb.nbytes = jb.data_bytes = (uint64_t)out_bytes;
    jb.src0 = (uint32_t)ptrs.size();
    jb.nsrc = (uint32_t)S;
    for (int32_t t = 0; t < S; ++t) ptrs.push_back((uint64_t)rs_in[d * S + t] + (uint64_t)(s * out_bytes));
    jb.dst0 = (uint32_t)ptrs.size();
    jb.ndst = 1;
    ptrs.push_back((uint64_t)rs_out[g]);
    jobs.push_back(jb);
  }
  return run_reduce(std::move(key), jobs, ptrs, dtype, op == FSDP_AVG, Reuse::kReadNext,
                    static_cast<hipStream_t>(stream));
}

// The jobs of an RS copy-reduce call (validated first), for the cached
// entry point and the one that allocates nothing.
struct CopyReducePlan {
  std::vector<fsdp::RedJob> jobs;
  std::vector<uint64_t> ptrs;
  std::vector<fsdp::FoldRed> folds;
  std::vector<uint64_t> fold_ptrs;
};

int plan_rs_copy_reduce(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dp_size,
                        int32_t op, int32_t dtype, const void* const* grads, void* const* rs_out,
                        CopyReducePlan* out) {
  int rc = FSDP_OK;
  if ((rc = check_groups(rank_size, shard_size))) return rc;
  if (dp_size != rank_size / shard_size)
    return fail(FSDP_EINVAL, "dp_size %d != rank_size / shard_size = %d", dp_size, rank_size / shard_size);
  if (op != FSDP_SUM && op != FSDP_AVG) return fail(FSDP_EINVAL, "reduce op %d", op);
  const int es = reduce_elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "rs_copy_reduce takes fp32, bf16 or fp16 (dtype %d)", dtype);
  Layout L;
  if ((rc = make_layout(bucket, shard_size, &L))) return rc;
  const int32_t R = rank_size, S = shard_size, P = L.P;
  const int64_t out_bytes = L.I * es;
  if (!rs_out) return fail(FSDP_EINVAL, "rs_out array is NULL");
  if ((int64_t)R * P > 0 && !grads) return fail(FSDP_EINVAL, "grads array is NULL");
  std::vector<Span> outs, ins;
  for (int32_t g = 0; g < R; ++g) {
    if ((rc = check_ptr(rs_out[g], out_bytes, es, "rs_out", g))) return rc;
    outs.push_back({(uint64_t)rs_out[g], (uint64_t)rs_out[g] + (uint64_t)out_bytes, g});
    for (int32_t i = 0; i < P; ++i) {
      const void* gp = grads[(size_t)g * P + i];
      if ((rc = check_ptr(gp, L.numel[i] * es, es, "grads", (long)g * P + i))) return rc;
      ins.push_back({(uint64_t)gp, (uint64_t)gp + (uint64_t)(L.numel[i] * es), g * P + i});
    }
  }
  if ((rc = check_overlap(outs, ins))) return rc;
  // one job per (rank g, parameter i): rank g's region of parameter i is the
  // sum over its shard group of chunk s of gradient i, then zeros
  std::vector<fsdp::RedJob> jobs;
  std::vector<uint64_t> ptrs;
  const uint64_t CH = uint64_t(1) << fsdp::tuning().reduce_shift;
  // rows [r0, r0 + nr) of rank g's chunk of parameter i (runs of `run`
  // elements, no tail) as one strided job, or one plain job for one row
  auto push_block = [&](int32_t g, int32_t i, uint64_t r0, uint64_t nr) {
    const int32_t d = g / S, s = g % S;
    const int64_t run = L.row_len[(size_t)i * S + s] * L.inner[i];
    const uint64_t pitch = (uint64_t)(L.dk[i] * L.inner[i] * es);
    const uint64_t src_off = (uint64_t)(L.row_off[(size_t)i * S + s] * L.inner[i] * es) + r0 * pitch;
    fsdp::RedJob jb;
    jb.nbytes = jb.data_bytes = (uint64_t)(run * es);
    jb.src0 = (uint32_t)ptrs.size();
    jb.nsrc = (uint32_t)S;
    for (int32_t t = 0; t < S; ++t) ptrs.push_back((uint64_t)grads[(size_t)(d * S + t) * P + i] + src_off);
    jb.dst0 = (uint32_t)ptrs.size();
    jb.ndst = 1;
    ptrs.push_back((uint64_t)rs_out[g] + (uint64_t)(L.in_off[i] * es) + r0 * jb.nbytes);
    if (nr > 1) {
      jb.rows = nr;
      jb.src_pitch = pitch;
      jb.dst_pitch = jb.nbytes;
      jb.rows_per_chunk = CH / jb.nbytes;
    }
    jobs.push_back(jb);
  };
  // Rank s's chunk of parameter i, for rank g = d*S + s: outer runs of
  // row_len*inner elements (stride dk*inner in the gradients, dense in the
  // output), then the zero tail.  block: one strided job fits (the rows fit
  // a chunk, both pitches keep the rows' alignment or the rows are short,
  // and there is no tail); else one job per run, the last one with the tail.
  auto block_ok = [&](int32_t i, int32_t s) {
    const int64_t run = L.row_len[(size_t)i * S + s] * L.inner[i];
    return L.padded[i] == L.outer[i] * run &&
           reduce_block_ok((uint64_t)(L.dk[i] * L.inner[i] * es), (uint64_t)(run * es), (uint64_t)(run * es),
                           (uint64_t)L.outer[i], fsdp::tuning().reduce_shift);
  };
  auto emit_rank = [&](int32_t g, int32_t i) {
    const int32_t d = g / S, s = g % S;
    const int64_t run = L.row_len[(size_t)i * S + s] * L.inner[i];
    const uint64_t src_off = (uint64_t)(L.row_off[(size_t)i * S + s] * L.inner[i] * es);
    const uint64_t out0 = (uint64_t)rs_out[g] + (uint64_t)(L.in_off[i] * es);
    const uint64_t pitch = (uint64_t)(L.dk[i] * L.inner[i] * es);
    if (block_ok(i, s)) {
      push_block(g, i, 0, (uint64_t)L.outer[i]);
      return;
    }
    for (int64_t o = 0; o < L.outer[i]; ++o) {
      const bool last = o + 1 == L.outer[i];
      const uint64_t row_src = src_off + (uint64_t)o * pitch;
      fsdp::RedJob jb;
      jb.nbytes = (uint64_t)((last ? L.padded[i] - o * run : run) * es);
      jb.data_bytes = (uint64_t)(run * es);
      jb.src0 = (uint32_t)ptrs.size();
      jb.nsrc = (uint32_t)S;
      for (int32_t t = 0; t < S; ++t)
        ptrs.push_back(run ? (uint64_t)grads[(size_t)(d * S + t) * P + i] + row_src : 0);
      jb.dst0 = (uint32_t)ptrs.size();
      jb.ndst = 1;
      ptrs.push_back(out0 + (uint64_t)(o * run * es));
      if (jb.nbytes) jobs.push_back(jb);
    }
  };
  // Dim-k chunks (every rank the same run, no tail) whose rows the fold
  // takes, and short rows that fit one block: the S ranks of a shard group
  // read pieces of the same gradient rows, so they are planned per group
  // below; everything else per rank here.
  std::vector<uint8_t> per_group((size_t)P, 0);
  for (int32_t i = 0; i < P; ++i) {
    const int64_t run = L.row_len[(size_t)i * S] * L.inner[i];
    const uint64_t row = (uint64_t)(run * es), rows = (uint64_t)L.outer[i];
    per_group[(size_t)i] = L.padded[i] > 0 && L.outer[i] > 1 && L.padded[i] == L.outer[i] * run &&
                           (fold_rows(row, rows, (uint64_t)S, fold_reduce_max_chunk(), 16) ||
                            long_rows(row, rows, (uint64_t)S, fold_reduce_max_chunk(), 16) ||
                            (block_ok(i, 0) && interleave_rows(row, rows)));
  }
  for (int32_t g = 0; g < R; ++g)
    for (int32_t i = 0; i < P; ++i)
      if (L.padded[i] > 0 && !per_group[(size_t)i]) emit_rank(g, i);
  // One fold-reduce item per group sums whole gradient rows and hands each
  // rank its piece; where the widths do not allow it, short rows go as the
  // ranks' jobs for the same rows next to each other, one job per chunk of
  // rows, and longer ones rank by rank
  std::vector<fsdp::FoldRed> folds;
  std::vector<uint64_t> fold_ptrs;
  for (int32_t d = 0; d < R / S; ++d) {
    for (int32_t i = 0; i < P; ++i) {
      if (!per_group[(size_t)i]) continue;
      const uint64_t rows = (uint64_t)L.outer[i];
      const uint64_t row = (uint64_t)(L.row_len[(size_t)i * S] * L.inner[i] * es);
      std::vector<uint64_t> src, dst;
      for (int32_t t = 0; t < S; ++t) {
        src.push_back((uint64_t)grads[(size_t)(d * S + t) * P + i]);
        dst.push_back((uint64_t)rs_out[d * S + t] + (uint64_t)(L.in_off[i] * es));
      }
      if (push_fold_reduce(folds, fold_ptrs, src, dst, row, rows, es)) continue;
      if (block_ok(i, 0) && interleave_rows(row, rows)) {
        const uint64_t per = CH / row;
        for (uint64_t r0 = 0; r0 < rows; r0 += per)
          for (int32_t s = 0; s < S; ++s) push_block(d * S + s, i, r0, std::min(per, rows - r0));
        continue;
      }
      for (int32_t s = 0; s < S; ++s) emit_rank(d * S + s, i);
    }
  }
  if (jobs.size() > 0xffffffffu || ptrs.size() > 0xffffffffu) return fail(FSDP_EINVAL, "too many jobs");
  out->jobs = std::move(jobs);
  out->ptrs = std::move(ptrs);
  out->folds = std::move(folds);
  out->fold_ptrs = std::move(fold_ptrs);
  return FSDP_OK;
}

int rs_copy_reduce_impl(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dp_size,
                        int32_t op, int32_t dtype, const void* const* grads, void* const* rs_out,
                        void* stream) {
  Key key(kRsCopyReduce);
  if (key.bucket(bucket)) {
    for (int64_t v : {(int64_t)rank_size, (int64_t)shard_size, (int64_t)dp_size, (int64_t)op, (int64_t)dtype})
      key.add(v);
    key.ptrs(grads, (int64_t)rank_size * bucket->n_params);
    key.ptrs(rs_out, rank_size);
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  CopyReducePlan cp;
  if ((rc = plan_rs_copy_reduce(bucket, rank_size, shard_size, dp_size, op, dtype, grads, rs_out, &cp))) return rc;
  return run_reduce(std::move(key), cp.jobs, cp.ptrs, dtype, op == FSDP_AVG, Reuse::kReadNext,
                    static_cast<hipStream_t>(stream), cp.folds, cp.fold_ptrs);
}

// The same call with its descriptor tables written into the current GPU's
// scratch array instead of cached device allocations: planned on every call
// (nothing is cached), the tables carried to the GPU in the kernel
// arguments of small writer launches on the call's stream, then the same
// kernels launched on the same stream.  No device or pinned memory is
// allocated, so the call can run under graph capture.
int rs_copy_reduce_noalloc_impl(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                                int32_t dp_size, int32_t op, int32_t dtype, const void* const* grads,
                                void* const* rs_out, void* stream) {
  CopyReducePlan cp;
  int rc = plan_rs_copy_reduce(bucket, rank_size, shard_size, dp_size, op, dtype, grads, rs_out, &cp);
  if (rc) return rc;
  uint64_t job_out = 0;
  for (const auto& jb : cp.jobs) job_out += jb.nbytes * jb.ndst * jb.rows;
  Plan p;
  std::vector<uint8_t> job_table, fold_table;
  rc = plan_reduce(cp.jobs, cp.ptrs, dtype, op == FSDP_AVG, Reuse::kReadNext, fold_reduce_out_bytes(cp.folds), &p,
                   &job_table);
  if (!rc) rc = plan_fold_reduce(cp.folds, cp.fold_ptrs, dtype, op == FSDP_AVG, Reuse::kReadNext, job_out, &p,
                                 &fold_table);
  if (rc) return rc;
  if (job_table.empty() && fold_table.empty()) return ok();
  const size_t fold_at = (job_table.size() + 255) / 256 * 256;
  const size_t need = fold_at + fold_table.size();
  if (need > fsdp::kScratchBytes)
    return fail(FSDP_EINVAL, "fsdp_rs_copy_reduce_noalloc: the call's descriptor tables need %zu bytes, more than "
                "the %zu-byte scratch array holds (use fsdp_rs_copy_reduce, or split the bucket)",
                need, fsdp::kScratchBytes);
  void* base = nullptr;
  int he = fsdp_scratch_ptr(&base);
  if (he != hipSuccess) return fail(FSDP_EHIP, "scratch array address: %s", hipGetErrorString((hipError_t)he));
  if (!job_table.empty() &&
      (he = fsdp_scratch_write(base, job_table.data(), job_table.size(), 0, stream)) != hipSuccess)
    return fail(FSDP_EHIP, "descriptor table write: %s", hipGetErrorString((hipError_t)he));
  if (!fold_table.empty() &&
      (he = fsdp_scratch_write(base, fold_table.data(), fold_table.size(), fold_at, stream)) != hipSuccess)
    return fail(FSDP_EHIP, "descriptor table write: %s", hipGetErrorString((hipError_t)he));
  if (!job_table.empty()) {
    p.dev = base;
    p.bytes = job_table.size();
  }
  if (!fold_table.empty()) {
    p.fold_dev = static_cast<uint8_t*>(base) + fold_at;
    p.fold_bytes = fold_table.size();
  }
  // the plan's tables belong to the scratch array: never freed
  return enqueue(p, static_cast<hipStream_t>(stream));
}

int fused_ar_impl(int32_t n_seg, const int64_t* seg_numel, int32_t rank_size, int32_t shard_size,
                  int32_t dp_size, int32_t op, int32_t dtype, void* const* fused, void* stream) {
  Key key(kFusedAr);
  if (n_seg >= 0 && (n_seg == 0 || seg_numel)) {
    for (int64_t v : {(int64_t)n_seg, (int64_t)rank_size, (int64_t)shard_size, (int64_t)dp_size, (int64_t)op,
                      (int64_t)dtype})
      key.add(v);
    for (int32_t j = 0; j < n_seg; ++j) key.add(seg_numel[j]);
    key.ptrs(fused, rank_size);
  } else {
    key.ptrs(nullptr, 1);  // unreadable: validation reports it
  }
  int rc = FSDP_OK;
  if (launch_cached(key, static_cast<hipStream_t>(stream), &rc)) return rc;
  if ((rc = check_groups(rank_size, shard_size))) return rc;
  if (dp_size != rank_size / shard_size)
    return fail(FSDP_EINVAL, "dp_size %d != rank_size / shard_size = %d", dp_size, rank_size / shard_size);
  if (op != FSDP_SUM && op != FSDP_AVG) return fail(FSDP_EINVAL, "reduce op %d", op);
  const int es = reduce_elem_size(dtype);
  if (!es) return fail(FSDP_ENOTIMPL, "fused_ar takes fp32, bf16 or fp16 (dtype %d)", dtype);
  int64_t F = 0;
  if ((rc = fused_layout_impl(n_seg, seg_numel, es, nullptr, &F))) return rc;
  const int32_t R = rank_size, S = shard_size, D = dp_size;
  const int64_t nbytes = F * es;
  if (!fused) return fail(FSDP_EINVAL, "fused array is NULL");
  std::vector<Span> outs;
  for (int32_t g = 0; g < R; ++g) {
    if ((rc = check_ptr(fused[g], nbytes, FSDP_FUSED_ALIGN_BYTES, "fused", g))) return rc;
    outs.push_back({(uint64_t)fused[g], (uint64_t)fused[g] + (uint64_t)nbytes, g});
  }
  if ((rc = check_overlap(outs, {}))) return rc;
  if (nbytes == 0 || D == 1) return ok();  // a group of one: the identity
  std::vector<fsdp::RedJob> jobs;
  std::vector<uint64_t> ptrs;
  for (int32_t s = 0; s < S; ++s) {
    fsdp::RedJob jb;
    jb.nbytes = jb.data_bytes = (uint64_t)nbytes;
    jb.src0 = (uint32_t)ptrs.size();
    jb.nsrc = (uint32_t)D;
    for (int32_t d = 0; d < D; ++d) ptrs.push_back((uint64_t)fused[d * S + s]);
    jb.dst0 = jb.src0;  // in place: every replica receives the result
    jb.ndst = (uint32_t)D;
    jobs.push_back(jb);
  }
  return run_reduce(std::move(key), jobs, ptrs, dtype, op == FSDP_AVG, Reuse::kFinal,
                    static_cast<hipStream_t>(stream));
}

// No C++ exception may cross the C ABI: host allocation failures while
// planning become FSDP_ENOMEM, anything else FSDP_EINVAL.  Nothing has been
// enqueued when an exception is thrown (launches come last).
template <class F>
int guarded(F&& f) noexcept {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(FSDP_ENOMEM, "out of host memory while planning the call");
  } catch (const std::length_error&) {
    return fail(FSDP_ENOMEM, "the call's host tables would exceed the largest allocation");
  } catch (const std::exception& e) {
    return fail(FSDP_EINVAL, "internal error: %s", e.what());
  } catch (...) {
    return fail(FSDP_EINVAL, "internal error");
  }
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

const char* fsdp_last_error(void) { return g_err.c_str(); }

int fsdp_time_next_launch(void* start_event, void* stop_event) {
  if (!start_event != !stop_event)
    return fail(FSDP_EINVAL, "fsdp_time_next_launch: give both events or neither");
  g_time_start = start_event;
  g_time_stop = stop_event;
  return ok();
}

void fsdp_release_cache(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  try {
    if (!g_lru.empty()) (void)sync_cached_devices();
  } catch (...) {  // no memory to list the devices: wait for every one
    int n = 0, cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && hipGetDeviceCount(&n) == hipSuccess) {
      for (int d = 0; d < n; ++d)
        if (hipSetDevice(d) == hipSuccess) (void)hipDeviceSynchronize();
      (void)hipSetDevice(cur);
    }
  }
  while (!g_lru.empty()) drop_entry(g_lru.begin());
}

int fsdp_cache_info(int64_t* n_plans, int64_t* n_pinned, int64_t* table_bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  int64_t pinned = 0;
  for (const Entry& en : g_lru) pinned += en.pinned ? 1 : 0;
  if (n_plans) *n_plans = (int64_t)g_lru.size();
  if (n_pinned) *n_pinned = pinned;
  if (table_bytes) *table_bytes = (int64_t)g_table_bytes;
  return ok();
}

int fsdp_bucket_layout(const fsdp_bucket_t* bucket, int32_t shard_size, int64_t* slice_numel,
                       int64_t* padded, int64_t* in_off, int64_t* row_off, int64_t* row_len) {
  return guarded([&] { return bucket_layout_impl(bucket, shard_size, slice_numel, padded, in_off, row_off, row_len); });
}

int fsdp_fused_layout(int32_t n_seg, const int64_t* seg_numel, int32_t elem_bytes, int64_t* seg_off,
                      int64_t* fused_numel) {
  return guarded([&] { return fused_layout_impl(n_seg, seg_numel, elem_bytes, seg_off, fused_numel); });
}

int fsdp_group_ranks(int32_t rank_size, int32_t shard_size, int32_t* n_rs_groups, int32_t* rs_ranks,
                     int32_t* n_ar_groups, int32_t* ar_ranks) {
  return guarded([&] { return group_ranks_impl(rank_size, shard_size, n_rs_groups, rs_ranks, n_ar_groups, ar_ranks); });
}

int fsdp_ag_copy_in(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype,
                    const void* const* shards, void* ag, void* stream) {
  return guarded([&] { return ag_copy_in_impl(bucket, shard_size, dtype, shards, ag, stream); });
}

int fsdp_ag_copy_out(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype, const void* ag,
                     void* const* full, void* stream) {
  return guarded([&] { return ag_copy_out_impl(bucket, shard_size, dtype, ag, full, stream); });
}

int fsdp_rs_copy_in(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dtype,
                    const void* const* grads, void* const* rs_in, void* stream) {
  return guarded([&] { return rs_copy_in_impl(bucket, rank_size, shard_size, dtype, grads, rs_in, stream); });
}

int fsdp_rs_reduce(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dp_size,
                   int32_t op, int32_t dtype, const void* const* rs_in, void* const* rs_out, void* stream) {
  return guarded([&] { return rs_reduce_impl(bucket, rank_size, shard_size, dp_size, op, dtype, rs_in, rs_out, stream); });
}

int fsdp_rs_copy_reduce(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size, int32_t dp_size,
                        int32_t op, int32_t dtype, const void* const* grads, void* const* rs_out,
                        void* stream) {
  return guarded([&] { return rs_copy_reduce_impl(bucket, rank_size, shard_size, dp_size, op, dtype, grads, rs_out, stream); });
}

int fsdp_rs_copy_reduce_noalloc(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                                int32_t dp_size, int32_t op, int32_t dtype, const void* const* grads,
                                void* const* rs_out, void* stream) {
  return guarded([&] {
    return rs_copy_reduce_noalloc_impl(bucket, rank_size, shard_size, dp_size, op, dtype, grads, rs_out, stream);
  });
}

int fsdp_fused_ar(int32_t n_seg, const int64_t* seg_numel, int32_t rank_size, int32_t shard_size,
                  int32_t dp_size, int32_t op, int32_t dtype, void* const* fused, void* stream) {
  return guarded([&] { return fused_ar_impl(n_seg, seg_numel, rank_size, shard_size, dp_size, op, dtype, fused, stream); });
}

}  // extern "C"
