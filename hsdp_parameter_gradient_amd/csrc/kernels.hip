// gfx950 kernels of the FSDP/HSDP flat-buffer hot path.
//
// Four kernels serve the six device entry points:
//   seg_copy  — segmented copy with zero fill: AG copy-in (pack shards into
//               padded rank slices), AG copy-out (unpack into the full
//               parameters) and RS copy-in (chunk gradients into the padded
//               rank-major RS input).  Bits are moved, never converted.
//   fold_copy — AG copy-out and RS copy-in of parameters sharded on a
//               non-zero dim whose chunk rows are short: all shard ranks'
//               pieces of whole full-tensor rows per workgroup, so both
//               sides move whole cache lines (2- and 4-byte pieces staged
//               through LDS).
//   reduce    — fixed-order reduction, in fp32, of K operands into M
//               destinations, with a zero-filled tail per job: the RS of a
//               shard group (K = S, M = 1), the RS read straight from the
//               full gradients (one job per rank and parameter, its
//               padding zero filled), and the in-place fused AR of a
//               replicate group (K = M = D).  fp32, bf16 or fp16 elements
//               (16-bit elements widened exactly, summed in fp32, rounded
//               once to nearest even).
//   fold_reduce — the RS read straight from the full gradients for the
//               short-row parameters of fold_copy: one shard group's
//               gradients summed over whole full-tensor rows (the reduce
//               arithmetic), each rank's piece written to its output.
//
// All four are HBM-bound streaming kernels (no data reuse, no dense
// contraction): one workgroup (512 lanes for the copy, two 16-byte vectors
// each per 16 KiB chunk; 256 lanes for the others) handles one chunk of
// destination bytes at a time, with 128-bit loads and stores on 16-byte-aligned
// destination addresses.  A source whose address differs from the
// destination's modulo 16 is read as the two aligned 16-byte blocks around
// each destination vector and realigned in registers with v_alignbyte
// (each block read holds at least one byte the copy needs, so no read
// leaves the source's own pages).  The few 16-byte vectors that straddle a
// segment edge or the data/padding edge are written element by element, so
// that no byte outside the segment is touched.  Every loop over a chunk's
// vectors runs whole unguarded iterations (all loads of an iteration in
// flight before the first use) and then a short guarded tail.
//
// The chunk of a parameter sharded on a non-zero dim is a strided block
// (`outer` rows, one per index of the dims before the shard dim).  When both
// pitches are multiples of 16 bytes (every row then has the alignment of the
// first) the planner hands it over as one item; each chunk of it is a group
// of whole rows: their whole aligned destination vectors form one flat range
// (row and column from one integer division), and each row's head and tail
// bytes are moved element by element.
//
// Arithmetic: the reduce kernel adds operands one at a time in ascending
// rank order, the accumulator starting from the first operand, in IEEE
// fp32 with denormals preserved; AVG divides the sum by the operand count
// with a correctly rounded division (for a power of two that is the exact
// multiply by its reciprocal); bf16 and fp16 results are rounded once, at
// the store.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <mutex>
#include <type_traits>

#include "plan.hpp"

// Sources are read exactly once: nontemporal loads keep them from
// displacing the outputs in L2 and MALL (measured faster on MI355X for every
// op).  Stores are nontemporal only when the planner asks (NTS): for the
// path's final outputs and for outputs too large to be re-read from the
// MALL; an output the next step reads back stays cacheable.
#ifndef FSDP_NT_LOADS
#define FSDP_NT_LOADS 1
#endif
// The copy kernel's workgroup shape: FSDP_COPY_BLOCK lanes, each with
// FSDP_COPY_UNROLL 16-byte vectors in flight per iteration, so a 16 KiB chunk
// is one iteration.  Fewer bytes in flight per wave keep the HBM better fed:
// measured on MI355X, 512 lanes x 2 vectors move the 51.8 GB RS copy-in of
// four Llama-7B-shaped layers at 6.4 TB/s and a plain 4 GiB copy at 6.5 TB/s,
// against 6.0-6.1 TB/s for both with 256 lanes x 4 vectors; 1024 lanes x 1
// vector is no faster on the large copies and slower on buckets of a few
// thousand chunks (fewer, larger workgroups fill the chip unevenly).
#ifndef FSDP_COPY_UNROLL
#define FSDP_COPY_UNROLL 2
#endif
#ifndef FSDP_COPY_BLOCK
#define FSDP_COPY_BLOCK 512
#endif

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Data pointers are rebuilt from the byte addresses in the descriptor
// tables; marking them global lets the compiler emit global_* (not flat_*)
// memory instructions.
#define GMEM __attribute__((address_space(1)))
typedef GMEM u32x4 gvec;
template <typename T>
__device__ __forceinline__ GMEM T* gptr(uint64_t a) {
  return reinterpret_cast<GMEM T*>(a);
}

constexpr int kBlock = 256;  // every kernel but the copy
constexpr int kCopyBlock = FSDP_COPY_BLOCK;
constexpr int kCopyUnroll = FSDP_COPY_UNROLL;
static_assert(kCopyBlock % 64 == 0 && kCopyBlock <= 1024, "the copy block is whole waves");

// XCD-aware chunk order.  Workgroups are dispatched to the 8 XCDs
// round-robin in blockIdx order (and every grid-stride step is a multiple
// of 8 workgroups), so workgroup-slot c runs on XCD c % 8.  Within every
// group of 8*kXcdRun consecutive chunks, XCD x takes the kXcdRun
// consecutive chunks [x*kXcdRun, (x+1)*kXcdRun): each XCD streams runs of
// contiguous memory (1 MiB for the copy, 512 KiB for the reduce, at the
// default chunk sizes) while all XCDs stay near the same front.  A
// bijection on [0, n): the last partial group keeps the plain order.
// Measured on MI355X against the plain order: the HSDP block step -1.8 %,
// a 4-layer Llama-7B bucket -3.6 %, the ragged fp32 set -3.9 % (runs of 16
// to 128 chunks are all better than the plain order; runs of 256 and one
// contiguous eighth per XCD are worse on the small bucket).
constexpr uint64_t kXcdRun = 64;
#ifndef FSDP_COPY_XCD_RUN
#define FSDP_COPY_XCD_RUN 64
#endif
constexpr uint64_t kCopyXcdRun = FSDP_COPY_XCD_RUN;

template <uint64_t RUN = kXcdRun>
__device__ __forceinline__ uint64_t xcd_chunk(uint64_t c, uint64_t n) {
  constexpr uint64_t G = 8 * RUN;
  if (c >= n / G * G) return c;
  const uint64_t rem = c % G;
  return c - rem + (rem & 7) * RUN + (rem >> 3);
}

__device__ __forceinline__ uint64_t align_down16(uint64_t a) { return a & ~uint64_t(15); }
__device__ __forceinline__ uint64_t align_up16(uint64_t a) { return (a + 15) & ~uint64_t(15); }

__device__ __forceinline__ u32x4 ldv(const gvec* p) {
  if (FSDP_NT_LOADS) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NTS>
__device__ __forceinline__ void stv(gvec* p, u32x4 v) {
  if (NTS)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// Largest j with begin[j] <= c, for begin[0] == 0 <= c and begin strictly
// increasing.  64-ary search: every lane of the wave probes one entry, so a
// table of up to 4096 items takes two dependent loads.
__device__ __forceinline__ uint32_t find_item(const uint64_t* __restrict__ begin, uint32_t n,
                                              uint64_t c) {
  const uint32_t lane = threadIdx.x & 63u;
  uint32_t lo = 0, cnt = n;
  while (cnt > 1) {
    const uint32_t step = (cnt + 63u) >> 6;
    const uint32_t off = lane * step;
    const bool le = off < cnt && begin[lo + off] <= c;
    const uint64_t m = __ballot(le);
    const uint32_t k = (uint32_t)__popcll(m) - 1u;  // lane 0 always holds
    lo += k * step;
    const uint32_t rest = cnt - k * step;
    cnt = rest < step ? rest : step;
  }
  return lo;
}

// Bytes [4*Q + b, 4*Q + b + 16) of the 32-byte concatenation a || c.
template <int Q>
__device__ __forceinline__ u32x4 funnel(u32x4 a, u32x4 c, uint32_t b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  u32x4 o;
  o.x = __builtin_amdgcn_alignbyte(w[Q + 1], w[Q + 0], b);
  o.y = __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], b);
  o.z = __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], b);
  o.w = __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], b);
  return o;
}

// Lane l of a full wave receives v from lane l + 1 (lane 63 receives lane
// 0's value, which the callers replace); ds_bpermute moves data through the
// LDS crossbar without touching LDS memory.
__device__ __forceinline__ u32x4 from_next_lane(u32x4 v, uint32_t lane) {
  const int addr = (int)(((lane + 1u) & 63u) << 2);
  u32x4 o;
  o.x = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.x);
  o.y = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.y);
  o.z = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.z);
  o.w = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v.w);
  return o;
}

// Lane 0's value of v, in every lane (the wave must be full).
__device__ __forceinline__ u32x4 lane0(u32x4 v) {
  u32x4 o;
  o.x = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.x);
  o.y = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.y);
  o.z = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.z);
  o.w = (uint32_t)__builtin_amdgcn_readfirstlane((int)v.w);
  return o;
}

// Shifted view of U consecutive 64-block groups held one block per lane:
// a[u] is block wb + 64u + lane, tail is block wb + 64U (wave-uniform).
// Returns, in a[u], the 16 bytes starting r = 4*Q + b bytes into a[u]; each
// source block is loaded once.
template <int Q, int U>
__device__ __forceinline__ void realign_groups(u32x4 (&a)[U], u32x4 tail, uint32_t lane, uint32_t b) {
  u32x4 nxt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const u32x4 first_of_next = (u + 1 < U) ? lane0(a[u + 1 < U ? u + 1 : u]) : tail;
    const u32x4 up = from_next_lane(a[u], lane);
    nxt[u] = lane == 63u ? first_of_next : up;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = funnel<Q>(a[u], nxt[u], b);
}

// 16 source bytes starting r bytes into aligned block s[j] (0 <= r < 16).
__device__ __forceinline__ u32x4 load_shifted(const gvec* __restrict__ s, uint64_t j, uint32_t r) {
  if (r == 0) return ldv(s + j);
  const u32x4 a = ldv(s + j);
  const u32x4 c = ldv(s + j + 1);
  const uint32_t b = r & 3u;
  switch (r >> 2) {
    case 0: return funnel<0>(a, c, b);
    case 1: return funnel<1>(a, c, b);
    case 2: return funnel<2>(a, c, b);
    default: return funnel<3>(a, c, b);
  }
}

// ---------------------------------------------------------------------------
// seg_copy
// ---------------------------------------------------------------------------

// nv destination vectors d[0..nv) from source blocks s[0..nv] realigned by
// r = 4*Q + b bytes (Q = -1: aligned, s[0..nv) read directly).
template <int Q, bool NTS>
__device__ __forceinline__ void copy_run(gvec* __restrict__ d, const gvec* __restrict__ s, uint64_t nv,
                                         uint32_t b) {
  constexpr int U = kCopyUnroll;
  constexpr int QQ = Q >= 0 ? Q : 0;
  const uint32_t lane = threadIdx.x & 63u;
  uint64_t base = 0;
  for (; base + (uint64_t)kCopyBlock * U <= nv; base += (uint64_t)kCopyBlock * U) {
    u32x4 a[U];
    if (Q < 0) {
      const uint64_t j = base + threadIdx.x;
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = ldv(s + j + u * kCopyBlock);
#pragma unroll
      for (int u = 0; u < U; ++u) stv<NTS>(d + j + u * kCopyBlock, a[u]);
    } else {
      // each wave owns 64*U consecutive vectors; one extra uniform block
      // (the first of the next wave's range, at most block nv) closes it
      const uint64_t wb = base + (uint64_t)(threadIdx.x >> 6) * 64u * U;
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = ldv(s + wb + u * 64 + lane);
      const u32x4 tail = s[wb + 64 * U];
      realign_groups<QQ, U>(a, tail, lane, b);
#pragma unroll
      for (int u = 0; u < U; ++u) stv<NTS>(d + wb + u * 64 + lane, a[u]);
    }
  }
  for (uint64_t j = base + threadIdx.x; j < nv; j += kCopyBlock) {
    const u32x4 a = ldv(s + j);
    if (Q >= 0) {
      const u32x4 c = ldv(s + j + 1);
      stv<NTS>(d + j, funnel<QQ>(a, c, b));
    } else {
      stv<NTS>(d + j, a);
    }
  }
}

// nv destination vectors from dst (16-aligned), source bytes from src.
template <bool NTS>
__device__ __forceinline__ void copy_vectors(uint64_t dst, uint64_t src, uint64_t nv) {
  gvec* __restrict__ d = gptr<u32x4>(dst);
  const uint32_t r = (uint32_t)(src & 15u);
  const gvec* __restrict__ s = gptr<u32x4>(src - r);
  const uint32_t b = r & 3u;
  if (r == 0) {
    copy_run<-1, NTS>(d, s, nv, 0);
    return;
  }
  switch (r >> 2) {
    case 0: copy_run<0, NTS>(d, s, nv, b); break;
    case 1: copy_run<1, NTS>(d, s, nv, b); break;
    case 2: copy_run<2, NTS>(d, s, nv, b); break;
    default: copy_run<3, NTS>(d, s, nv, b); break;
  }
}

// nv zero vectors from dst, by a workgroup of BLK lanes.
template <int BLK, bool NTS>
__device__ __forceinline__ void zero_vectors(uint64_t dst, uint64_t nv) {
  gvec* __restrict__ d = gptr<u32x4>(dst);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (uint64_t j = threadIdx.x; j < nv; j += BLK) stv<NTS>(d + j, z);
}

template <typename T>
__device__ __forceinline__ void copy_partial(uint64_t a, uint64_t lo, uint64_t hi,
                                             const fsdp::CopySeg& sg) {
  const uint64_t cend = sg.dst + sg.copy_bytes;
  const uint64_t x0 = a > lo ? a : lo;
  const uint64_t x1 = (a + 16) < hi ? (a + 16) : hi;
  for (uint64_t x = x0; x < x1; x += sizeof(T)) {
    T v = 0;
    if (x < cend) v = *gptr<T>(sg.src + (x - sg.dst));
    *gptr<T>(x) = v;
  }
}

// Vector q of a strided block of whole-vector rows, vpr vectors per row:
// its byte offsets from the block's first source and destination rows.
struct RowVec {
  uint64_t src, dst;
};
__device__ __forceinline__ RowVec row_vec(uint32_t q, uint32_t vpr, uint64_t src_pitch, uint64_t dst_pitch) {
  const uint32_t row = q / vpr;
  const uint64_t col = (uint64_t)(q - row * vpr) << 4;
  return {row * src_pitch + col, row * dst_pitch + col};
}

// The whole destination vectors of nr rows: vpr per row, row r's first at
// d0 + r*dst_pitch (16-byte aligned), its source bytes at s0 + r*src_pitch
// (Q < 0: 16-byte aligned; else shifted by 4*Q + b bytes past an aligned
// block, read as two aligned blocks and realigned; plain loads, so the
// second block of a pair is an L1/L2 hit).  U vectors per lane per
// iteration, all loads before the first store.
template <int Q, bool NTS>
__device__ __forceinline__ void rows_run(uint64_t s0, uint64_t d0, uint32_t nr, uint32_t vpr, uint64_t src_pitch,
                                         uint64_t dst_pitch, uint32_t b) {
  // a shifted vector takes two loads: half as many per lane
  constexpr int U = Q < 0 ? kCopyUnroll : (kCopyUnroll > 1 ? kCopyUnroll / 2 : 1);
  constexpr int QQ = Q >= 0 ? Q : 0;
  const uint32_t nv = nr * vpr;
  uint32_t base = 0;
  for (; base + (uint32_t)kCopyBlock * U <= nv; base += (uint32_t)kCopyBlock * U) {
    u32x4 a[U];
    uint64_t dof[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const RowVec x = row_vec(base + threadIdx.x + u * kCopyBlock, vpr, src_pitch, dst_pitch);
      const gvec* sp = gptr<u32x4>(s0 + x.src);
      a[u] = Q < 0 ? ldv(sp) : funnel<QQ>(sp[0], sp[1], b);
      dof[u] = x.dst;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) stv<NTS>(gptr<u32x4>(d0 + dof[u]), a[u]);
  }
  for (uint32_t q = base + threadIdx.x; q < nv; q += kCopyBlock) {
    const RowVec x = row_vec(q, vpr, src_pitch, dst_pitch);
    const gvec* sp = gptr<u32x4>(s0 + x.src);
    stv<NTS>(gptr<u32x4>(d0 + x.dst), Q < 0 ? ldv(sp) : funnel<QQ>(sp[0], sp[1], b));
  }
}

// Width in bytes of the units a block of rows can move whole: 8 or 4 when
// both first-row addresses, both pitches and the row length are multiples of
// it (then every unit of every row is aligned), else the element size.
template <typename T>
__device__ __forceinline__ uint32_t unit_bytes(uint64_t s0, uint64_t d0, uint64_t sp, uint64_t dp, uint64_t row) {
  const uint64_t m = s0 | d0 | sp | dp | row;
  return (m & 7u) == 0 ? 8u : (m & 3u) == 0 ? 4u : (uint32_t)sizeof(T);
}

// The nr rows of a strided block as one flat range of W-typed units, upr
// per row: unit q is row q / upr, column q % upr.  For pitches that are not
// multiples of 16 (each row starts at another offset mod 16).  The planner
// keeps a chunk's rows within 4 GiB of its first row on both sides, so
// offsets are 32-bit (the workgroup-uniform base plus a 32-bit offset per
// lane keeps the register count of the whole kernel down).  U units per
// lane per iteration (as many as a 16 KiB chunk needs, at most 4), all loads
// before the first store; the remainder is one predicated iteration.
template <typename W, bool NTS>
__device__ __forceinline__ void rows_units(uint64_t s0, uint64_t d0, uint32_t nr, uint32_t upr, uint32_t sp,
                                           uint32_t dp) {
  constexpr int UC = 16384 / (kCopyBlock * (int)sizeof(W));
  constexpr int U = UC < 1 ? 1 : UC > 4 ? 4 : UC;
  const uint32_t n = nr * upr;
  const GMEM uint8_t* __restrict__ sb = gptr<uint8_t>(s0);
  GMEM uint8_t* __restrict__ db = gptr<uint8_t>(d0);
  auto off = [&](uint32_t q, uint32_t pitch) -> uint32_t {
    const uint32_t row = q / upr;
    return row * pitch + (q - row * upr) * (uint32_t)sizeof(W);
  };
  auto ld = [&](uint32_t o) { return __builtin_nontemporal_load(reinterpret_cast<const GMEM W*>(sb + o)); };
  auto st = [&](uint32_t o, W v) {
    GMEM W* a = reinterpret_cast<GMEM W*>(db + o);
    if (NTS)
      __builtin_nontemporal_store(v, a);
    else
      *a = v;
  };
  uint32_t base = 0;
  for (; base + (uint32_t)kCopyBlock * U <= n; base += (uint32_t)kCopyBlock * U) {
    W v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld(off(base + threadIdx.x + u * kCopyBlock, sp));
#pragma unroll
    for (int u = 0; u < U; ++u) st(off(base + threadIdx.x + u * kCopyBlock, dp), v[u]);
  }
  if (base < n) {
    W v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t q = base + threadIdx.x + u * kCopyBlock;
      if (q < n) v[u] = ld(off(q, sp));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t q = base + threadIdx.x + u * kCopyBlock;
      if (q < n) st(off(q, dp), v[u]);
    }
  }
}

// Chunk k of a strided block (CopySeg with rows > 1): rows
// [k*rows_per_chunk, ...).  When both pitches are multiples of 16, every row
// has the same alignment: a head of up to 15 bytes before the row's first
// aligned destination vector, whole vectors, and a tail after the last one.
// The whole vectors of all rows are one flat range (rows_run); heads and
// tails are copied element by element, one row end per lane.  Other pitches
// move the rows in 8-, 4- or element-sized units (rows_units).
template <typename T, bool NTS>
__device__ __forceinline__ void copy_rows(const fsdp::CopySeg& sg, uint64_t k) {
  const uint64_t r0 = k * sg.rows_per_chunk;
  const uint64_t left = sg.rows - r0;
  const uint32_t nr = (uint32_t)(left < sg.rows_per_chunk ? left : sg.rows_per_chunk);
  const uint64_t B = sg.copy_bytes;
  const uint64_t s0 = sg.src + r0 * sg.src_pitch;
  const uint64_t d0 = sg.dst + r0 * sg.dst_pitch;
  if ((sg.src_pitch | sg.dst_pitch) & 15u) {
    const uint32_t w = unit_bytes<T>(s0, d0, sg.src_pitch, sg.dst_pitch, B);
    const uint32_t sp = (uint32_t)sg.src_pitch, dp = (uint32_t)sg.dst_pitch;
    if (w == 8)
      rows_units<uint64_t, NTS>(s0, d0, nr, (uint32_t)(B >> 3), sp, dp);
    else if (w == 4)
      rows_units<uint32_t, NTS>(s0, d0, nr, (uint32_t)(B >> 2), sp, dp);
    else
      rows_units<T, NTS>(s0, d0, nr, (uint32_t)(B / sizeof(T)), sp, dp);
    return;
  }
  uint64_t head = (16u - (uint32_t)(d0 & 15u)) & 15u;
  if (head > B) head = B;
  const uint32_t vpr = (uint32_t)((B - head) >> 4);
  const uint64_t tail = head + ((uint64_t)vpr << 4);
  if (vpr) {
    const uint64_t sv = s0 + head;
    const uint32_t r = (uint32_t)(sv & 15u);
    const uint32_t b = r & 3u;
    const uint64_t sa = sv - r, da = d0 + head;
    if (r == 0) {
      rows_run<-1, NTS>(sa, da, nr, vpr, sg.src_pitch, sg.dst_pitch, 0);
    } else {
      switch (r >> 2) {
        case 0: rows_run<0, NTS>(sa, da, nr, vpr, sg.src_pitch, sg.dst_pitch, b); break;
        case 1: rows_run<1, NTS>(sa, da, nr, vpr, sg.src_pitch, sg.dst_pitch, b); break;
        case 2: rows_run<2, NTS>(sa, da, nr, vpr, sg.src_pitch, sg.dst_pitch, b); break;
        default: rows_run<3, NTS>(sa, da, nr, vpr, sg.src_pitch, sg.dst_pitch, b); break;
      }
    }
  }
  if (head || tail < B) {
    for (uint32_t t = threadIdx.x; t < 2 * nr; t += kCopyBlock) {
      const uint32_t row = t >> 1;
      const uint64_t lo = (t & 1) ? tail : 0, hi = (t & 1) ? B : head;
      const uint64_t sr = s0 + row * sg.src_pitch, dr = d0 + row * sg.dst_pitch;
      for (uint64_t x = lo; x < hi; x += sizeof(T)) *gptr<T>(dr + x) = *gptr<T>(sr + x);
    }
  }
}

// Chunk k of item sg.
template <typename T, bool NTS>
__device__ __forceinline__ void copy_chunk(const fsdp::CopySeg& sg, uint64_t k, uint32_t shift) {
  if (sg.rows > 1) {
    copy_rows<T, NTS>(sg, k);
    return;
  }
  const uint64_t CH = uint64_t(1) << shift;
  const uint64_t base = (sg.dst >> shift) << shift;
  const uint64_t seg_end = sg.dst + sg.total_bytes;
  const uint64_t cend = sg.dst + sg.copy_bytes;
  const uint64_t w0 = base + k * CH;
  const uint64_t lo = w0 > sg.dst ? w0 : sg.dst;
  const uint64_t hi = (w0 + CH) < seg_end ? (w0 + CH) : seg_end;

  // whole vectors of data
  const uint64_t ca = align_up16(lo);
  const uint64_t cb = align_down16(hi < cend ? hi : cend);
  if (ca < cb) copy_vectors<NTS>(ca, sg.src + (ca - sg.dst), (cb - ca) >> 4);
  // whole vectors of padding
  const uint64_t za = align_up16(lo > cend ? lo : cend);
  const uint64_t zb = align_down16(hi);
  if (za < zb) zero_vectors<kCopyBlock, NTS>(za, (zb - za) >> 4);
  // vectors cut by the window start, the data/padding edge, the segment end
  if (threadIdx.x < 3) {
    const uint64_t a_lo = align_down16(lo);
    const uint64_t a_c = align_down16(cend);
    const uint64_t a_hi = align_down16(hi);
    const bool p_lo = (lo & 15) != 0;
    const bool p_c = (cend & 15) != 0 && lo < cend && cend < hi && !(p_lo && a_c == a_lo);
    const bool p_hi = (hi & 15) != 0 && !(p_lo && a_hi == a_lo) && !(p_c && a_hi == a_c);
    if (threadIdx.x == 0 && p_lo) copy_partial<T>(a_lo, lo, hi, sg);
    if (threadIdx.x == 1 && p_c) copy_partial<T>(a_c, lo, hi, sg);
    if (threadIdx.x == 2 && p_hi) copy_partial<T>(a_hi, lo, hi, sg);
  }
}

// item_of[c] is the item that chunk c belongs to (the planner's table), so
// a workgroup finds its item with one scalar load; a search of the chunk
// prefix (64 lanes probing 64 cache lines) cost the one-vector-per-lane
// copy a fifth of its rate.  The grid is the chunk count, or a multiple of 8
// below it (n_chunks < 2^31); the loop tests for the exit right after the
// stores, so no wave waits for its stores to land before it ends.
template <typename T, bool NTS>
__global__ __launch_bounds__(kCopyBlock) void seg_copy_kernel(const uint64_t* __restrict__ begin,
                                                              const fsdp::CopySeg* __restrict__ segs,
                                                              const uint32_t* __restrict__ item_of,
                                                              uint32_t n_chunks, uint32_t shift, uint32_t grid) {
  // grid (the launch's workgroup count) comes in with the other kernel
  // arguments, so the exit test needs no load after the stores
  for (uint32_t slot = blockIdx.x;;) {
    const uint32_t c = (uint32_t)xcd_chunk<kCopyXcdRun>(slot, n_chunks);
    const uint32_t j = item_of[c];
    copy_chunk<T, NTS>(segs[j], c - begin[j], shift);
    slot += grid;
    if (slot >= n_chunks) return;
  }
}

// ---------------------------------------------------------------------------
// reduce
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4 as_f4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ u32x4 as_u4(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t x = __builtin_bit_cast(uint32_t, f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

// Element kinds of the reductions (the values of the FSDP dtype codes).
enum : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

// float32 -> float16 bits, round to nearest, ties to even (the hardware
// conversion; overflow to infinity, float16 denormals kept).
__device__ __forceinline__ uint32_t f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// One element of kind E (its bits in the low bits of w) in float32, exactly.
template <int E>
__device__ __forceinline__ float elt_to_f32(uint32_t w) {
  if constexpr (E == kF32) return __builtin_bit_cast(float, w);
  else if constexpr (E == kBF16) return __builtin_bit_cast(float, w << 16);
  else return f16_to_f32(w & 0xffffu);
}
// float32 rounded once to kind E, as bits.
template <int E>
__device__ __forceinline__ uint32_t f32_to_elt(float f) {
  if constexpr (E == kF32) return __builtin_bit_cast(uint32_t, f);
  else if constexpr (E == kBF16) return bf16_rne(f);
  else return f16_rne(f);
}

// The values of one 16-byte vector in float32: 4 fp32, or 8 bf16 / fp16
// widened exactly.  16-bit element 2i is the low half of dword i.
template <int E>
struct Acc {
  static constexpr int N = E == kF32 ? 1 : 2;
  f32x4 v[N];
};

template <int E>
__device__ __forceinline__ Acc<E> widen(u32x4 w) {
  Acc<E> a;
  if constexpr (E == kF32) {
    a.v[0] = as_f4(w);
  } else if constexpr (E == kBF16) {
    const uint32_t hi = 0xffff0000u;
    a.v[0] = as_f4(u32x4{w.x << 16, w.x & hi, w.y << 16, w.y & hi});
    a.v[1] = as_f4(u32x4{w.z << 16, w.z & hi, w.w << 16, w.w & hi});
  } else {
    a.v[0] = f32x4{f16_to_f32(w.x & 0xffffu), f16_to_f32(w.x >> 16), f16_to_f32(w.y & 0xffffu),
                   f16_to_f32(w.y >> 16)};
    a.v[1] = f32x4{f16_to_f32(w.z & 0xffffu), f16_to_f32(w.z >> 16), f16_to_f32(w.w & 0xffffu),
                   f16_to_f32(w.w >> 16)};
  }
  return a;
}

template <int E>
__device__ __forceinline__ void accumulate(Acc<E>& a, u32x4 w) {
  const Acc<E> b = widen<E>(w);
#pragma unroll
  for (int i = 0; i < Acc<E>::N; ++i) a.v[i] = a.v[i] + b.v[i];
}

template <int E>
__device__ __forceinline__ u32x4 narrow(Acc<E>& a, int avg, float nf) {
  if (avg) {
#pragma unroll
    for (int i = 0; i < Acc<E>::N; ++i) a.v[i] = a.v[i] / nf;
  }
  if constexpr (E == kF32) {
    return as_u4(a.v[0]);
  } else {
    const f32x4 l = a.v[0], h = a.v[1];
    return u32x4{f32_to_elt<E>(l.x) | (f32_to_elt<E>(l.y) << 16), f32_to_elt<E>(l.z) | (f32_to_elt<E>(l.w) << 16),
                 f32_to_elt<E>(h.x) | (f32_to_elt<E>(h.y) << 16), f32_to_elt<E>(h.z) | (f32_to_elt<E>(h.w) << 16)};
  }
}

// Operand vector q: MODE 0 aligned, MODE 2 any shift r (two aligned
// blocks, realigned).
template <int MODE>
__device__ __forceinline__ u32x4 operand(const gvec* __restrict__ s, uint64_t q, uint32_t r) {
  if (MODE == 0) return ldv(s + q);
  return load_shifted(s, q, r);
}

template <int U, bool NTS>
__device__ __forceinline__ void store_vectors(const u32x4 (&o)[U], const fsdp::RedJob& jb,
                                              const uint64_t* __restrict__ ptr, uint64_t va, uint64_t j,
                                              uint64_t stride) {
  for (uint32_t m = 0; m < jb.ndst; ++m) {
    gvec* __restrict__ d = gptr<u32x4>(ptr[jb.dst0 + m] + va);
#pragma unroll
    for (int u = 0; u < U; ++u) stv<NTS>(d + j + u * stride, o[u]);
  }
}

// 16-byte blocks between the start of the 128-byte line holding address a
// and a.  The loops below start their lane-linear index that many blocks
// before the first vector, so that every wave's 64 consecutive blocks (1 KiB)
// cover whole lines of the operands: a line cut by two waves' ranges is
// requested by both, and under streaming loads the second request often
// misses L2 (measured on MI355X: the RS of the ragged-heavy set, whose
// slices sit at 4-byte offsets, fetched 3.5 % more than its operands hold
// with unrotated runs).  The blocks before the first vector lie in the line
// of the first one (never outside its page); they are read and discarded.
__device__ __forceinline__ uint32_t line_phase(uint64_t a) { return (uint32_t)((a >> 4) & 7u); }

// All data vectors [0, nv) of one job window for a compile-time operand
// count K, every operand aligned (MODE 0) or at shifts of its own (MODE 2):
// whole iterations of U vectors per lane with the K*U operand loads in
// flight together, then a tail of single vectors, the lanes rotated by the
// operands' common line phase e (line_phase; 0 when they differ).
template <int E, int K, int U, int MODE, bool NTS>
__device__ __forceinline__ void reduce_run(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                           const uint64_t (&sb)[K], const uint32_t (&sr)[K], uint64_t va,
                                           uint64_t nv, int avg, float nf, uint32_t e) {
  const uint64_t n = nv + e;  // lane-linear index j is vector j - e
  uint64_t base = 0;
  for (; base + (uint64_t)kBlock * U <= n; base += (uint64_t)kBlock * U) {
    u32x4 v[K][U];
    const uint64_t j = base + threadIdx.x;  // this lane's U indices are j + u * kBlock
#pragma unroll
    for (int t = 0; t < K; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) v[t][u] = operand<MODE>(gptr<u32x4>(sb[t]) - e, j + u * kBlock, sr[t]);
    u32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Acc<E> acc = widen<E>(v[0][u]);
#pragma unroll
      for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t][u]);
      o[u] = narrow<E>(acc, avg, nf);
    }
    if (base >= e) {  // every index of the iteration is a vector: U stores per destination
      store_vectors<U, NTS>(o, jb, ptr, va, j - e, kBlock);
    } else {  // the first iteration of a rotated run: the indices before vector 0 are not stored
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4 w[1] = {o[u]};
        if (j + u * kBlock >= e) store_vectors<1, NTS>(w, jb, ptr, va, j + u * kBlock - e, kBlock);
      }
    }
  }
  for (uint64_t j = base + threadIdx.x; j < n; j += kBlock) {
    u32x4 v[K];
#pragma unroll
    for (int t = 0; t < K; ++t) v[t] = operand<MODE>(gptr<u32x4>(sb[t]) - e, j, sr[t]);
    Acc<E> acc = widen<E>(v[0]);
#pragma unroll
    for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t]);
    const u32x4 o[1] = {narrow<E>(acc, avg, nf)};
    if (j >= e) store_vectors<1, NTS>(o, jb, ptr, va, j - e, kBlock);
  }
}

// Destination vectors per LDS piece of the shifted reduction (one 8 KiB
// reduce chunk at the default chunk size); its LDS holds the piece's result
// blocks and up to 7 blocks of line phase before them.
constexpr uint32_t kRedPiece = 512;
constexpr uint32_t kRedLds = kRedPiece + 8;

// All data vectors [0, nv) of one job window whose K operands share one
// shift r = 4*Q + b != 0 against the destination (compile-time K): the
// operands are summed block by block in their own aligned frame (block j =
// bytes [16 j, 16 j + 16) past sb[t]), each result block finished (AVG,
// 16-bit rounding; both act per element, so they commute with the shift)
// and written to LDS; destination vector q is then bytes [r, r + 16) of
// result blocks q and q + 1.  A piece of P destination vectors reads P + 1
// aligned blocks per operand (and the e blocks of their common line phase
// before them, line_phase), each once, and realigns only the results, not
// every operand.  Measured on MI355X on the RS of the ragged-heavy set (8
// slices at 4-byte shifts): realigning each operand in registers
// (neighbour lane's block through ds_bpermute, a closing block per operand
// and wave, one vector per lane) 1227 us; this path 1190 us; with the lanes
// rotated to the line phase 1166-1170 us, its fetched bytes 1.035 -> 1.011
// times its operands' (the rest: the line at each window edge, read by both
// windows; making those edge loads cacheable changes nothing, and moving
// the window edges to the operands' line starts, which splits a destination
// vector at every edge, fetched 1.028 times and took 1272 us).
template <int E, int K, int U, int Q, bool NTS>
__device__ __forceinline__ void reduce_run_lds(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                               const uint64_t (&sb)[K], uint64_t va, uint64_t nv, uint32_t b,
                                               int avg, float nf, u32x4* __restrict__ lds, uint32_t e) {
  // LDS slot i holds result block i - e
  for (uint64_t p0 = 0; p0 < nv; p0 += kRedPiece) {
    const uint32_t np = (uint32_t)((nv - p0) < kRedPiece ? (nv - p0) : kRedPiece);
    const uint32_t nb = np + 1 + e;  // result blocks p0 - e .. p0 + np
    uint32_t j0 = 0;
    for (; j0 + (uint32_t)kBlock * U <= nb; j0 += (uint32_t)kBlock * U) {
      u32x4 v[K][U];
#pragma unroll
      for (int t = 0; t < K; ++t) {
        const gvec* __restrict__ s = gptr<u32x4>(sb[t]) + p0 - e;
#pragma unroll
        for (int u = 0; u < U; ++u) v[t][u] = ldv(s + j0 + threadIdx.x + u * kBlock);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        Acc<E> acc = widen<E>(v[0][u]);
#pragma unroll
        for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t][u]);
        lds[j0 + threadIdx.x + u * kBlock] = narrow<E>(acc, avg, nf);
      }
    }
    for (uint32_t j = j0 + threadIdx.x; j < nb; j += kBlock) {
      u32x4 v[K];
#pragma unroll
      for (int t = 0; t < K; ++t) v[t] = ldv(gptr<u32x4>(sb[t]) + p0 - e + j);
      Acc<E> acc = widen<E>(v[0]);
#pragma unroll
      for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t]);
      lds[j] = narrow<E>(acc, avg, nf);
    }
    __syncthreads();
    for (uint32_t q = threadIdx.x; q < np; q += kBlock) {
      const u32x4 o[1] = {funnel<Q>(lds[q + e], lds[q + e + 1], b)};
      store_vectors<1, NTS>(o, jb, ptr, va, p0 + q, kBlock);
    }
    __syncthreads();  // the next piece reuses the LDS
  }
}

// Data vectors of one job window: destination vector q at byte offset
// va + 16 q of every destination, operand t read at the same offset of its
// source.  K > 0: compile-time operand count; K == 0: any count, one operand
// at a time.
template <int E, int K, bool NTS>
__device__ __forceinline__ void reduce_vectors(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                               uint64_t va, uint64_t nv, int avg, float nf,
                                               u32x4* __restrict__ lds) {
  if constexpr (K > 0) {
    constexpr int U = (K >= 3 || E != kF32) ? 2 : 4;
    // Operands at different shifts realign each operand in registers; with
    // 8 of them one vector per lane keeps the kernel at 4 waves per SIMD.
    constexpr int US = K >= 8 ? 1 : U;
    uint64_t sb[K];
    uint32_t sr[K];
    bool same = true, same_phase = true;
#pragma unroll
    for (int t = 0; t < K; ++t) {
      const uint64_t sa = ptr[jb.src0 + t] + va;
      sr[t] = (uint32_t)(sa & 15u);
      sb[t] = sa - sr[t];
      same = same && sr[t] == sr[0];
      same_phase = same_phase && line_phase(sb[t]) == line_phase(sb[0]);
    }
    // the lanes are rotated to the operands' common line phase; operands at
    // different phases are not rotated (a rotation by another operand's
    // phase could reach into the line before an operand's first one)
    const uint32_t e = same_phase ? line_phase(sb[0]) : 0u;
    if (same && sr[0] == 0) {
      reduce_run<E, K, U, 0, NTS>(jb, ptr, sb, sr, va, nv, avg, nf, e);
    } else if (same) {
      const uint32_t b = sr[0] & 3u;
      switch (sr[0] >> 2) {
        case 0: reduce_run_lds<E, K, U, 0, NTS>(jb, ptr, sb, va, nv, b, avg, nf, lds, e); break;
        case 1: reduce_run_lds<E, K, U, 1, NTS>(jb, ptr, sb, va, nv, b, avg, nf, lds, e); break;
        case 2: reduce_run_lds<E, K, U, 2, NTS>(jb, ptr, sb, va, nv, b, avg, nf, lds, e); break;
        default: reduce_run_lds<E, K, U, 3, NTS>(jb, ptr, sb, va, nv, b, avg, nf, lds, e); break;
      }
    } else {
      reduce_run<E, K, US, 2, NTS>(jb, ptr, sb, sr, va, nv, avg, nf, 0u);
    }
  } else {
    for (uint64_t j = threadIdx.x; j < nv; j += kBlock) {
      Acc<E> acc;
      for (uint32_t t = 0; t < jb.nsrc; ++t) {
        const uint64_t sa = ptr[jb.src0 + t] + va;
        const uint32_t r = (uint32_t)(sa & 15u);
        const u32x4 w = load_shifted(gptr<u32x4>(sa - r), j, r);
        if (t == 0)
          acc = widen<E>(w);
        else
          accumulate<E>(acc, w);
      }
      const u32x4 o[1] = {narrow<E>(acc, avg, nf)};
      store_vectors<1, NTS>(o, jb, ptr, va, j, kBlock);
    }
  }
}

// 16 operand bytes at byte address a: MODE 0 a is 16-byte aligned; MODE 1
// a is 4*Q + b bytes past an aligned block; MODE 2 any address.  Shifted
// reads take the two aligned blocks around the bytes (plain loads: the
// second block of a pair is an L1/L2 hit) and realign them.
template <int MODE, int Q>
__device__ __forceinline__ u32x4 row_operand(uint64_t a, uint32_t b) {
  if (MODE == 0) return ldv(gptr<u32x4>(a));
  const uint32_t r = (uint32_t)(a & 15u);
  const gvec* p = gptr<u32x4>(a - r);
  if (MODE == 1) return funnel<Q>(p[0], p[1], b);
  if (r == 0) return p[0];
  const u32x4 x = p[0], y = p[1];
  const uint32_t bb = r & 3u;
  switch (r >> 2) {
    case 0: return funnel<0>(x, y, bb);
    case 1: return funnel<1>(x, y, bb);
    case 2: return funnel<2>(x, y, bb);
    default: return funnel<3>(x, y, bb);
  }
}

// The whole destination vectors of a strided reduction block's chunk, for a
// compile-time operand count K: vector q of the flat range is row q / vpr,
// column q % vpr; operand t's bytes at sb[t] + the row's source offset, the
// result at every destination + the row's destination offset.  U vectors
// per lane per iteration with the K*U loads in flight together.
template <int E, int K, int MODE, int Q, bool NTS>
__device__ __forceinline__ void reduce_rows_run(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                                const uint64_t (&sb)[K], uint64_t doff, uint32_t nr, uint32_t vpr,
                                                uint32_t b, int avg, float nf) {
  // a shifted operand vector takes two loads: half as many per lane
  constexpr int U0 = (K >= 3 || E != kF32) ? 2 : 4;
  constexpr int U = MODE == 0 ? U0 : (U0 > 1 ? U0 / 2 : 1);
  const uint32_t nv = nr * vpr;
  auto store = [&](uint64_t dof, u32x4 o) {
    for (uint32_t m = 0; m < jb.ndst; ++m) stv<NTS>(gptr<u32x4>(ptr[jb.dst0 + m] + doff + dof), o);
  };
  uint32_t base = 0;
  for (; base + (uint32_t)kBlock * U <= nv; base += (uint32_t)kBlock * U) {
    u32x4 v[K][U];
    RowVec x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = row_vec(base + threadIdx.x + u * kBlock, vpr, jb.src_pitch, jb.dst_pitch);
#pragma unroll
    for (int t = 0; t < K; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) v[t][u] = row_operand<MODE, Q>(sb[t] + x[u].src, b);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Acc<E> acc = widen<E>(v[0][u]);
#pragma unroll
      for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t][u]);
      store(x[u].dst, narrow<E>(acc, avg, nf));
    }
  }
  for (uint32_t q = base + threadIdx.x; q < nv; q += kBlock) {
    const RowVec x = row_vec(q, vpr, jb.src_pitch, jb.dst_pitch);
    u32x4 v[K];
#pragma unroll
    for (int t = 0; t < K; ++t) v[t] = row_operand<MODE, Q>(sb[t] + x.src, b);
    Acc<E> acc = widen<E>(v[0]);
#pragma unroll
    for (int t = 1; t < K; ++t) accumulate<E>(acc, v[t]);
    store(x.dst, narrow<E>(acc, avg, nf));
  }
}

// The nr rows of a strided reduction block, element by element, as one
// flat range (element q is row q / epr, column q % epr), for pitches that
// are not multiples of 16.  Same arithmetic and operand order as the vector
// paths; a compile-time operand count keeps all K loads in flight.
template <int E, int K, bool NTS>
__device__ __forceinline__ void reduce_rows_elems(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                                  uint64_t soff, uint64_t doff, uint32_t nr, int avg, float nf) {
  typedef typename std::conditional<E == kF32, uint32_t, uint16_t>::type T;
  constexpr int ES = sizeof(T);
  const uint32_t epr = (uint32_t)(jb.nbytes / ES);
  const uint32_t n = nr * epr;
  auto offs = [&](uint32_t q, uint64_t* so, uint64_t* dof) {
    const uint32_t row = q / epr;
    const uint64_t col = (uint64_t)(q - row * epr) * ES;
    *so = row * jb.src_pitch + col;
    *dof = doff + row * jb.dst_pitch + col;
  };
  auto put = [&](uint64_t dof, float acc) {
    if (avg) acc = acc / nf;
    const T out = (T)f32_to_elt<E>(acc);
    for (uint32_t m = 0; m < jb.ndst; ++m) {
      if (NTS)
        __builtin_nontemporal_store(out, gptr<T>(ptr[jb.dst0 + m] + dof));
      else
        *gptr<T>(ptr[jb.dst0 + m] + dof) = out;
    }
  };
  uint32_t base = 0;
  if constexpr (K > 0) {
    // U elements per lane per iteration, all K*U loads in flight together
    constexpr int U = K >= 4 ? 2 : 4;
    uint64_t sb[K];
#pragma unroll
    for (int t = 0; t < K; ++t) sb[t] = ptr[jb.src0 + t] + soff;
    for (; base + (uint32_t)kBlock * U <= n; base += (uint32_t)kBlock * U) {
      uint64_t so[U], dof[U];
      T w[K][U];
#pragma unroll
      for (int u = 0; u < U; ++u) offs(base + threadIdx.x + u * kBlock, &so[u], &dof[u]);
#pragma unroll
      for (int t = 0; t < K; ++t)
#pragma unroll
        for (int u = 0; u < U; ++u) w[t][u] = __builtin_nontemporal_load(gptr<T>(sb[t] + so[u]));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float acc = elt_to_f32<E>((uint32_t)w[0][u]);
#pragma unroll
        for (int t = 1; t < K; ++t) acc = acc + elt_to_f32<E>((uint32_t)w[t][u]);
        put(dof[u], acc);
      }
    }
  }
  for (uint32_t q = base + threadIdx.x; q < n; q += kBlock) {
    uint64_t so, dof;
    offs(q, &so, &dof);
    float acc = 0.0f;
    for (uint32_t i = 0; i < jb.nsrc; ++i) {
      const float v = elt_to_f32<E>((uint32_t)*gptr<T>(ptr[jb.src0 + i] + soff + so));
      acc = (i == 0) ? v : acc + v;
    }
    put(dof, acc);
  }
}

// Chunk k of a strided reduction block (RedJob with rows > 1): rows
// [k*rows_per_chunk, ...).  When both pitches are multiples of 16, every row
// has the alignment of the first: a head of up to 15 destination bytes
// before its first aligned vector, whole vectors, a tail.  The whole
// vectors of all rows are one flat range; heads and tails are reduced
// element by element, one row end per lane, in the same operand order.
// Other pitches go element by element (reduce_rows_elems).
template <int E, int K, bool NTS>
__device__ __forceinline__ void reduce_rows(const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr, uint64_t k,
                                            int avg, float nf) {
  typedef typename std::conditional<E == kF32, uint32_t, uint16_t>::type T;
  constexpr int ES = sizeof(T);
  const uint64_t r0 = k * jb.rows_per_chunk;
  const uint64_t left = jb.rows - r0;
  const uint32_t nr = (uint32_t)(left < jb.rows_per_chunk ? left : jb.rows_per_chunk);
  const uint64_t B = jb.nbytes;
  const uint64_t soff = r0 * jb.src_pitch, doff = r0 * jb.dst_pitch;
  if ((jb.src_pitch | jb.dst_pitch) & 15u) {
    reduce_rows_elems<E, K, NTS>(jb, ptr, soff, doff, nr, avg, nf);
    return;
  }
  uint64_t head = (16u - (uint32_t)((ptr[jb.dst0] + doff) & 15u)) & 15u;
  if (head > B) head = B;
  const uint32_t vpr = (uint32_t)((B - head) >> 4);
  const uint64_t tail = head + ((uint64_t)vpr << 4);
  if (vpr) {
    if constexpr (K > 0) {
      uint64_t sb[K];
      bool same = true;
#pragma unroll
      for (int t = 0; t < K; ++t) {
        sb[t] = ptr[jb.src0 + t] + soff + head;
        same = same && ((sb[t] ^ sb[0]) & 15u) == 0;
      }
      const uint32_t r = (uint32_t)(sb[0] & 15u), b = r & 3u;
      const uint64_t dh = doff + head;
      if (same && r == 0) {
        reduce_rows_run<E, K, 0, 0, NTS>(jb, ptr, sb, dh, nr, vpr, 0, avg, nf);
      } else if (same) {
        switch (r >> 2) {
          case 0: reduce_rows_run<E, K, 1, 0, NTS>(jb, ptr, sb, dh, nr, vpr, b, avg, nf); break;
          case 1: reduce_rows_run<E, K, 1, 1, NTS>(jb, ptr, sb, dh, nr, vpr, b, avg, nf); break;
          case 2: reduce_rows_run<E, K, 1, 2, NTS>(jb, ptr, sb, dh, nr, vpr, b, avg, nf); break;
          default: reduce_rows_run<E, K, 1, 3, NTS>(jb, ptr, sb, dh, nr, vpr, b, avg, nf); break;
        }
      } else {
        reduce_rows_run<E, K, 2, 0, NTS>(jb, ptr, sb, dh, nr, vpr, 0, avg, nf);
      }
    } else {
      const uint32_t nv = nr * vpr;
      for (uint32_t q = threadIdx.x; q < nv; q += kBlock) {
        const RowVec x = row_vec(q, vpr, jb.src_pitch, jb.dst_pitch);
        Acc<E> acc = widen<E>(row_operand<2, 0>(ptr[jb.src0] + soff + head + x.src, 0));
        for (uint32_t t = 1; t < jb.nsrc; ++t)
          accumulate<E>(acc, row_operand<2, 0>(ptr[jb.src0 + t] + soff + head + x.src, 0));
        const u32x4 o = narrow<E>(acc, avg, nf);
        for (uint32_t m = 0; m < jb.ndst; ++m) stv<NTS>(gptr<u32x4>(ptr[jb.dst0 + m] + doff + head + x.dst), o);
      }
    }
  }
  if (head || tail < B) {
    for (uint32_t t = threadIdx.x; t < 2 * nr; t += kBlock) {
      const uint64_t row = t >> 1;
      const uint64_t lo = (t & 1) ? tail : 0, hi = (t & 1) ? B : head;
      for (uint64_t x = lo; x < hi; x += ES) {
        const uint64_t so = soff + row * jb.src_pitch + x;
        float acc = 0.0f;
        for (uint32_t i = 0; i < jb.nsrc; ++i) {
          const T w = *gptr<T>(ptr[jb.src0 + i] + so);
          const float v = elt_to_f32<E>((uint32_t)w);
          acc = (i == 0) ? v : acc + v;
        }
        if (avg) acc = acc / nf;
        const T out = (T)f32_to_elt<E>(acc);
        const uint64_t dof = doff + row * jb.dst_pitch + x;
        for (uint32_t m = 0; m < jb.ndst; ++m) *gptr<T>(ptr[jb.dst0 + m] + dof) = out;
      }
    }
  }
}

// Elements [max(a, lo), min(a + 16, hi)) of the 16-byte vector at d0-relative
// address a: reduced below the data end, zero above it.
template <int E>
__device__ __forceinline__ void reduce_partial(uint64_t a, uint64_t lo, uint64_t hi, uint64_t cend,
                                               const fsdp::RedJob& jb, const uint64_t* __restrict__ ptr,
                                               uint64_t d0, int avg, float nf) {
  typedef typename std::conditional<E == kF32, uint32_t, uint16_t>::type T;
  constexpr int ES = sizeof(T);
  const uint64_t x0 = a > lo ? a : lo;
  const uint64_t x1 = (a + 16) < hi ? (a + 16) : hi;
  for (uint64_t x = x0; x < x1; x += ES) {
    const uint64_t off = x - d0;
    T out = 0;
    if (x < cend) {
      float acc = 0.0f;
      for (uint32_t t = 0; t < jb.nsrc; ++t) {
        const T w = *gptr<T>(ptr[jb.src0 + t] + off);
        const float v = elt_to_f32<E>((uint32_t)w);
        acc = (t == 0) ? v : acc + v;
      }
      if (avg) acc = acc / nf;
      out = (T)f32_to_elt<E>(acc);
    }
    for (uint32_t m = 0; m < jb.ndst; ++m) *gptr<T>(ptr[jb.dst0 + m] + off) = out;
  }
}

template <int E, int K, bool NTS>
__global__ __launch_bounds__(kBlock) void reduce_kernel(const uint64_t* __restrict__ begin,
                                                        const fsdp::RedJob* __restrict__ jobs,
                                                        const uint64_t* __restrict__ ptr,
                                                        uint32_t n_job, uint64_t n_chunks,
                                                        uint32_t shift, int avg) {
  // result blocks of the shifted path (reduce_run_lds)
  __shared__ u32x4 lds[kRedLds];
  const uint64_t CH = uint64_t(1) << shift;
  for (uint64_t slot = blockIdx.x; slot < n_chunks; slot += gridDim.x) {
    const uint64_t c = xcd_chunk(slot, n_chunks);
    const uint32_t j = find_item(begin, n_job, c);
    const fsdp::RedJob jb = jobs[j];
    const uint64_t k = c - begin[j];
    if (jb.rows > 1) {
      reduce_rows<E, K, NTS>(jb, ptr, k, avg, (float)jb.nsrc);
      continue;
    }
    const uint64_t d0 = ptr[jb.dst0];
    const uint64_t base = (d0 >> shift) << shift;
    const uint64_t w0 = base + k * CH;
    const uint64_t lo = w0 > d0 ? w0 : d0;
    const uint64_t end = d0 + jb.nbytes;
    const uint64_t hi = (w0 + CH) < end ? (w0 + CH) : end;
    const uint64_t cend = d0 + jb.data_bytes;
    const float nf = (float)jb.nsrc;

    // whole vectors of data: offsets [va, vb) relative to d0
    const uint64_t ca = align_up16(lo);
    const uint64_t cb = align_down16(hi < cend ? hi : cend);
    if (ca < cb) reduce_vectors<E, K, NTS>(jb, ptr, ca - d0, (cb - ca) >> 4, avg, nf, lds);
    // whole vectors of padding (zero) in every destination
    const uint64_t za = align_up16(lo > cend ? lo : cend);
    const uint64_t zb = align_down16(hi);
    if (za < zb) {
      for (uint32_t m = 0; m < jb.ndst; ++m) zero_vectors<kBlock, NTS>(ptr[jb.dst0 + m] + (za - d0), (zb - za) >> 4);
    }
    // vectors cut by the window start, the data/padding edge, the job end
    if (threadIdx.x < 3) {
      const uint64_t a_lo = align_down16(lo);
      const uint64_t a_c = align_down16(cend);
      const uint64_t a_hi = align_down16(hi);
      const bool p_lo = (lo & 15) != 0;
      const bool p_c = (cend & 15) != 0 && lo < cend && cend < hi && !(p_lo && a_c == a_lo);
      const bool p_hi = (hi & 15) != 0 && !(p_lo && a_hi == a_lo) && !(p_c && a_hi == a_c);
      if (threadIdx.x == 0 && p_lo) reduce_partial<E>(a_lo, lo, hi, cend, jb, ptr, d0, avg, nf);
      if (threadIdx.x == 1 && p_c) reduce_partial<E>(a_c, lo, hi, cend, jb, ptr, d0, avg, nf);
      if (threadIdx.x == 2 && p_hi) reduce_partial<E>(a_hi, lo, hi, cend, jb, ptr, d0, avg, nf);
    }
  }
}

// ---------------------------------------------------------------------------
// fold_copy
// ---------------------------------------------------------------------------

// Rows [r0, r0 + nr) of a fold item in W-sized units: unit q of the chunk is
// full-tensor row q / upf of the chunk, rank s = (q % upf) / upr and unit
// col = q % upr of that rank's piece.  Its full-side offset is q units from
// the chunk's first full row (the full side is contiguous), its rank-side
// address rank0 + s * rank_pitch + (r0 + row) * run_bytes + col units.
// Consecutive lanes take consecutive full-side units, so both sides are
// read and written in whole lines.  U units per lane per iteration, all
// loads before the first store; the units left after the whole iterations
// take one more such iteration with predicated stores (a loop of one unit
// at a time would cost a memory round trip per unit).
template <typename W, bool NTS, int UL = 0>
__device__ __forceinline__ void fold_units(const fsdp::FoldSeg& f, uint64_t r0, uint32_t nr) {
  constexpr int U = UL > 0 ? UL : sizeof(W) >= 16 ? 4 : 8;
  const uint32_t upr = (uint32_t)(f.run_bytes / sizeof(W));
  const uint32_t upf = f.nrank * upr;
  const uint32_t n = nr * upf;
  const uint32_t run = (uint32_t)f.run_bytes;
  const uint64_t full0 = f.full + r0 * f.nrank * f.run_bytes;
  const uint64_t rank0 = f.rank0 + r0 * f.run_bytes;
  auto rank_addr = [&](uint32_t q) -> uint64_t {
    const uint32_t row = q / upf;
    const uint32_t rem = q - row * upf;
    const uint32_t s = rem / upr;
    const uint32_t col = rem - s * upr;
    return rank0 + s * f.rank_pitch + (row * run + col * (uint32_t)sizeof(W));
  };
  auto ld = [](uint64_t a) { return __builtin_nontemporal_load(gptr<W>(a)); };
  auto st = [](uint64_t a, W v) {
    if (NTS)
      __builtin_nontemporal_store(v, gptr<W>(a));
    else
      *gptr<W>(a) = v;
  };
  uint32_t base = 0;
  for (; base + (uint32_t)kBlock * U <= n; base += (uint32_t)kBlock * U) {
    W v[U];
    if (f.gather) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld(rank_addr(base + threadIdx.x + u * kBlock));
#pragma unroll
      for (int u = 0; u < U; ++u) st(full0 + (uint64_t)(base + threadIdx.x + u * kBlock) * sizeof(W), v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld(full0 + (uint64_t)(base + threadIdx.x + u * kBlock) * sizeof(W));
#pragma unroll
      for (int u = 0; u < U; ++u) st(rank_addr(base + threadIdx.x + u * kBlock), v[u]);
    }
  }
  if (base < n) {  // the rest: one iteration, all loads first
    // lanes past the end load the last unit again (no branch around the
    // loads, which made the compiler wait for each load before the next)
    // and store nothing
    W v[U];
    if (f.gather) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + threadIdx.x + u * kBlock;
        v[u] = ld(rank_addr(q < n ? q : n - 1));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + threadIdx.x + u * kBlock;
        if (q < n) st(full0 + (uint64_t)q * sizeof(W), v[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + threadIdx.x + u * kBlock;
        v[u] = ld(full0 + (uint64_t)(q < n ? q : n - 1) * sizeof(W));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = base + threadIdx.x + u * kBlock;
        if (q < n) st(rank_addr(q), v[u]);
      }
    }
  }
}

// LDS staging of a fold chunk.  The chunk's source bytes are read as the
// aligned 16-byte blocks that hold them (each block holds at least one byte
// of its range, so no read leaves the source's pages) and kept in LDS; the
// destination is then written in aligned 16-byte vectors, each assembled
// element by element (G: 2 or 4 bytes, dividing the unit) from its permuted
// place in LDS, and the destination ends (under 16 bytes each) element by
// element.  Gather: LDS window s holds rank s's rows of the chunk, the full
// rows are written.  Scatter: LDS holds the full rows, every rank's rows
// are written.  Used for 2- and 4-byte units (measured on MI355X against the
// unit-wise path: AG copy-out 18-27 % faster, RS copy-in up to 2.4x; with 8-
// and 16-byte units it is 5-25 % slower).  A chunk whose windows do not fit
// kFoldLds keeps the unit-wise path.
constexpr uint32_t kFoldLds = 18u * 1024u;

// LDS bytes a fold chunk of nr rows needs (0: it does not fit).
__device__ __forceinline__ uint32_t fold_lds_bytes(const fsdp::FoldSeg& f, uint64_t r0, uint32_t nr) {
  const uint64_t L = (uint64_t)nr * f.run_bytes;
  uint64_t need;
  if (f.gather) {
    need = (uint64_t)f.nrank * ((L + 15) / 16 + 1) * 16;
  } else {
    const uint64_t F0 = f.full + r0 * f.nrank * f.run_bytes;
    need = align_up16(F0 + L * f.nrank) - align_down16(F0);
  }
  return need <= kFoldLds ? (uint32_t)need : 0u;
}

// Loads in flight per lane while a chunk is staged through LDS: a loop of
// one load and one LDS store per block waits a whole memory round trip per
// block, which caps each workgroup's share of the bandwidth.  Five blocks per
// lane cover the whole 18 KiB staging buffer (1152 blocks) in one pass; with
// four, the few blocks past 1024 (each rank window's edge block of a gather,
// a scatter's row-edge blocks) cost every chunk a second round trip.
// Measured on MI355X: RS copy-in of (30000, 2050, 1) and (20000, 1540) bf16
// on dim 1 3-4 % faster, AG copy-outs of short-row gathers 1-2 % faster,
// six blocks per lane no better.
#ifndef FSDP_FOLD_STAGE
#define FSDP_FOLD_STAGE 5
#endif
constexpr int kStage = FSDP_FOLD_STAGE;
static_assert(FSDP_FOLD_STAGE < 5 || (uint32_t)kStage * kBlock * 16u >= kFoldLds,
              "one staging pass covers the LDS buffer");

// x / d in one high multiply, exact whenever x * d < 2^32: with
// m = ceil(2^32 / d), x * m / 2^32 exceeds x / d by less than x / 2^32, which
// is below 1 / d, so the floor never reaches the next integer.  The LDS paths
// of the fold kernels divide offsets inside one chunk's staging window by
// sizes inside it (both below 2^15), once per vector; the generic 32-bit
// division takes a reciprocal and two correction steps each time.
struct FastDiv {
  uint32_t m;  // 0 stands for d = 1
  __device__ __forceinline__ explicit FastDiv(uint32_t d) : m(d > 1u ? 0xFFFFFFFFu / d + 1u : 0u) {}
  __device__ __forceinline__ uint32_t operator()(uint32_t x) const { return m ? __umulhi(x, m) : x; }
};

// Stages blocks [0, n) of a chunk in LDS: block i (16 bytes at the aligned
// global address src(i), or nothing when src(i) is 0) goes to LDS bytes
// [16 i, 16 i + 16); each lane issues up to kStage loads before their LDS
// stores.
template <typename Src>
__device__ __forceinline__ void stage_blocks(uint8_t* lds, uint32_t n, Src src) {
  for (uint32_t i0 = threadIdx.x; i0 < n; i0 += (uint32_t)kStage * kBlock) {
    u32x4 v[kStage];
    uint64_t a[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const uint32_t i = i0 + u * kBlock;
      a[u] = i < n ? src(i) : 0;
      if (a[u]) v[u] = ldv(gptr<u32x4>(a[u]));
    }
#pragma unroll
    for (int u = 0; u < kStage; ++u)
      if (a[u]) *reinterpret_cast<u32x4*>(lds + 16u * (i0 + u * kBlock)) = v[u];
  }
}

// Reduces blocks [0, n) of a chunk into LDS: block i of every operand t
// (16 bytes at sb[t] + 16 i) summed in operand order, finished (AVG, 16-bit
// rounding) and stored at LDS bytes [16 i, 16 i + 16); each lane issues the
// K loads of two blocks (of one for K = 8) before the first add.  Measured on
// MI355X: two blocks make the 4-rank fold reductions 2-3.5 % faster than
// one; over 8 ranks they cost occupancy and run 2 % slower.
template <int E, int K>
__device__ __forceinline__ void reduce_blocks(uint8_t* lds, uint32_t n, const uint64_t (&sb)[K], int avg,
                                              float nf) {
  constexpr int B = K >= 8 ? 1 : 2;
  for (uint32_t i0 = threadIdx.x; i0 < n; i0 += (uint32_t)B * kBlock) {
    u32x4 v[B][K];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t i = i0 + u * kBlock;
      if (i < n) {
#pragma unroll
        for (int t = 0; t < K; ++t) v[u][t] = ldv(gptr<u32x4>(sb[t] + (uint64_t)i * 16));
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const uint32_t i = i0 + u * kBlock;
      if (i < n) {
        Acc<E> acc = widen<E>(v[u][0]);
#pragma unroll
        for (int t = 1; t < K; ++t) accumulate<E>(acc, v[u][t]);
        *reinterpret_cast<u32x4*>(lds + 16u * i) = narrow<E>(acc, avg, nf);
      }
    }
  }
}

// The element runs [lo, hi) of a destination range not covered by its whole
// aligned vectors: its head and tail, or all of it when it has no whole
// vector.  Element x (absolute address) gets get(x).
template <typename G, bool NTS, typename Get>
__device__ __forceinline__ void fold_ends(uint64_t lo, uint64_t hi, uint32_t lane_task, Get get) {
  const uint64_t va = align_up16(lo), vb = align_down16(hi);
  uint64_t a, b;
  if (va < vb) {
    a = lane_task == 0 ? lo : vb;
    b = lane_task == 0 ? va : hi;
  } else {
    a = lane_task == 0 ? lo : hi;
    b = hi;
  }
  for (uint64_t x = a; x < b; x += sizeof(G)) {
    const G v = get(x);
    if (NTS)
      __builtin_nontemporal_store(v, gptr<G>(x));
    else
      *gptr<G>(x) = v;
  }
}

__device__ __forceinline__ u32x4 lds_vec(const uint8_t* lds, uint32_t o);
template <typename G>
__device__ __forceinline__ u32x4 pack_elts(const G (&e)[16 / sizeof(G)]);

// Bytes [0, k) of a and [k, 16) of b (0 < k < 16): a destination vector
// that spans the end of one run and the start of the next.
__device__ __forceinline__ u32x4 merge_bytes(u32x4 a, u32x4 b, uint32_t k) {
  auto m = [k](int d) {
    const int r = (int)k - 4 * d;
    return r <= 0 ? 0u : r >= 4 ? ~0u : (1u << (8 * r)) - 1u;
  };
  return u32x4{(a.x & m(0)) | (b.x & ~m(0)), (a.y & m(1)) | (b.y & ~m(1)), (a.z & m(2)) | (b.z & ~m(2)),
               (a.w & m(3)) | (b.w & ~m(3))};
}

// Scatter of an LDS-staged chunk of nr full rows (S runs of run bytes each,
// full-side byte x at LDS byte delta + x, nblk blocks staged): rank s's L =
// nr * run bytes go to dst(s) in aligned 16-byte vectors and element-wise
// ends.  With 2-byte elements and runs of at least 16 bytes a vector is one
// unaligned LDS read (inside a run) or two merged ones (across the end of a
// row), else it is assembled element by element (4-byte elements take as
// many LDS reads either way, and measured faster element by element); the
// choice is per chunk, so each loop keeps its own schedule.
template <typename G, bool NTS, typename Dst>
__device__ __forceinline__ void scatter_rows(const uint8_t* lds, uint32_t delta, uint32_t nblk, uint32_t S,
                                             uint32_t run, uint32_t nr, Dst dst) {
  constexpr uint32_t gb = sizeof(G);
  constexpr uint32_t NE = 16 / gb;
  const uint32_t FR = S * run, L = nr * run;
  auto rd = [&](uint32_t off) { return *reinterpret_cast<const G*>(lds + off); };
  // rank s's byte y of the chunk: row y / run, column y % run
  auto at = [&](uint32_t row, uint32_t s, uint32_t col) { return delta + row * FR + s * run + col; };
  auto elements = [&](uint32_t s, uint32_t row, uint32_t col) {
    G e[NE];
#pragma unroll
    for (uint32_t k = 0; k < NE; ++k) {
      e[k] = rd(at(row, s, col));
      col += gb;
      if (col == run) col = 0, ++row;
    }
    return pack_elts<G>(e);
  };
  const uint32_t vmax = L / 16;  // whole vectors of one rank's L bytes, at most
  // i < S * vmax and y < L, both within the staged window (below 2^15)
  const FastDiv by_vmax(vmax), by_run(run);
  if (gb == 2 && run >= 16) {
    for (uint32_t i = threadIdx.x; i < S * vmax; i += kBlock) {
      const uint32_t s = by_vmax(i), j = i - s * vmax;
      const uint64_t d = dst(s);
      const uint64_t va = align_up16(d), vb = align_down16(d + L);
      if (va + (uint64_t)j * 16 >= vb) continue;
      const uint32_t y = (uint32_t)(va - d) + j * 16;
      const uint32_t row = by_run(y), col = y - row * run;
      // rank s's bytes from col of row on, then (k1 < 16) from the start of
      // its next row
      const uint32_t k1 = run - col, o = at(row, s, col);
      const uint32_t o2 = k1 < 16 ? at(row + 1, s, 0) - k1 : 0u;
      u32x4 v;
      if (k1 >= 16 && o + 20 <= nblk * 16)
        v = lds_vec(lds, o);
      else if (o + 20 <= nblk * 16 && o2 + 20 <= nblk * 16)
        v = merge_bytes(lds_vec(lds, o), lds_vec(lds, o2), k1);
      else
        v = elements(s, row, col);
      stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), v);
    }
  } else {
    for (uint32_t i = threadIdx.x; i < S * vmax; i += kBlock) {
      const uint32_t s = by_vmax(i), j = i - s * vmax;
      const uint64_t d = dst(s);
      const uint64_t va = align_up16(d), vb = align_down16(d + L);
      if (va + (uint64_t)j * 16 >= vb) continue;
      const uint32_t y = (uint32_t)(va - d) + j * 16;
      const uint32_t row = by_run(y);
      stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), elements(s, row, y - row * run));
    }
  }
  for (uint32_t t = threadIdx.x; t < 2 * S; t += kBlock) {
    const uint32_t s = t >> 1;
    const uint64_t d = dst(s);
    fold_ends<G, NTS>(d, d + L, t & 1u, [&](uint64_t ya) {
      const uint32_t y = (uint32_t)(ya - d);
      const uint32_t row = y / run;
      return rd(at(row, s, y - row * run));
    });
  }
}

template <typename G, bool NTS>
__device__ __forceinline__ void fold_lds(const fsdp::FoldSeg& f, uint64_t r0, uint32_t nr, uint8_t* lds) {
  constexpr uint32_t gb = sizeof(G);
  constexpr uint32_t NE = 16 / gb;
  const uint32_t S = f.nrank, run = (uint32_t)f.run_bytes;
  const uint32_t FR = S * run, L = nr * run;
  const uint64_t F0 = f.full + r0 * FR;
  const uint64_t R0 = f.rank0 + r0 * run;  // rank s's rows of the chunk start at R0 + s * rank_pitch
  auto rd = [&](uint32_t off) { return *reinterpret_cast<const G*>(lds + off); };
  auto pack = [](const G (&e)[NE]) {
    u32x4 v;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (uint32_t k = 0; k < NE; ++k) w[k * gb / 4] |= (uint32_t)e[k] << ((k * gb) % 4 * 8);
    v.x = w[0], v.y = w[1], v.z = w[2], v.w = w[3];
    return v;
  };
  if (f.gather) {
    // window s: the aligned blocks of rank s's L bytes, rank byte y at
    // s * nb * 16 + (rank base & 15) + y
    const uint32_t nb = (L + 15) / 16 + 1;
    // block indices, chunk offsets and sizes all lie within the staged
    // window (below 2^15)
    const FastDiv by_nb(nb), by_fr(FR), by_run(run);
    stage_blocks(lds, S * nb, [&](uint32_t i) -> uint64_t {
      const uint32_t s = by_nb(i), k = i - s * nb;
      const uint64_t a = R0 + s * f.rank_pitch;
      const uint64_t blk = align_down16(a) + (uint64_t)k * 16;
      return blk < align_up16(a + L) ? blk : 0;
    });
    __syncthreads();
    // full-side byte x of the chunk: row x / FR, rank (x % FR) / run, column x % run
    auto at = [&](uint32_t row, uint32_t s, uint32_t col) {
      return s * nb * 16 + (uint32_t)((R0 + s * f.rank_pitch) & 15u) + row * run + col;
    };
    const uint64_t va = align_up16(F0), vb = align_down16(F0 + (uint64_t)nr * FR);
    const uint32_t nv = va < vb ? (uint32_t)((vb - va) >> 4) : 0u;
    const uint32_t x0 = (uint32_t)(va - F0);
    const uint32_t staged = S * nb * 16;
    // 2-byte elements and runs of at least 16 bytes: whole vectors from LDS
    // (as in scatter_rows)
    const bool vec = gb == 2 && run >= 16;
    auto elements = [&](uint32_t row, uint32_t s, uint32_t col) {
      G e[NE];
#pragma unroll
      for (uint32_t k = 0; k < NE; ++k) {
        e[k] = rd(at(row, s, col));
        col += gb;
        if (col == run) {
          col = 0;
          if (++s == S) s = 0, ++row;
        }
      }
      return pack(e);
    };
    if (vec) {
      for (uint32_t j = threadIdx.x; j < nv; j += kBlock) {
        const uint32_t x = x0 + j * 16;
        const uint32_t row = by_fr(x);
        const uint32_t rem = x - row * FR;
        const uint32_t s = by_run(rem), col = rem - s * run;
        // the vector's bytes in rank s's row from col on, then (k1 < 16)
        // in the next piece of the full row (rank s + 1, or rank 0 of the
        // next row): one or two unaligned LDS reads
        const uint32_t k1 = run - col, o = at(row, s, col);
        const uint32_t o2 = k1 < 16 ? (s + 1 == S ? at(row + 1, 0, 0) : at(row, s + 1, 0)) - k1 : 0u;
        u32x4 v;
        if (k1 >= 16 && o + 20 <= staged)
          v = lds_vec(lds, o);
        else if (o + 20 <= staged && o2 + 20 <= staged)
          v = merge_bytes(lds_vec(lds, o), lds_vec(lds, o2), k1);
        else
          v = elements(row, s, col);
        stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), v);
      }
    } else {
      for (uint32_t j = threadIdx.x; j < nv; j += kBlock) {
        const uint32_t x = x0 + j * 16;
        const uint32_t row = by_fr(x);
        const uint32_t rem = x - row * FR;
        const uint32_t s = by_run(rem);
        stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), elements(row, s, rem - s * run));
      }
    }
    if (threadIdx.x < 2) {
      fold_ends<G, NTS>(F0, F0 + (uint64_t)nr * FR, threadIdx.x, [&](uint64_t xa) {
        const uint32_t x = (uint32_t)(xa - F0);
        const uint32_t row = x / FR, rem = x - row * FR, s = rem / run;
        return rd(at(row, s, rem - s * run));
      });
    }
  } else {
    // LDS byte delta + x is full-side byte x of the chunk
    const uint64_t fa = align_down16(F0);
    const uint32_t delta = (uint32_t)(F0 - fa);
    const uint32_t nblk = (uint32_t)((align_up16(F0 + (uint64_t)nr * FR) - fa) >> 4);
    stage_blocks(lds, nblk, [&](uint32_t i) -> uint64_t { return fa + (uint64_t)i * 16; });
    __syncthreads();
    scatter_rows<G, NTS>(lds, delta, nblk, S, run, nr, [&](uint32_t s) { return R0 + s * f.rank_pitch; });
  }
  __syncthreads();  // the next chunk reuses the LDS
}

// Flat chunks of a fold item whose full-tensor row does not fit one chunk
// (rows_per_chunk == 0, fsdp::FoldSeg): the full tensor is contiguous, so
// chunk k is its bytes [X0, X1) = [k sub, (k + 1) sub) (the last one
// shorter), whatever rows they cross.  The full tensor is a sequence of
// pieces of run bytes, piece p being row p / S of rank p % S; the chunk
// meets pieces p_lo .. p_hi, piece p's part being its bytes [a, b)
// (chunk-relative, a multiple of the unit apart).  Each part is contiguous
// on both sides; the chunk is staged through LDS so that both sides move
// aligned 16-byte vectors, the ends element by element (G-sized elements,
// 2 or 4 bytes).
struct FlatChunk {
  uint64_t X0;      // first full-tensor byte
  uint32_t n;       // bytes
  uint64_t p_lo;    // first piece
  uint32_t off0;    // X0 - p_lo * run (< run)
  uint32_t pieces;  // p_hi - p_lo + 1
};

__device__ __forceinline__ FlatChunk flat_chunk(uint64_t k, uint64_t total, uint32_t sub, uint32_t run) {
  FlatChunk c;
  c.X0 = k * sub;
  c.n = (uint32_t)(total - c.X0 < sub ? total - c.X0 : sub);
  c.p_lo = c.X0 / run;
  c.off0 = (uint32_t)(c.X0 - c.p_lo * run);
  c.pieces = (c.off0 + c.n - 1) / run + 1;
  return c;
}

// Piece q of a chunk (q < pieces): chunk-relative bytes [a, b).
__device__ __forceinline__ void flat_part(const FlatChunk& c, uint32_t run, uint32_t q, uint32_t* a, uint32_t* b) {
  const uint32_t lo = q * run, hi = lo + run;  // in off0-shifted coordinates
  *a = (lo > c.off0 ? lo : c.off0) - c.off0;
  *b = (hi < c.off0 + c.n ? hi : c.off0 + c.n) - c.off0;
}

// LDS bytes kept at the end of the fold LDS for the gather's window table
// (one FlatWin per piece, at most kFlatWinMax pieces, then one entry whose
// start is the blocks of all windows).
constexpr uint32_t kFlatAdj = 256;
struct FlatWin {
  uint64_t blk0;   // first aligned global block of the window
  uint32_t start;  // first LDS block of the window
  int32_t adj;     // LDS offset of chunk byte 0 in the piece's frame
};
constexpr uint32_t kFlatWinMax = kFlatAdj / sizeof(FlatWin) - 1;
static_assert(fsdp::kFlatMaxPieces <= kFlatWinMax, "a flat chunk's windows must fit the LDS table");

template <typename G>
__device__ __forceinline__ u32x4 pack_elts(const G (&e)[16 / sizeof(G)]) {
  constexpr uint32_t gb = sizeof(G);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (uint32_t k = 0; k < 16 / gb; ++k) w[k * gb / 4] |= (uint32_t)e[k] << ((k * gb) % 4 * 8);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// The 16 bytes at LDS byte offset o (a multiple of the element): four
// dwords when o is 4-byte aligned, else five from the one holding o,
// realigned (the fifth may lie past the bytes written, never past the LDS
// array).
__device__ __forceinline__ u32x4 lds_vec(const uint8_t* lds, uint32_t o) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(lds + (o & ~3u));
  const uint32_t b = o & 3u;
  if (b == 0) return u32x4{w[0], w[1], w[2], w[3]};
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
  return u32x4{__builtin_amdgcn_alignbyte(w1, w0, b), __builtin_amdgcn_alignbyte(w2, w1, b),
               __builtin_amdgcn_alignbyte(w3, w2, b), __builtin_amdgcn_alignbyte(w4, w3, b)};
}

// Scatter of a flat chunk whose full-tensor bytes sit in LDS at offset
// delta + (chunk-relative byte): every piece's part, piece p's at
// dst(p, a) (its bytes from the part's start), written as aligned vectors
// (16 consecutive LDS bytes each) and element-wise ends.
template <typename G, bool NTS, typename Dst>
__device__ __forceinline__ void flat_scatter(const FlatChunk& c, uint32_t run, uint32_t delta, const uint8_t* lds,
                                             Dst dst) {
  for (uint32_t q = 0; q < c.pieces; ++q) {
    uint32_t a, b;
    flat_part(c, run, q, &a, &b);
    const uint64_t d = dst(c.p_lo + q, a);
    const uint64_t va = align_up16(d), vb = align_down16(d + (b - a));
    const uint32_t nv = va < vb ? (uint32_t)((vb - va) >> 4) : 0u;
    const uint32_t o0 = delta + a + (uint32_t)(va - d);
    for (uint32_t j = threadIdx.x; j < nv; j += kBlock)
      stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), lds_vec(lds, o0 + j * 16));
    if (threadIdx.x < 2)
      fold_ends<G, NTS>(d, d + (b - a), threadIdx.x, [&](uint64_t y) {
        return *reinterpret_cast<const G*>(lds + delta + a + (uint32_t)(y - d));
      });
  }
}

template <typename G, bool NTS>
__device__ __forceinline__ void fold_flat(const fsdp::FoldSeg& f, uint64_t k, uint8_t* lds) {
  constexpr uint32_t gb = sizeof(G);
  constexpr uint32_t NE = 16 / gb;
  const uint32_t run = (uint32_t)f.run_bytes, S = f.nrank;
  const FlatChunk c = flat_chunk(k, f.rows * S * run, f.reserved, run);
  const uint64_t F = f.full + c.X0;  // the chunk's first full-tensor byte
  // rank-side address of byte a (chunk-relative) of piece p
  auto src = [&](uint64_t p, uint32_t a) {
    const uint64_t r = p / S;
    const uint32_t s = (uint32_t)(p - r * S);
    return f.rank0 + s * f.rank_pitch + r * run + (c.X0 + a - p * run);
  };
  if (f.gather) {
    // window of piece q: the aligned blocks of its part, the windows one
    // after another in LDS.  Lane q < pieces describes window q in the
    // table at the end of the LDS: its first global block, its first LDS
    // block, and adj = the LDS offset of chunk byte 0 in piece q's frame.
    FlatWin* win = reinterpret_cast<FlatWin*>(lds + kFoldLds - kFlatAdj);
    auto window = [&](uint32_t q, uint64_t* blk0, uint32_t* a) {
      uint32_t b;
      flat_part(c, run, q, a, &b);
      const uint64_t p = src(c.p_lo + q, *a);
      *blk0 = align_down16(p);
      return p;
    };
    auto blocks = [&](uint32_t q) {
      uint64_t blk0;
      uint32_t a, b;
      const uint64_t p = window(q, &blk0, &a);
      flat_part(c, run, q, &a, &b);
      return (uint32_t)((align_up16(p + (b - a)) - blk0) >> 4);
    };
    if (threadIdx.x < c.pieces) {
      const uint32_t q = threadIdx.x;
      uint32_t start = 0;
      for (uint32_t k = 0; k < q; ++k) start += blocks(k);
      uint64_t blk0;
      uint32_t a;
      const uint64_t p = window(q, &blk0, &a);
      win[q] = FlatWin{blk0, start, (int32_t)(start * 16 + (uint32_t)(p & 15u)) - (int32_t)a};
      if (q + 1 == c.pieces) win[kFlatWinMax].start = start + blocks(q);  // the blocks of all windows
    }
    __syncthreads();
    stage_blocks(lds, win[kFlatWinMax].start, [&](uint32_t i) -> uint64_t {
      uint32_t q = 0;
      while (q + 1 < c.pieces && win[q + 1].start <= i) ++q;
      return win[q].blk0 + (uint64_t)(i - win[q].start) * 16;
    });
    __syncthreads();
    auto elt = [&](uint32_t x) {  // chunk-relative byte x
      const uint32_t q = (x + c.off0) / run;
      return *reinterpret_cast<const G*>(lds + (win[q].adj + (int32_t)x));
    };
    const uint64_t va = align_up16(F), vb = align_down16(F + c.n);
    const uint32_t nv = va < vb ? (uint32_t)((vb - va) >> 4) : 0u;
    const uint32_t xa = (uint32_t)(va - F);
    for (uint32_t j = threadIdx.x; j < nv; j += kBlock) {
      const uint32_t x = xa + j * 16;
      const uint32_t q = (x + c.off0) / run;
      u32x4 v;
      if (x + c.off0 + 16 <= (q + 1) * run) {  // inside one piece: 16 consecutive LDS bytes
        v = lds_vec(lds, (uint32_t)(win[q].adj + (int32_t)x));
      } else {
        G e[NE];
#pragma unroll
        for (uint32_t i = 0; i < NE; ++i) e[i] = elt(x + i * gb);
        v = pack_elts<G>(e);
      }
      stv<NTS>(gptr<u32x4>(va + (uint64_t)j * 16), v);
    }
    if (threadIdx.x < 2)
      fold_ends<G, NTS>(F, F + c.n, threadIdx.x, [&](uint64_t xb) { return elt((uint32_t)(xb - F)); });
  } else {
    const uint64_t fa = align_down16(F);
    const uint32_t nblk = (uint32_t)((align_up16(F + c.n) - fa) >> 4);
    stage_blocks(lds, nblk, [&](uint32_t i) -> uint64_t { return fa + (uint64_t)i * 16; });
    __syncthreads();
    flat_scatter<G, NTS>(c, run, (uint32_t)(F - fa), lds, src);
  }
  __syncthreads();  // the next chunk reuses the LDS
}

// NARROW: every item has a unit of at most fsdp::kFoldLdsMaxUnit bytes, so
// the unit-wise path only serves chunks whose windows do not fit the LDS;
// it then moves one unit per lane per iteration, which keeps this variant's
// registers (and so its occupancy) those of the LDS path.
template <bool NTS, bool NARROW>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(NARROW ? 8 : 1))) void fold_copy_kernel(const uint64_t* __restrict__ begin,
                                                           const fsdp::FoldSeg* __restrict__ folds, uint32_t n_fold,
                                                           uint64_t n_chunks) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFoldLds];
  for (uint64_t slot = blockIdx.x; slot < n_chunks; slot += gridDim.x) {
    const uint64_t c = xcd_chunk(slot, n_chunks);
    const uint32_t j = find_item(begin, n_fold, c);
    const fsdp::FoldSeg f = folds[j];
    if (f.rows_per_chunk == 0) {  // rows too long for one chunk: flat chunks
      if (f.unit >= 4)
        fold_flat<uint32_t, NTS>(f, c - begin[j], lds);
      else
        fold_flat<uint16_t, NTS>(f, c - begin[j], lds);
      continue;
    }
    const uint64_t r0 = (c - begin[j]) * f.rows_per_chunk;
    const uint64_t left = f.rows - r0;
    const uint32_t nr = (uint32_t)(left < f.rows_per_chunk ? left : f.rows_per_chunk);
    if (f.unit <= fsdp::kFoldLdsMaxUnit && fold_lds_bytes(f, r0, nr)) {
      if (f.unit >= 4)
        fold_lds<uint32_t, NTS>(f, r0, nr, lds);
      else
        fold_lds<uint16_t, NTS>(f, r0, nr, lds);
      continue;
    }
    if constexpr (NARROW) {
      if (f.unit == 4)
        fold_units<uint32_t, NTS, 1>(f, r0, nr);
      else
        fold_units<uint16_t, NTS, 1>(f, r0, nr);
      continue;
    }
    switch (f.unit) {
      case 16: fold_units<u32x4, NTS>(f, r0, nr); break;
      case 8: fold_units<uint64_t, NTS>(f, r0, nr); break;
      case 4: fold_units<uint32_t, NTS>(f, r0, nr); break;
      default: fold_units<uint16_t, NTS>(f, r0, nr); break;
    }
  }
}

// ---------------------------------------------------------------------------
// fold_reduce
// ---------------------------------------------------------------------------

// A unit of W bytes as 32-bit words (a 2-byte unit in the low half of one).
template <typename W>
struct UnitWords {
  static constexpr int N = sizeof(W) >= 4 ? (int)(sizeof(W) / 4) : 1;
  uint32_t w[N];
};
template <typename W>
__device__ __forceinline__ UnitWords<W> to_words(W v) {
  UnitWords<W> u;
  if constexpr (sizeof(W) == 16) {
    u.w[0] = v.x, u.w[1] = v.y, u.w[2] = v.z, u.w[3] = v.w;
  } else if constexpr (sizeof(W) == 8) {
    u.w[0] = (uint32_t)v, u.w[1] = (uint32_t)(v >> 32);
  } else {
    u.w[0] = (uint32_t)v;
  }
  return u;
}
template <typename W>
__device__ __forceinline__ W from_words(const UnitWords<W>& u) {
  if constexpr (sizeof(W) == 16) return W{u.w[0], u.w[1], u.w[2], u.w[3]};
  else if constexpr (sizeof(W) == 8) return (W)u.w[0] | ((W)u.w[1] << 32);
  else return (W)u.w[0];
}

// Element e of kind E of a unit, in float32 (exactly).
template <int E, typename W>
__device__ __forceinline__ float unit_elt(const UnitWords<W>& u, int e) {
  if constexpr (E == kF32) return __builtin_bit_cast(float, u.w[e]);
  else return elt_to_f32<E>((u.w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
}

// The reduction of K operand units of kind E: summed in ascending operand
// order from the first operand, in float32; AVG divides by nf; rounded once.
template <int E, typename W, int K>
__device__ __forceinline__ W reduce_unit(const W (&v)[K], int avg, float nf) {
  constexpr int NE = (int)sizeof(W) / (E == kF32 ? 4 : 2);
  UnitWords<W> in[K];
#pragma unroll
  for (int t = 0; t < K; ++t) in[t] = to_words<W>(v[t]);
  UnitWords<W> out;
#pragma unroll
  for (int i = 0; i < UnitWords<W>::N; ++i) out.w[i] = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    float acc = unit_elt<E, W>(in[0], e);
#pragma unroll
    for (int t = 1; t < K; ++t) acc = acc + unit_elt<E, W>(in[t], e);
    if (avg) acc = acc / nf;
    if constexpr (E == kF32) out.w[e] = __builtin_bit_cast(uint32_t, acc);
    else out.w[e >> 1] |= f32_to_elt<E>(acc) << ((e & 1) * 16);
  }
  return from_words<W>(out);
}

// Rows [r0, r0 + nr) of a fold-reduce item in W-sized units: unit q of the
// chunk is full-tensor row q / upf of the chunk, rank s = (q % upf) / upr
// and unit col = q % upr of that rank's piece.  Every operand is read at q
// units from its chunk start (whole lines, consecutive lanes on consecutive
// units); the result goes to rank s's rows.  Compile-time K: the operand
// and destination bases are wave-uniform registers, the destination of a
// unit a select among the K bases, and U units per lane per iteration keep
// all K*U loads in flight; over 2 ranks with units under 16 bytes the rest
// takes one or two more such iterations (a chunk of one 8 KiB row of 8-byte
// units is only that).  K = 0: any operand count, loads one at a time.
template <int E, int K, typename W, bool NTS>
__device__ __forceinline__ void fold_reduce_units(const fsdp::FoldRed& f, const uint64_t* __restrict__ ptr,
                                                  uint64_t r0, uint32_t nr, int avg) {
  const uint32_t S = f.nrank;
  const uint32_t upr = (uint32_t)(f.run_bytes / sizeof(W));
  const uint32_t upf = S * upr;
  const uint32_t n = nr * upf;
  const uint32_t run = (uint32_t)f.run_bytes;
  const uint64_t src_off = r0 * S * f.run_bytes;
  const uint64_t dst_off = r0 * f.run_bytes;
  const float nf = (float)S;
  auto split = [&](uint32_t q, uint32_t* s, uint32_t* dof) {
    const uint32_t row = q / upf;
    const uint32_t rem = q - row * upf;
    *s = rem / upr;
    *dof = row * run + (rem - *s * upr) * (uint32_t)sizeof(W);
  };
  auto st = [](uint64_t a, W v) {
    if (NTS)
      __builtin_nontemporal_store(v, gptr<W>(a));
    else
      *gptr<W>(a) = v;
  };
  uint32_t base = 0;
  if constexpr (K > 0) {
    constexpr int U0 = sizeof(W) >= 16 ? 8 : 16;
    constexpr int U = U0 / K > 1 ? U0 / K : 1;
    uint64_t sb[K], db[K];
#pragma unroll
    for (int t = 0; t < K; ++t) {
      sb[t] = ptr[f.src0 + t] + src_off;
      db[t] = ptr[f.dst0 + t] + dst_off;
    }
    // a mask, not a select: the compiler turns a chain of selects among the
    // array's elements into one lane-indexed load, which puts db in scratch
    auto dst_base = [&](uint32_t s) {
      uint64_t d = db[0];
#pragma unroll
      for (int t = 1; t < K; ++t) d ^= (db[t] ^ d) & (0ull - (uint64_t)(s == (uint32_t)t));
      return d;
    };
    for (; base + (uint32_t)kBlock * U <= n; base += (uint32_t)kBlock * U) {
      W v[U][K];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < K; ++t)
          v[u][t] = __builtin_nontemporal_load(gptr<W>(sb[t] + (uint64_t)(base + threadIdx.x + u * kBlock) * sizeof(W)));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t s, dof;
        split(base + threadIdx.x + u * kBlock, &s, &dof);
        st(dst_base(s) + dof, reduce_unit<E, W, K>(v[u], avg, nf));
      }
    }
    if constexpr (K == 2 && sizeof(W) < 16) {
      // the rest of a 2-rank group's chunk (never staged through LDS with
      // such units, so this path carries every chunk): iterations of UT
      // units per lane, all loads of each first; lanes past the end load
      // the last unit again (no branch around the loads, which made the
      // compiler wait for each load before the next) and store nothing.
      // One iteration for fp32, two for 16-bit elements (which keeps them
      // out of scratch).
      constexpr int UT = E != kF32 ? U / 2 : U;
      for (; base < n; base += (uint32_t)kBlock * UT) {
        W v[UT][K];
#pragma unroll
        for (int u = 0; u < UT; ++u) {
          const uint32_t q = base + threadIdx.x + u * kBlock;
          const uint64_t o = (uint64_t)(q < n ? q : n - 1) * sizeof(W);
#pragma unroll
          for (int t = 0; t < K; ++t) v[u][t] = __builtin_nontemporal_load(gptr<W>(sb[t] + o));
        }
#pragma unroll
        for (int u = 0; u < UT; ++u) {
          const uint32_t q = base + threadIdx.x + u * kBlock;
          if (q < n) {
            uint32_t s, dof;
            split(q, &s, &dof);
            st(dst_base(s) + dof, reduce_unit<E, W, K>(v[u], avg, nf));
          }
        }
      }
    } else {  // groups of 4 and 8 ranks stage their chunks through LDS where they can
      for (uint32_t q = base + threadIdx.x; q < n; q += kBlock) {
        W v[K];
#pragma unroll
        for (int t = 0; t < K; ++t) v[t] = __builtin_nontemporal_load(gptr<W>(sb[t] + (uint64_t)q * sizeof(W)));
        uint32_t s, dof;
        split(q, &s, &dof);
        st(dst_base(s) + dof, reduce_unit<E, W, K>(v, avg, nf));
      }
    }
  } else {
    constexpr int NE = (int)sizeof(W) / (E == kF32 ? 4 : 2);
    for (uint32_t q = threadIdx.x; q < n; q += kBlock) {
      const uint64_t so = src_off + (uint64_t)q * sizeof(W);
      float acc[NE];
      {
        const UnitWords<W> u = to_words<W>(__builtin_nontemporal_load(gptr<W>(ptr[f.src0] + so)));
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = unit_elt<E, W>(u, e);
      }
      for (uint32_t t = 1; t < S; ++t) {
        const UnitWords<W> u = to_words<W>(__builtin_nontemporal_load(gptr<W>(ptr[f.src0 + t] + so)));
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = acc[e] + unit_elt<E, W>(u, e);
      }
      UnitWords<W> out;
#pragma unroll
      for (int i = 0; i < UnitWords<W>::N; ++i) out.w[i] = 0;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float a = avg ? acc[e] / nf : acc[e];
        if constexpr (E == kF32) out.w[e] = __builtin_bit_cast(uint32_t, a);
        else out.w[e >> 1] |= f32_to_elt<E>(a) << ((e & 1) * 16);
      }
      uint32_t s, dof;
      split(q, &s, &dof);
      st(ptr[f.dst0 + s] + dst_off + dof, from_words<W>(out));
    }
  }
}

// LDS staging of a fold-reduce chunk with 2- or 4-byte units, or wider ones
// in groups of at least 4 ranks, when every operand has the same address
// modulo 16 (measured on MI355X against the unit path: wider units 4-14 %
// faster over 4 and 8 ranks, 4-17 % slower over 2 and 3): the operands' aligned 16-byte
// blocks over the chunk's full rows are reduced block by block (the reduce
// kernel's arithmetic and operand order; the bytes of the edge blocks
// outside the chunk are reduced too but never read back) into LDS, then
// every rank's rows are written as in the scatter of fold_lds.
__device__ __forceinline__ bool fold_reduce_lds_ok(const fsdp::FoldRed& f, const uint64_t* __restrict__ ptr,
                                                   uint64_t r0, uint32_t nr) {
  if (f.unit > fsdp::kFoldLdsMaxUnit && f.nrank < 4) return false;
  const uint64_t a = ptr[f.src0];
  for (uint32_t t = 1; t < f.nrank; ++t)
    if ((ptr[f.src0 + t] ^ a) & 15u) return false;
  const uint64_t F0 = a + r0 * f.nrank * f.run_bytes;
  return align_up16(F0 + (uint64_t)nr * f.nrank * f.run_bytes) - align_down16(F0) <= kFoldLds;
}

template <int E, int K, typename G, bool NTS>
__device__ __forceinline__ void fold_reduce_lds(const fsdp::FoldRed& f, const uint64_t* __restrict__ ptr,
                                                uint64_t r0, uint32_t nr, int avg, uint8_t* lds) {
  const uint32_t S = f.nrank, run = (uint32_t)f.run_bytes;
  const uint32_t FR = S * run;
  const uint64_t off = r0 * FR;  // the chunk's first byte in every operand
  const uint64_t F0 = ptr[f.src0] + off;
  const uint64_t fa = align_down16(F0);
  const uint32_t delta = (uint32_t)(F0 - fa);
  const uint32_t nblk = (uint32_t)((align_up16(F0 + (uint64_t)nr * FR) - fa) >> 4);
  const float nf = (float)S;
  if constexpr (K > 0) {
    uint64_t sb[K];
#pragma unroll
    for (int t = 0; t < K; ++t) sb[t] = align_down16(ptr[f.src0 + t] + off);
    reduce_blocks<E, K>(lds, nblk, sb, avg, nf);
  } else {
    for (uint32_t i = threadIdx.x; i < nblk; i += kBlock) {
      Acc<E> acc = widen<E>(ldv(gptr<u32x4>(align_down16(ptr[f.src0] + off) + (uint64_t)i * 16)));
      for (uint32_t t = 1; t < S; ++t)
        accumulate<E>(acc, ldv(gptr<u32x4>(align_down16(ptr[f.src0 + t] + off) + (uint64_t)i * 16)));
      *reinterpret_cast<u32x4*>(lds + i * 16) = narrow<E>(acc, avg, nf);
    }
  }
  __syncthreads();
  scatter_rows<G, NTS>(lds, delta, nblk, S, run, nr, [&](uint32_t s) { return ptr[f.dst0 + s] + r0 * run; });
  __syncthreads();  // the next chunk reuses the LDS
}

// Flat chunks of a fold-reduce item (rows_per_chunk == 0, as in fold_flat):
// the operands' aligned blocks over full-tensor bytes [X0, X1) (every
// operand at the same address modulo 16, which the planner checks) are
// reduced block by block into LDS (the reduce kernel's arithmetic and
// order), then every piece's part is written as in fold_flat's scatter.
template <int E, int K, typename G, bool NTS>
__device__ __forceinline__ void fold_reduce_flat(const fsdp::FoldRed& f, const uint64_t* __restrict__ ptr,
                                                 uint64_t k, int avg, uint8_t* lds) {
  const uint32_t S = f.nrank, run = (uint32_t)f.run_bytes;
  const FlatChunk c = flat_chunk(k, f.rows * S * run, (uint32_t)f.reserved[0], run);
  const uint64_t F0 = ptr[f.src0] + c.X0;
  const uint64_t fa = align_down16(F0);
  const uint32_t nblk = (uint32_t)((align_up16(F0 + c.n) - fa) >> 4);
  const float nf = (float)S;
  if constexpr (K > 0) {
    uint64_t sb[K];
#pragma unroll
    for (int t = 0; t < K; ++t) sb[t] = align_down16(ptr[f.src0 + t] + c.X0);
    reduce_blocks<E, K>(lds, nblk, sb, avg, nf);
  } else {
    for (uint32_t i = threadIdx.x; i < nblk; i += kBlock) {
      Acc<E> acc = widen<E>(ldv(gptr<u32x4>(align_down16(ptr[f.src0] + c.X0) + (uint64_t)i * 16)));
      for (uint32_t t = 1; t < S; ++t)
        accumulate<E>(acc, ldv(gptr<u32x4>(align_down16(ptr[f.src0 + t] + c.X0) + (uint64_t)i * 16)));
      *reinterpret_cast<u32x4*>(lds + i * 16) = narrow<E>(acc, avg, nf);
    }
  }
  __syncthreads();
  flat_scatter<G, NTS>(c, run, (uint32_t)(F0 - fa), lds, [&](uint64_t p, uint32_t a) {
    const uint64_t r = p / S;
    const uint32_t s = (uint32_t)(p - r * S);
    return ptr[f.dst0 + s] + r * run + (c.X0 + a - p * run);
  });
  __syncthreads();  // the next chunk reuses the LDS
}

// NARROW: every item has a unit of at most fsdp::kFoldLdsMaxUnit bytes; a
// chunk that cannot be staged (operands at different offsets modulo 16, or
// too large for the LDS) takes the runtime-count unit loop, which keeps
// this variant's registers those of the LDS path.
template <int E, int K, bool NTS, bool NARROW>
__global__ __launch_bounds__(kBlock, 4) void fold_reduce_kernel(const uint64_t* __restrict__ begin,
                                                             const fsdp::FoldRed* __restrict__ items,
                                                             const uint64_t* __restrict__ ptr, uint32_t n_item,
                                                             uint64_t n_chunks, int avg) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFoldLds];
  for (uint64_t slot = blockIdx.x; slot < n_chunks; slot += gridDim.x) {
    const uint64_t c = xcd_chunk(slot, n_chunks);
    const uint32_t j = find_item(begin, n_item, c);
    const fsdp::FoldRed f = items[j];
    if (f.rows_per_chunk == 0) {  // rows too long for one chunk: flat chunks
      if (f.unit >= 4)
        fold_reduce_flat<E, K, uint32_t, NTS>(f, ptr, c - begin[j], avg, lds);
      else if constexpr (E != kF32)
        fold_reduce_flat<E, K, uint16_t, NTS>(f, ptr, c - begin[j], avg, lds);
      continue;
    }
    const uint64_t r0 = (c - begin[j]) * f.rows_per_chunk;
    const uint64_t left = f.rows - r0;
    const uint32_t nr = (uint32_t)(left < f.rows_per_chunk ? left : f.rows_per_chunk);
    if (fold_reduce_lds_ok(f, ptr, r0, nr)) {
      if (f.unit >= 4)
        fold_reduce_lds<E, K, uint32_t, NTS>(f, ptr, r0, nr, avg, lds);
      else if constexpr (E != kF32)
        fold_reduce_lds<E, K, uint16_t, NTS>(f, ptr, r0, nr, avg, lds);
      continue;
    }
    if constexpr (NARROW) {
      if (f.unit == 4)
        fold_reduce_units<E, 0, uint32_t, NTS>(f, ptr, r0, nr, avg);
      else if constexpr (E != kF32)
        fold_reduce_units<E, 0, uint16_t, NTS>(f, ptr, r0, nr, avg);
      continue;
    }
    switch (f.unit) {
      case 16: fold_reduce_units<E, K, u32x4, NTS>(f, ptr, r0, nr, avg); break;
      case 8: fold_reduce_units<E, K, uint64_t, NTS>(f, ptr, r0, nr, avg); break;
      case 4: fold_reduce_units<E, K, uint32_t, NTS>(f, ptr, r0, nr, avg); break;
      default:
        if constexpr (E != kF32) fold_reduce_units<E, K, uint16_t, NTS>(f, ptr, r0, nr, avg);
        break;
    }
  }
}

// One workgroup per chunk up to max_grid; a capped grid is a multiple of 8
// so that every grid-stride step keeps each workgroup on its XCD.
inline uint32_t grid_for(uint64_t n_chunks, uint32_t max_grid) {
  if (n_chunks < (uint64_t)max_grid) return (uint32_t)n_chunks;
  return max_grid >= 8 ? max_grid & ~7u : max_grid;
}

}  // namespace

namespace {
// One launch: grid, block, stream and, when the caller times the kernel,
// the events its dispatch records at the kernel's start and end.
struct Launch {
  dim3 grid, block;
  hipStream_t stream;
  hipEvent_t start, stop;
  template <typename... KArgs, typename... Args>
  void operator()(void (*kernel)(KArgs...), Args... args) const {
    if (start || stop)
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
    else
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  }
};
}  // namespace

int fsdp_launch_seg_copy(int elem_bytes, const void* dev_table, uint32_t n_seg, uint64_t n_chunks,
                         uint32_t chunk_shift, uint32_t max_grid, int stream_stores, void* stream,
                         void* start_event, void* stop_event) {
  if (n_chunks == 0 || n_chunks >= (uint64_t(1) << 31)) return (int)hipErrorInvalidValue;
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::CopySeg* segs = reinterpret_cast<const fsdp::CopySeg*>(begin + n_seg);
  const uint32_t* item_of = reinterpret_cast<const uint32_t*>(segs + n_seg);
  const uint32_t nc = (uint32_t)n_chunks;
  const uint32_t grid = grid_for(n_chunks, max_grid);
  const Launch go{dim3(grid), dim3(kCopyBlock), static_cast<hipStream_t>(stream),
                  static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  if (elem_bytes == 4) {
    if (stream_stores)
      go(seg_copy_kernel<uint32_t, true>, begin, segs, item_of, nc, chunk_shift, grid);
    else
      go(seg_copy_kernel<uint32_t, false>, begin, segs, item_of, nc, chunk_shift, grid);
  } else {
    if (stream_stores)
      go(seg_copy_kernel<uint16_t, true>, begin, segs, item_of, nc, chunk_shift, grid);
    else
      go(seg_copy_kernel<uint16_t, false>, begin, segs, item_of, nc, chunk_shift, grid);
  }
  return (int)hipGetLastError();
}

namespace {
template <int E, bool NTS>
void launch_reduce_k(const Launch& go, uint32_t n_src, const uint64_t* begin, const fsdp::RedJob* jobs,
                     const uint64_t* ptr, uint32_t n_job, uint64_t n_chunks, uint32_t chunk_shift, int avg) {
  switch (n_src) {
    case 1: go(reduce_kernel<E, 1, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case 2: go(reduce_kernel<E, 2, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case 3: go(reduce_kernel<E, 3, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case 4: go(reduce_kernel<E, 4, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case 6: go(reduce_kernel<E, 6, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case 8: go(reduce_kernel<E, 8, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    default: go(reduce_kernel<E, 0, NTS>, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
  }
}

template <int E>
void launch_reduce_e(const Launch& go, int stream_stores, uint32_t n_src, const uint64_t* begin,
                     const fsdp::RedJob* jobs, const uint64_t* ptr, uint32_t n_job, uint64_t n_chunks,
                     uint32_t chunk_shift, int avg) {
  if (stream_stores)
    launch_reduce_k<E, true>(go, n_src, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg);
  else
    launch_reduce_k<E, false>(go, n_src, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg);
}
}  // namespace

int fsdp_launch_reduce(int elt, const void* dev_table, uint32_t n_job, uint32_t n_src, uint64_t n_chunks,
                       uint32_t chunk_shift, uint32_t max_grid, int avg, int stream_stores, void* stream,
                       void* start_event, void* stop_event) {
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::RedJob* jobs = reinterpret_cast<const fsdp::RedJob*>(begin + n_job);
  // the pointer array follows the jobs (64-byte records, so it is 8-byte aligned)
  const uint64_t* ptr = reinterpret_cast<const uint64_t*>(jobs + n_job);
  const Launch go{dim3(grid_for(n_chunks, max_grid)), dim3(kBlock), static_cast<hipStream_t>(stream),
                  static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  switch (elt) {
    case kF32: launch_reduce_e<kF32>(go, stream_stores, n_src, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case kBF16: launch_reduce_e<kBF16>(go, stream_stores, n_src, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    case kF16: launch_reduce_e<kF16>(go, stream_stores, n_src, begin, jobs, ptr, n_job, n_chunks, chunk_shift, avg); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int fsdp_launch_fold(const void* dev_table, uint32_t n_fold, uint64_t n_chunks, uint32_t max_grid, int narrow,
                     int stream_stores, void* stream, void* start_event, void* stop_event) {
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::FoldSeg* folds = reinterpret_cast<const fsdp::FoldSeg*>(begin + n_fold);
  const Launch go{dim3(grid_for(n_chunks, max_grid)), dim3(kBlock), static_cast<hipStream_t>(stream),
                  static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  if (narrow) {
    if (stream_stores)
      go(fold_copy_kernel<true, true>, begin, folds, n_fold, n_chunks);
    else
      go(fold_copy_kernel<false, true>, begin, folds, n_fold, n_chunks);
  } else {
    if (stream_stores)
      go(fold_copy_kernel<true, false>, begin, folds, n_fold, n_chunks);
    else
      go(fold_copy_kernel<false, false>, begin, folds, n_fold, n_chunks);
  }
  return (int)hipGetLastError();
}

namespace {
template <int E, bool NTS, bool NARROW>
void launch_fold_reduce_k(const Launch& go, uint32_t n_src, const uint64_t* begin, const fsdp::FoldRed* items,
                          const uint64_t* ptr, uint32_t n_item, uint64_t n_chunks, int avg) {
  switch (n_src) {
    case 2: go(fold_reduce_kernel<E, 2, NTS, NARROW>, begin, items, ptr, n_item, n_chunks, avg); break;
    case 4: go(fold_reduce_kernel<E, 4, NTS, NARROW>, begin, items, ptr, n_item, n_chunks, avg); break;
    case 8: go(fold_reduce_kernel<E, 8, NTS, NARROW>, begin, items, ptr, n_item, n_chunks, avg); break;
    default: go(fold_reduce_kernel<E, 0, NTS, NARROW>, begin, items, ptr, n_item, n_chunks, avg); break;
  }
}

template <int E>
void launch_fold_reduce_e(const Launch& go, int narrow, int stream_stores, uint32_t n_src, const uint64_t* begin,
                          const fsdp::FoldRed* items, const uint64_t* ptr, uint32_t n_item, uint64_t n_chunks,
                          int avg) {
  if (narrow) {
    if (stream_stores)
      launch_fold_reduce_k<E, true, true>(go, n_src, begin, items, ptr, n_item, n_chunks, avg);
    else
      launch_fold_reduce_k<E, false, true>(go, n_src, begin, items, ptr, n_item, n_chunks, avg);
  } else {
    if (stream_stores)
      launch_fold_reduce_k<E, true, false>(go, n_src, begin, items, ptr, n_item, n_chunks, avg);
    else
      launch_fold_reduce_k<E, false, false>(go, n_src, begin, items, ptr, n_item, n_chunks, avg);
  }
}
}  // namespace

int fsdp_launch_fold_reduce(int elt, const void* dev_table, uint32_t n_item, uint32_t n_src, uint64_t n_chunks,
                            uint32_t max_grid, int narrow, int avg, int stream_stores, void* stream,
                            void* start_event, void* stop_event) {
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::FoldRed* items = reinterpret_cast<const fsdp::FoldRed*>(begin + n_item);
  const uint64_t* ptr = reinterpret_cast<const uint64_t*>(items + n_item);
  const Launch go{dim3(grid_for(n_chunks, max_grid)), dim3(kBlock), static_cast<hipStream_t>(stream),
                  static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  switch (elt) {
    case kF32: launch_fold_reduce_e<kF32>(go, narrow, stream_stores, n_src, begin, items, ptr, n_item, n_chunks, avg); break;
    case kBF16: launch_fold_reduce_e<kBF16>(go, narrow, stream_stores, n_src, begin, items, ptr, n_item, n_chunks, avg); break;
    case kF16: launch_fold_reduce_e<kF16>(go, narrow, stream_stores, n_src, begin, items, ptr, n_item, n_chunks, avg); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch: the descriptor tables of the entry point that allocates nothing
// (fsdp_rs_copy_reduce_noalloc).  One array per GPU, held until the process
// ends; every such call on a GPU rewrites it, so calls that overlap in time
// on one GPU (different streams) race on it.
// ---------------------------------------------------------------------------

namespace {

static __device__ __align__(256) uint8_t scratch[fsdp::kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Table bytes carried by one writer launch, in its kernel arguments (which
// the launch copies, so the host buffer may go away when the call returns).
constexpr uint32_t kTablePiece = 3072;

struct TablePiece {
  uint64_t offset;  // into the scratch array
  uint32_t bytes;   // a multiple of 16, at most kTablePiece
  uint32_t reserved;
  u32x4 data[kTablePiece / 16];
};

// Writes one piece of a descriptor table into the scratch array: 16-byte
// vector stores, one per lane.
__global__ __launch_bounds__(kBlock) void table_write_kernel(uint8_t* __restrict__ dst, TablePiece piece) {
  for (uint32_t i = threadIdx.x; i * 16u < piece.bytes; i += kBlock)
    *reinterpret_cast<u32x4*>(dst + piece.offset + 16u * i) = piece.data[i];
}

}  // namespace

int fsdp_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxScratchDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the host-side name of the array is not a device address: look up this
    // device's copy once, with the device current, and use that address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return (int)hipSuccess;
}

int fsdp_scratch_write(void* base, const void* host, size_t bytes, size_t offset, void* stream) {
  const uint8_t* src = static_cast<const uint8_t*>(host);
  for (size_t done = 0; done < bytes; done += kTablePiece) {
    TablePiece piece;
    const size_t n = bytes - done < kTablePiece ? bytes - done : kTablePiece;
    std::memset(&piece, 0, sizeof piece);
    std::memcpy(piece.data, src + done, n);
    piece.offset = offset + done;
    piece.bytes = (uint32_t)((n + 15) & ~size_t(15));
    hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t*>(base), piece);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}
