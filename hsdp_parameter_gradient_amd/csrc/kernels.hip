// gfx950 kernels of the FSDP/HSDP flat-buffer hot path.
//
// Two kernels serve the five entry points:
//   seg_copy  — segmented copy with zero fill: AG copy-in (pack shards into
//               padded rank slices), AG copy-out (unpack into the full
//               parameters) and RS copy-in (chunk gradients into the padded
//               rank-major RS input).  Bits are moved, never converted.
//   reduce    — fixed-order fp32 reduction of K operands into M
//               destinations: the RS of a shard group (K = S, M = 1) and the
//               in-place fused AR of a replicate group (K = M = D).
//
// Both are HBM-bound streaming kernels (no data reuse, no dense
// contraction): one workgroup of 256 lanes handles one chunk of destination
// bytes at a time, with 128-bit loads and stores on 16-byte-aligned
// destination addresses.  A source whose address differs from the
// destination's modulo 16 is read as the two aligned 16-byte blocks around
// each destination vector and realigned in registers with v_alignbyte
// (each block read holds at least one byte the copy needs, so no read
// leaves the source's own pages).  The few 16-byte vectors that straddle a
// segment edge or the data/padding edge are written element by element, so
// that no byte outside the segment is touched.
//
// Arithmetic: the reduce kernel adds operands one at a time in ascending
// rank order, the accumulator starting from the first operand, in IEEE
// fp32 with denormals preserved; AVG divides by the operand count (an
// exact multiply for a power of two, a correctly rounded divide otherwise).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

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

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ uint64_t align_down16(uint64_t a) { return a & ~uint64_t(15); }
__device__ __forceinline__ uint64_t align_up16(uint64_t a) { return (a + 15) & ~uint64_t(15); }

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

// 16 source bytes starting r bytes into aligned block s[j] (0 <= r < 16).
__device__ __forceinline__ u32x4 load_shifted(const gvec* __restrict__ s, uint64_t j,
                                              uint32_t r) {
  if (r == 0) return s[j];
  const u32x4 a = s[j];
  const u32x4 c = s[j + 1];
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

template <int Q>
__device__ __forceinline__ void copy_funnel(gvec* __restrict__ d, const gvec* __restrict__ s,
                                            uint64_t nv, uint32_t b) {
  for (uint64_t j0 = threadIdx.x; j0 < nv; j0 += (uint64_t)kBlock * kUnroll) {
    u32x4 a[kUnroll], c[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t j = j0 + (uint64_t)u * kBlock;
      if (j < nv) {
        a[u] = s[j];
        c[u] = s[j + 1];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t j = j0 + (uint64_t)u * kBlock;
      if (j < nv) d[j] = funnel<Q>(a[u], c[u], b);
    }
  }
}

// nv destination vectors from dst (16-aligned), source bytes from src.
__device__ __forceinline__ void copy_vectors(uint64_t dst, uint64_t src, uint64_t nv) {
  gvec* __restrict__ d = gptr<u32x4>(dst);
  const uint32_t r = (uint32_t)(src & 15u);
  if (r == 0) {
    const gvec* __restrict__ s = gptr<u32x4>(src);
    for (uint64_t j0 = threadIdx.x; j0 < nv; j0 += (uint64_t)kBlock * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kBlock;
        if (j < nv) v[u] = s[j];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint64_t j = j0 + (uint64_t)u * kBlock;
        if (j < nv) d[j] = v[u];
      }
    }
    return;
  }
  const gvec* __restrict__ s = gptr<u32x4>(src - r);
  const uint32_t b = r & 3u;
  switch (r >> 2) {
    case 0: copy_funnel<0>(d, s, nv, b); break;
    case 1: copy_funnel<1>(d, s, nv, b); break;
    case 2: copy_funnel<2>(d, s, nv, b); break;
    default: copy_funnel<3>(d, s, nv, b); break;
  }
}

__device__ __forceinline__ void zero_vectors(uint64_t dst, uint64_t nv) {
  gvec* __restrict__ d = gptr<u32x4>(dst);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (uint64_t j = threadIdx.x; j < nv; j += kBlock) d[j] = z;
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

template <typename T>
__global__ __launch_bounds__(kBlock) void seg_copy_kernel(const uint64_t* __restrict__ begin,
                                                          const fsdp::CopySeg* __restrict__ segs,
                                                          uint32_t n_seg, uint64_t n_chunks,
                                                          uint32_t shift) {
  const uint64_t CH = uint64_t(1) << shift;
  for (uint64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const uint32_t j = find_item(begin, n_seg, c);
    const fsdp::CopySeg sg = segs[j];
    const uint64_t k = c - begin[j];
    const uint64_t base = (sg.dst >> shift) << shift;
    const uint64_t seg_end = sg.dst + sg.total_bytes;
    const uint64_t cend = sg.dst + sg.copy_bytes;
    const uint64_t w0 = base + k * CH;
    const uint64_t lo = w0 > sg.dst ? w0 : sg.dst;
    const uint64_t hi = (w0 + CH) < seg_end ? (w0 + CH) : seg_end;

    // whole vectors of data
    const uint64_t ca = align_up16(lo);
    const uint64_t cb = align_down16(hi < cend ? hi : cend);
    if (ca < cb) copy_vectors(ca, sg.src + (ca - sg.dst), (cb - ca) >> 4);
    // whole vectors of padding
    const uint64_t za = align_up16(lo > cend ? lo : cend);
    const uint64_t zb = align_down16(hi);
    if (za < zb) zero_vectors(za, (zb - za) >> 4);
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
}

// ---------------------------------------------------------------------------
// reduce
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4 as_f4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ u32x4 as_u4(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float scale_avg(float acc, float n, float inv, bool pow2) {
  return pow2 ? acc * inv : acc / n;
}

__global__ __launch_bounds__(kBlock) void reduce_kernel(const uint64_t* __restrict__ begin,
                                                        const fsdp::RedJob* __restrict__ jobs,
                                                        const uint64_t* __restrict__ ptr,
                                                        uint32_t n_job, uint64_t n_chunks,
                                                        uint32_t shift, int avg) {
  const uint64_t CH = uint64_t(1) << shift;
  for (uint64_t c = blockIdx.x; c < n_chunks; c += gridDim.x) {
    const uint32_t j = find_item(begin, n_job, c);
    const fsdp::RedJob jb = jobs[j];
    const uint64_t k = c - begin[j];
    const uint64_t d0 = ptr[jb.dst0];
    const uint64_t base = (d0 >> shift) << shift;
    const uint64_t w0 = base + k * CH;
    const uint64_t lo = w0 > d0 ? w0 : d0;
    const uint64_t end = d0 + jb.nbytes;
    const uint64_t hi = (w0 + CH) < end ? (w0 + CH) : end;
    const float nf = (float)jb.nsrc;
    const float inv = 1.0f / nf;
    const bool pow2 = (jb.nsrc & (jb.nsrc - 1u)) == 0u;

    // whole vectors: offsets [va, vb) relative to d0
    const uint64_t va = align_up16(lo) - d0;
    const uint64_t vb = align_down16(hi) - d0;
    if (va < vb) {
      const uint64_t nv = (vb - va) >> 4;
      for (uint64_t j0 = threadIdx.x; j0 < nv; j0 += (uint64_t)kBlock * kUnroll) {
        f32x4 acc[kUnroll];
        for (uint32_t t = 0; t < jb.nsrc; ++t) {
          const uint64_t sa = ptr[jb.src0 + t] + va;
          const uint32_t r = (uint32_t)(sa & 15u);
          const gvec* __restrict__ s = gptr<u32x4>(sa - r);
          u32x4 v[kUnroll] = {};
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const uint64_t q = j0 + (uint64_t)u * kBlock;
            if (q < nv) v[u] = load_shifted(s, q, r);
          }
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) acc[u] = (t == 0) ? as_f4(v[u]) : acc[u] + as_f4(v[u]);
        }
        if (avg) {
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            acc[u].x = scale_avg(acc[u].x, nf, inv, pow2);
            acc[u].y = scale_avg(acc[u].y, nf, inv, pow2);
            acc[u].z = scale_avg(acc[u].z, nf, inv, pow2);
            acc[u].w = scale_avg(acc[u].w, nf, inv, pow2);
          }
        }
        for (uint32_t m = 0; m < jb.ndst; ++m) {
          gvec* __restrict__ d = gptr<u32x4>(ptr[jb.dst0 + m] + va);
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const uint64_t q = j0 + (uint64_t)u * kBlock;
            if (q < nv) d[q] = as_u4(acc[u]);
          }
        }
      }
    }
    // elements of the vectors cut by the window start and the job end
    const uint64_t e0 = lo - d0;
    const uint64_t e_head = (align_up16(lo) < hi ? align_up16(lo) : hi) - d0;
    const uint64_t e_tail = (align_down16(hi) > lo ? align_down16(hi) : lo) - d0;
    const uint64_t e1 = hi - d0;
    // head elements [e0, e_head), tail elements [max(e_tail, e_head), e1)
    const uint64_t n_head = (e_head - e0) >> 2;
    const uint64_t t0 = e_tail > e_head ? e_tail : e_head;
    const uint64_t n_tail = (e1 - t0) >> 2;
    if (threadIdx.x < n_head + n_tail) {
      const uint64_t x = threadIdx.x < n_head ? e0 + 4u * threadIdx.x : t0 + 4u * (threadIdx.x - n_head);
      float acc = 0.0f;
      for (uint32_t t = 0; t < jb.nsrc; ++t) {
        const float v = *gptr<float>(ptr[jb.src0 + t] + x);
        acc = (t == 0) ? v : acc + v;
      }
      if (avg) acc = scale_avg(acc, nf, inv, pow2);
      for (uint32_t m = 0; m < jb.ndst; ++m) *gptr<float>(ptr[jb.dst0 + m] + x) = acc;
    }
  }
}

inline uint32_t grid_for(uint64_t n_chunks, uint32_t max_grid) {
  return (uint32_t)(n_chunks < (uint64_t)max_grid ? n_chunks : (uint64_t)max_grid);
}

}  // namespace

int fsdp_launch_seg_copy(int elem_bytes, const void* dev_table, uint32_t n_seg, uint64_t n_chunks,
                         uint32_t chunk_shift, uint32_t max_grid, void* stream) {
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::CopySeg* segs = reinterpret_cast<const fsdp::CopySeg*>(begin + n_seg);
  const dim3 grid(grid_for(n_chunks, max_grid)), block(kBlock);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(seg_copy_kernel<uint32_t>, grid, block, 0, st, begin, segs, n_seg, n_chunks,
                       chunk_shift);
  else
    hipLaunchKernelGGL(seg_copy_kernel<uint16_t>, grid, block, 0, st, begin, segs, n_seg, n_chunks,
                       chunk_shift);
  return (int)hipGetLastError();
}

int fsdp_launch_reduce(const void* dev_table, uint32_t n_job, uint64_t n_chunks,
                       uint32_t chunk_shift, uint32_t max_grid, int avg, void* stream) {
  const uint64_t* begin = static_cast<const uint64_t*>(dev_table);
  const fsdp::RedJob* jobs = reinterpret_cast<const fsdp::RedJob*>(begin + n_job);
  // the pointer array follows the jobs, 8-byte aligned (24 * n_job is a multiple of 8)
  const uint64_t* ptr = reinterpret_cast<const uint64_t*>(jobs + n_job);
  const dim3 grid(grid_for(n_chunks, max_grid)), block(kBlock);
  hipLaunchKernelGGL(reduce_kernel, grid, block, 0, static_cast<hipStream_t>(stream), begin, jobs,
                     ptr, n_job, n_chunks, chunk_shift, avg);
  return (int)hipGetLastError();
}
