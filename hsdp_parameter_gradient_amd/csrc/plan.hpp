// Descriptor tables shared by the host planner and the gfx950 kernels.
//
// A table is one contiguous blob in device memory, uploaded once per
// distinct content and cached by the planner:
//
//   copy table    uint64 chunk_begin[n]  |  CopySeg seg[n]
//   reduce table  uint64 chunk_begin[n]  |  RedJob job[n]  |  uint64 ptr[m]
//
// Work is cut into chunks of (1 << chunk_shift) destination bytes.  Chunk k
// of an item covers the window [base + k*CH, base + (k+1)*CH) clipped to
// the item, where base is the item's first destination byte rounded down
// to a multiple of CH, so that chunk edges inside an item are CH-aligned
// (whole cache lines, never shared between workgroups).  chunk_begin[j] is
// the global index of item j's first chunk; items are never empty.
#pragma once

#include <stdint.h>

namespace fsdp {

// One destination segment of a copy: copy_bytes from src, then
// (total_bytes - copy_bytes) zero bytes.  copy_bytes may be 0.
struct CopySeg {
  uint64_t src;
  uint64_t dst;
  uint64_t copy_bytes;
  uint64_t total_bytes;
};

// One reduction job over nbytes of destination: the first data_bytes are
// the reduction of the operands ptr[src0 .. src0+nsrc) (read at the same
// offsets), the rest is zero filled; every destination ptr[dst0 ..
// dst0+ndst) gets the same result.  All destinations share their address
// modulo 16.  AVG divides by nsrc.
struct RedJob {
  uint64_t nbytes;
  uint64_t data_bytes;
  uint32_t src0;
  uint32_t nsrc;
  uint32_t dst0;
  uint32_t ndst;
};

static_assert(sizeof(CopySeg) == 32, "CopySeg layout");
static_assert(sizeof(RedJob) == 32, "RedJob layout");

// Number of chunks of an item [dst, dst + nbytes), nbytes > 0.
inline uint64_t chunk_count(uint64_t dst, uint64_t nbytes, uint32_t shift) {
  return ((dst + nbytes - 1) >> shift) - (dst >> shift) + 1;
}

}  // namespace fsdp

// Launchers (defined in kernels.hip).  Return hipSuccess or the launch error.
extern "C++" {
// stream_stores: nontemporal stores for the outputs (see the store policy in
// fsdp_flat.cpp).
int fsdp_launch_seg_copy(int elem_bytes, const void* dev_table, uint32_t n_seg,
                         uint64_t n_chunks, uint32_t chunk_shift, uint32_t max_grid,
                         int stream_stores, void* stream);
// Every job of one launch has the same operand count n_src; elem_bytes is 4
// (fp32) or 2 (bf16).
int fsdp_launch_reduce(int elem_bytes, const void* dev_table, uint32_t n_job, uint32_t n_src, uint64_t n_chunks,
                       uint32_t chunk_shift, uint32_t max_grid, int avg, int stream_stores,
                       void* stream);
}
