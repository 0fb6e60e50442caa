// Descriptor tables shared by the host planner and the gfx950 kernels.
//
// A table is one contiguous blob in device memory, uploaded once per
// distinct content and cached by the planner:
//
//   copy table    uint64 chunk_begin[n]  |  CopySeg seg[n]  |  uint32 item_of[chunks]
//   reduce table  uint64 chunk_begin[n]  |  RedJob job[n]  |  uint64 ptr[m]
//   fold table    uint64 chunk_begin[n]  |  FoldSeg fold[n]
//   fold-reduce   uint64 chunk_begin[n]  |  FoldRed item[n]  |  uint64 ptr[m]
//
// Work is cut into chunks of (1 << chunk_shift) destination bytes.  Chunk k
// of a one-row item covers the window [base + k*CH, base + (k+1)*CH)
// clipped to the item, where base is the item's first destination byte
// rounded down to a multiple of CH, so that chunk edges inside an item are
// CH-aligned (whole cache lines, never shared between workgroups).  An item
// of several rows (a strided block: the chunk of a parameter sharded on a
// non-zero dim) is cut into whole rows instead, rows_per_chunk rows (at most
// CH bytes) per chunk.  chunk_begin[j] is the global index of item j's first
// chunk; items are never empty.  The copy table also maps every chunk to
// its item (item_of[c] = j with chunk_begin[j] <= c < chunk_begin[j+1]).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fsdp {

// One destination segment of a copy: copy_bytes from src, then
// (total_bytes - copy_bytes) zero bytes.  copy_bytes may be 0.
//
// rows > 1 makes it a strided block of `rows` such rows, row r copied from
// src + r*src_pitch to dst + r*dst_pitch.  Such a block has no zero fill
// (copy_bytes == total_bytes).  When both pitches are multiples of 16 every
// row has the alignment of the first and rows_per_chunk * copy_bytes is at
// most the chunk size; otherwise the rows of a chunk lie within 4 GiB of
// its first row on both sides and rows_per_chunk * copy_bytes is less than
// the chunk size plus one row.
struct CopySeg {
  uint64_t src;
  uint64_t dst;
  uint64_t copy_bytes;
  uint64_t total_bytes;
  uint64_t rows = 1;
  uint64_t src_pitch = 0;
  uint64_t dst_pitch = 0;
  uint64_t rows_per_chunk = 1;
};

// One reduction job over nbytes of destination: the first data_bytes are
// the reduction of the operands ptr[src0 .. src0+nsrc) (read at the same
// offsets), the rest is zero filled; every destination ptr[dst0 ..
// dst0+ndst) gets the same result.  All destinations share their address
// modulo 16.  AVG divides by nsrc.
//
// rows > 1 makes it a strided block of `rows` rows of nbytes: row r of
// operand t at ptr[src0 + t] + r*src_pitch, of destination m at
// ptr[dst0 + m] + r*dst_pitch.  Such a job has no zero fill (data_bytes ==
// nbytes) and rows_per_chunk * nbytes is at most the chunk size.
struct RedJob {
  uint64_t nbytes;
  uint64_t data_bytes;
  uint32_t src0;
  uint32_t nsrc;
  uint32_t dst0;
  uint32_t ndst;
  uint64_t rows = 1;
  uint64_t src_pitch = 0;
  uint64_t dst_pitch = 0;
  uint64_t rows_per_chunk = 1;
};

// A parameter sharded on a non-zero dim, all nrank shard ranks at once:
// the full tensor is `rows` rows of nrank pieces of run_bytes (piece s of
// row r is row r of rank s's chunk), contiguous from `full`; rank s's rows
// are dense from rank0 + s*rank_pitch (row r at + r*run_bytes).
// gather != 0: ranks to full (AG copy-out); else full to ranks (RS copy-in).
// Used for short rows, where the ranks' pieces share every cache line of the
// full tensor: a chunk is rows_per_chunk whole full-tensor rows (at most the
// chunk size), so one workgroup reads and writes whole lines on both sides.
// unit (16, 8, 4 or 2) is the access width; it divides run_bytes, full,
// rank0 and rank_pitch.
//
// rows_per_chunk == 0 marks rows too long for one chunk: the contiguous
// full tensor is cut into flat chunks of `reserved` bytes (kFlatChunk),
// chunk k being its bytes [k * reserved, (k + 1) * reserved), whatever
// rows they cross; such chunks are staged through LDS.  The planner emits
// them only for rank rows of at least kFlatMinRun bytes, so a flat chunk
// meets at most kFlatMaxPieces rank rows.
constexpr uint64_t kFlatChunk = 12288;
constexpr uint64_t kFlatMinRun = 1024;
constexpr uint32_t kFlatMaxPieces = (uint32_t)(kFlatChunk / kFlatMinRun + 2);

// Fold chunks with units of at most kFoldLdsMaxUnit bytes (and fold-reduce
// chunks over at least 4 ranks) are staged through LDS where they fit.  A
// fold-reduce item with wider units over fewer ranks never is: its chunks
// hold kFoldUnitChunk bytes of full-tensor rows per operand, and at least
// two rows.  Over 2 ranks that is one whole iteration of the kernel's unit
// loop for 8- and 16-byte units (every load of the chunk in flight at
// once); a row longer than half of it would leave half an iteration idle,
// so such rows go two to a chunk.
#ifndef FSDP_FOLD_LDS_MAX_UNIT
#define FSDP_FOLD_LDS_MAX_UNIT 4
#endif
#ifndef FSDP_FOLD_UNIT_CHUNK
#define FSDP_FOLD_UNIT_CHUNK 16384
#endif
constexpr uint32_t kFoldLdsMaxUnit = FSDP_FOLD_LDS_MAX_UNIT;
constexpr uint64_t kFoldUnitChunk = FSDP_FOLD_UNIT_CHUNK;

struct FoldSeg {
  uint64_t full;
  uint64_t run_bytes;
  uint64_t rows;
  uint64_t rows_per_chunk;
  uint64_t rank0;
  uint64_t rank_pitch;
  uint32_t nrank;
  uint32_t unit;
  uint32_t gather;
  uint32_t reserved;
};

// The fused RS of a parameter sharded on a non-zero dim with short chunk
// rows, one shard group at a time: the group's nrank gradients are `rows`
// full-tensor rows of nrank pieces of run_bytes each (piece s of row r is
// row r of rank s's chunk), gradient t contiguous from ptr[src0 + t].  The
// rows are summed over t in ascending order (whole rows, whole lines) and
// piece s of the result goes to rank s's output, whose rows are dense from
// ptr[dst0 + s].  A chunk is rows_per_chunk whole full-tensor rows (at most
// the larger of the copy and reduce chunk sizes; where the kernel never
// stages the item through LDS, kFoldUnitChunk bytes or two rows).  unit (16, 8, 4 or 2, at least the
// element size) is the access width; it divides run_bytes and every pointer.
// rows_per_chunk == 0 marks flat chunks of reserved[0] bytes of the full
// tensor, as for FoldSeg; every operand then sits at the same address
// modulo 16.
struct FoldRed {
  uint64_t run_bytes;
  uint64_t rows;
  uint64_t rows_per_chunk;
  uint32_t src0;
  uint32_t dst0;
  uint32_t nrank;
  uint32_t unit;
  uint64_t reserved[3];
};

// Bytes of the per-GPU scratch array that holds the descriptor tables of
// the entry point that allocates nothing (fsdp_rs_copy_reduce_noalloc).
constexpr size_t kScratchBytes = size_t(1) << 20;

static_assert(sizeof(CopySeg) == 64, "CopySeg layout");
static_assert(sizeof(RedJob) == 64, "RedJob layout");
static_assert(sizeof(FoldSeg) == 64, "FoldSeg layout");
static_assert(sizeof(FoldRed) == 64, "FoldRed layout");

// Number of chunks of a one-row item [dst, dst + nbytes), nbytes > 0.
inline uint64_t chunk_count(uint64_t dst, uint64_t nbytes, uint32_t shift) {
  return ((dst + nbytes - 1) >> shift) - (dst >> shift) + 1;
}

// Number of chunks of any item whose first destination row starts at dst.
inline uint64_t item_chunks(uint64_t dst, uint64_t row_bytes, uint64_t rows, uint64_t rows_per_chunk,
                            uint32_t shift) {
  if (rows > 1) return (rows + rows_per_chunk - 1) / rows_per_chunk;
  return chunk_count(dst, row_bytes, shift);
}

}  // namespace fsdp

// Launchers (defined in kernels.hip).  Return hipSuccess or the launch error.
// start_event / stop_event: hipEvent_t handles the kernel's dispatch records
// at its start and end (for callers that time the kernel), or NULL.
extern "C++" {
// stream_stores: nontemporal stores for the outputs (see the store policy in
// fsdp_flat.cpp).
int fsdp_launch_seg_copy(int elem_bytes, const void* dev_table, uint32_t n_seg,
                         uint64_t n_chunks, uint32_t chunk_shift, uint32_t max_grid,
                         int stream_stores, void* stream, void* start_event, void* stop_event);
// Every job of one launch has the same operand count n_src; elt is the
// element kind, an FSDP dtype code: FSDP_F32, FSDP_BF16 or FSDP_F16.
int fsdp_launch_reduce(int elt, const void* dev_table, uint32_t n_job, uint32_t n_src, uint64_t n_chunks,
                       uint32_t chunk_shift, uint32_t max_grid, int avg, int stream_stores,
                       void* stream, void* start_event, void* stop_event);
// One chunk of a fold item is rows_per_chunk full-tensor rows.  narrow: every
// item's unit is 2 or 4 bytes (the kernel's LDS-staged path).
int fsdp_launch_fold(const void* dev_table, uint32_t n_fold, uint64_t n_chunks, uint32_t max_grid, int narrow,
                     int stream_stores, void* stream, void* start_event, void* stop_event);
// Every item of one launch has n_src = nrank operands; elt as for the
// reduce launch; one chunk of an item is rows_per_chunk full-tensor rows;
// narrow: every item's unit is 2 or 4 bytes (the LDS-staged path).
int fsdp_launch_fold_reduce(int elt, const void* dev_table, uint32_t n_item, uint32_t n_src, uint64_t n_chunks,
                            uint32_t max_grid, int narrow, int avg, int stream_stores, void* stream,
                            void* start_event, void* stop_event);
// The current device's scratch array (fsdp::kScratchBytes, 256-byte
// aligned; its address is looked up once per device).
int fsdp_scratch_ptr(void** out);
// Enqueue on `stream` the writes of `bytes` host bytes to base + offset
// (base: fsdp_scratch_ptr's address), carried in kernel arguments: the host
// buffer may be freed when this returns.  offset is a multiple of 16.
int fsdp_scratch_write(void* base, const void* host, size_t bytes, size_t offset, void* stream);
}
