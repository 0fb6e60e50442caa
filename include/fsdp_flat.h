/*
 * fsdp_flat.h — C ABI of the MI355X (gfx950) FSDP/HSDP flat-buffer hot path.
 *
 * One bucket of P parameters, sharded (on dim 0 unless a parameter states
 * another dim) over a shard group of S ranks and replicated over D = R / S
 * replicate groups, R simulated ranks resident in one GPU's HBM.  Every device entry point is one HIP kernel launch,
 * enqueued on the caller's stream.  A call whose descriptor table (a
 * function of its shapes, sizes and pointers) is new uploads that table
 * once with a blocking copy; a repeated call makes no HIP call besides the
 * launch and does not synchronise the host.
 *
 * Sources (cited by page title and section):
 *   [FS-MD]  FullyShard multi-dimensional parallel adaptation RFC
 *            (yide12/hyper-parallel issue 1): 2.2.1 two-group model,
 *            2.2.2 decision matrix, 2.2.5 rank/shard/dp sizes, 3.3.
 *   [HYPER]  Hyper communication-overlap scheme, PR #758 write-up
 *            (mindspore/hyper-parallel issue 184): 2.1 fused packing and the
 *            512-byte-aligned fused AR buffer, 2.3 SUM / AVG scaling,
 *            4.1 AG send buffer = this rank's slice of the AG output.
 *   [RAGGED] FSDP dim-0 non-uniform sharding RFC (mindspore/hyper-parallel
 *            issue 319): 5.1 interface and errors, 6.4 chunk rule, padded
 *            communication storage, AG / RS padding rules.
 *
 * Notation (all counts in elements unless a name says bytes), for a
 * parameter sharded on dim 0 (see fsdp_bucket_t for other dims):
 *   param i: shape (N0_i, ...), inner_i = product of dims after dim 0
 *   chunk_i = ceil(N0_i / S); rank s holds rows
 *     [row_off(i,s), row_off(i,s) + row_len(i,s)) with
 *     row_off = min(s*chunk_i, N0_i), row_len = min(chunk_i, N0_i - row_off)
 *   padded_i = outer_i * chunk_i * inner_i; in_off_i = sum_{j<i} padded_j;
 *   I = sum_i padded_i (elements of one rank slice)
 *   rank g = d*S + s: shard group d = {d*S .. d*S+S-1},
 *   replicate group s = {s, S+s, .., (D-1)*S+s}
 *
 * Conventions shared by every entry point:
 *   - Status: FSDP_OK (0) or a positive error code; fsdp_last_error() gives
 *     a message for the calling thread.  Arguments are validated completely
 *     before anything is enqueued: on error nothing is launched.  No C++
 *     exception leaves the library: a host allocation that fails while a
 *     call is planned returns FSDP_ENOMEM.
 *   - Device pointers are plain addresses of device memory owned by the
 *     caller.  The caller keeps every buffer alive and unchanged (inputs) or
 *     untouched (outputs) until the stream has passed the call.  Buffer
 *     capacities cannot be checked here: the caller guarantees that every
 *     buffer holds the element count stated for it.
 *   - Every pointer must be aligned to its element size (FSDP_EALIGN).
 *     A pointer whose buffer is empty (0 bytes) may be NULL.
 *   - Outputs must not overlap inputs or each other (FSDP_EOVERLAP), except
 *     fsdp_fused_ar, which works in place by definition.
 *   - Padding is written as zero on every call; no output needs to be
 *     cleared beforehand.
 *   - The library caches a plan per call signature (entry point, sizes,
 *     shapes, shard dims, pointers, device): the call's descriptor table in
 *     device memory and its launch parameters.  A repeated call launches its
 *     plan without validating or planning again (its result cannot differ).
 *     At most 256 plans and 256 MiB of tables; evicting waits for every
 *     device that holds a cached table.  fsdp_release_cache() frees them all.
 *   - A call whose plan is cached only enqueues its kernel launches (one,
 *     or two when some parameters take the fold kernel), so it can be
 *     captured into a HIP graph and replayed (the graph reads the buffers'
 *     contents at replay time).  A plan launched into a capture is pinned:
 *     eviction never frees it, since the graph holds its table's address.
 *     The first call of a signature allocates and uploads its tables and
 *     may evict (synchronizing devices), so it is refused with FSDP_EINVAL
 *     while its stream is being captured, before anything is enqueued:
 *     issue each call once before capturing it.  No graph that captured a
 *     call may be replayed after fsdp_release_cache().
 *   - Thread safe; calls that overlap in time on different streams must not
 *     share output buffers.
 */
#ifndef FSDP_FLAT_H
#define FSDP_FLAT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FSDP_OK        0
#define FSDP_EINVAL    1  /* bad size, count, pointer or group arithmetic */
#define FSDP_ENOTIMPL  2  /* an uneven non-zero shard dim, or a dtype the op does not take */
#define FSDP_EALIGN    3  /* pointer not aligned as required */
#define FSDP_EHIP      4  /* a HIP runtime call failed */
#define FSDP_EOVERLAP  5  /* an output overlaps an input or another output */
#define FSDP_ENOMEM    6  /* host memory for the call's plan could not be allocated */

/* element types: copies take any of them (bits are moved, not converted);
 * reductions take FSDP_F32, FSDP_BF16 or FSDP_F16 (16-bit elements are
 * widened exactly, summed in fp32 and rounded once to nearest even at the
 * store; a bf16 NaN stores as 0x7FC0, an fp16 NaN as a quiet NaN; fp16
 * overflows to infinity and keeps its denormals) */
#define FSDP_F32   0
#define FSDP_BF16  1
#define FSDP_F16   2

/* reduce ops ([HYPER] 2.3) */
#define FSDP_SUM   0
#define FSDP_AVG   1  /* sum, then divide by the group's size (IEEE fp32) */

/* Segment alignment of the fused AR buffer ([HYPER] 2.1). */
#define FSDP_FUSED_ALIGN_BYTES 512

/*
 * A bucket: P parameter shapes in bucket order.
 *   n_params   P >= 0
 *   ndim       [P] number of dims of each parameter, each >= 1
 *   shape      concatenation of all shapes (sum(ndim) entries, each >= 0)
 *   shard_dim  the dim every parameter is sharded on
 *   shard_dims [P] one shard dim per parameter, or NULL (= shard_dim for all)
 * Dim 0 may be uneven (fixed-size chunks, zero padding at the tail,
 * [RAGGED] 6.4).  Any other dim k must be divisible by shard_size: rank s
 * holds the s-th of S equal chunks along k, stored contiguously, with no
 * padding ([RAGGED] 3.2 keeps non-zero dims on the plain chunk/concatenate
 * path; an uneven non-zero dim is FSDP_ENOTIMPL, as the NotImplementedError
 * of its 5.1 interface table).  A dim outside [0, ndim) is FSDP_EINVAL.
 * Below, for a parameter sharded on k: outer = product of the dims before
 * k (1 for k = 0), inner = product of the dims after k, and "rows" are
 * indices along k; rank s's chunk is outer runs of row_len * inner elements.
 */
typedef struct fsdp_bucket {
  int32_t n_params;
  const int32_t* ndim;
  const int64_t* shape;
  int32_t shard_dim;
  const int32_t* shard_dims;
} fsdp_bucket_t;

/* ------------------------------------------------------------------------
 * Host-only queries (no HIP call, callable without a GPU)
 * ------------------------------------------------------------------------ */

/*
 * Layout of a bucket sharded over shard_size ranks ([RAGGED] 6.4).
 * Outputs (any may be NULL): *slice_numel = I; padded[P], in_off[P];
 * row_off[P*S] and row_len[P*S], indexed [i*S + s].
 * Errors: FSDP_EINVAL (shard_size < 1, ndim < 1, negative dim, shard dim
 * out of range, overflow), FSDP_ENOTIMPL (uneven non-zero shard dim).
 */
int fsdp_bucket_layout(const fsdp_bucket_t* bucket, int32_t shard_size,
                       int64_t* slice_numel, int64_t* padded, int64_t* in_off,
                       int64_t* row_off, int64_t* row_len);

/*
 * Layout of the fused AR buffer ([HYPER] 2.1): segment j (seg_numel[j]
 * elements of elem_bytes each) starts at element seg_off[j], on a 512-byte
 * boundary after the end of segment j-1; *fused_numel is the total, rounded
 * up to 512 bytes.  The gaps are padding and hold zero.
 * Errors: FSDP_EINVAL (n_seg < 0, negative size, elem_bytes not in {2, 4}).
 */
int fsdp_fused_layout(int32_t n_seg, const int64_t* seg_numel, int32_t elem_bytes,
                      int64_t* seg_off, int64_t* fused_numel);

/*
 * Backward communication decision matrix ([FS-MD] 2.2.2, 2.2.5, 3.3):
 * RS over the shard groups when shard_size > 1, then AR over the replicate
 * groups when dp_size = rank_size / shard_size > 1; nothing when both are 1.
 * Outputs: *n_rs_groups (D or 0) and rs_ranks[R] (group-major, may be NULL);
 * *n_ar_groups (S or 0) and ar_ranks[R] (group-major, may be NULL).
 * Errors: FSDP_EINVAL (sizes < 1, rank_size not a multiple of shard_size).
 */
int fsdp_group_ranks(int32_t rank_size, int32_t shard_size,
                     int32_t* n_rs_groups, int32_t* rs_ranks,
                     int32_t* n_ar_groups, int32_t* ar_ranks);

/* ------------------------------------------------------------------------
 * Device entry points (async on `stream`, a hipStream_t; NULL = null stream)
 * ------------------------------------------------------------------------ */

/*
 * AG copy-in ([HYPER] 2.1 and 4.1; [RAGGED] 6.4): for every shard rank s
 * and parameter i, copy shard (s, i) into ag[s*I + in_off_i ...] and write
 * zeros over the rest of its padded region.  All S slices are packed, so
 * the AllGather of one shard group is the identity on `ag`.
 *   shards  [S*P] device pointers, rank-major: shards[s*P + i] holds
 *           outer_i * row_len(i,s) * inner_i contiguous elements (rank s's
 *           chunk in its own dense layout; NULL allowed when 0)
 *   ag      device buffer of S*I elements (written entirely)
 *   dtype   FSDP_F32 / FSDP_BF16 / FSDP_F16 (element size only)
 */
int fsdp_ag_copy_in(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype,
                    const void* const* shards, void* ag, void* stream);

/*
 * AG copy-out ([HYPER] 2.1 copy-out; [RAGGED] 6.4: only the logical shape
 * is exposed): full parameter i = concatenation along its shard dim over s
 * of rank s's chunk in slice s's region of parameter i.  Padding is never
 * read.
 *   ag     device buffer of S*I elements
 *   full   [P] device pointers, full[i] holds N0_i * inner_i elements
 */
int fsdp_ag_copy_out(const fsdp_bucket_t* bucket, int32_t shard_size, int32_t dtype,
                     const void* ag, void* const* full, void* stream);

/*
 * RS copy-in ([RAGGED] 6.4 fused RS copy-in): for every rank g, chunk s of
 * every gradient i (along its shard dim, in dense layout) goes to
 * rs_in[g][s*I + in_off_i ...], zero padded to padded_i.
 *   grads  [R*P] device pointers, grads[g*P + i] holds N0_i * inner_i elements
 *   rs_in  [R] device pointers, each S*I elements (written entirely)
 */
int fsdp_rs_copy_in(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                    int32_t dtype, const void* const* grads, void* const* rs_in,
                    void* stream);

/*
 * RS over every shard group ([FS-MD] 2.2.1, 3.3; [HYPER] 2.3):
 *   rs_out[d*S+s][k] = op( sum_{t=0..S-1} rs_in[d*S+t][s*I + k] ),  k < I,
 * summed in ascending t in fp32, the accumulator starting from t = 0; AVG
 * divides the sum by S.  rs_out[g] may be a view into rank g's fused AR
 * buffer (zero-copy, [HYPER] 2.1).
 *   rs_in   [R] device pointers, S*I elements each
 *   rs_out  [R] device pointers, I elements each
 *   dtype   FSDP_F32, FSDP_BF16 or FSDP_F16 (else FSDP_ENOTIMPL)
 */
int fsdp_rs_reduce(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                   int32_t dp_size, int32_t op, int32_t dtype,
                   const void* const* rs_in, void* const* rs_out, void* stream);

/*
 * RS copy-in and RS in one pass, without materialising the RS input:
 *   rs_out[d*S+s][in_off_i + k] = op( sum_{t=0..S-1} chunk_s(grads[(d*S+t)*P + i])[k] )
 * for k below the chunk's size, and 0 over the rest of parameter i's padded
 * region (chunk_s = rank s's chunk along the shard dim, dense layout).  Bit for bit the result of fsdp_rs_copy_in followed by
 * fsdp_rs_reduce (same order, same rounding); each gradient element is read
 * once and no S*I buffer is written ([RAGGED] 6.4 padded RS input;
 * [FS-MD] 3.3 RS on the shard group).
 *   grads   [R*P] device pointers, grads[g*P + i] holds N0_i * inner_i elements
 *   rs_out  [R] device pointers, I elements each (may be fused-buffer views)
 *   dtype   FSDP_F32, FSDP_BF16 or FSDP_F16 (else FSDP_ENOTIMPL)
 */
int fsdp_rs_copy_reduce(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                        int32_t dp_size, int32_t op, int32_t dtype,
                        const void* const* grads, void* const* rs_out, void* stream);

/*
 * fsdp_rs_copy_reduce for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result (bit for bit), validation and
 * errors as fsdp_rs_copy_reduce; it allocates no device or pinned host
 * memory.  Its descriptor tables live in a static per-GPU scratch array of
 * 1 MiB (held until the process ends), written on every call by small
 * kernel launches on `stream` that carry the table bytes in their kernel
 * arguments, followed by the same kernels as fsdp_rs_copy_reduce.  Nothing
 * is cached: every call plans again on the host (host heap memory only).
 * Every call on a GPU rewrites that GPU's array, so calls that overlap in
 * time on one GPU (on different streams) race; calls in one stream order
 * are safe.  A call whose tables exceed the array (roughly 10,000 jobs) is
 * refused with FSDP_EINVAL before anything is enqueued.
 */
int fsdp_rs_copy_reduce_noalloc(const fsdp_bucket_t* bucket, int32_t rank_size, int32_t shard_size,
                                int32_t dp_size, int32_t op, int32_t dtype,
                                const void* const* grads, void* const* rs_out, void* stream);

/*
 * Fused AR over every replicate group, in place ([HYPER] 2.1, 2.3):
 *   acc = sum_{d=0..D-1} fused[d*S+s][k]  (ascending d, fp32),
 *   AVG: acc = acc / D;  fused[d*S+s][k] = acc for every d,
 * for every k of the whole fused buffer (segments and zero gaps).
 *   seg_numel  [n_seg] segment sizes; the buffer size is fsdp_fused_layout's
 *              for the dtype's element size
 *   fused      [R] device pointers, each 512-byte aligned (FSDP_EALIGN)
 *   dtype      FSDP_F32, FSDP_BF16 or FSDP_F16 (else FSDP_ENOTIMPL)
 */
int fsdp_fused_ar(int32_t n_seg, const int64_t* seg_numel, int32_t rank_size,
                  int32_t shard_size, int32_t dp_size, int32_t op, int32_t dtype,
                  void* const* fused, void* stream);

/* Message for the calling thread's last error ("" after success). */
const char* fsdp_last_error(void);

/* Free the cached descriptor tables, pinned ones included (waits first for
 * every device that holds one).  Not while a stream is being captured. */
void fsdp_release_cache(void);

/* State of the plan cache: the number of cached plans, how many of them
 * are pinned by a graph capture, and the device bytes their tables hold.
 * Any pointer may be NULL.  Always FSDP_OK. */
int fsdp_cache_info(int64_t* n_plans, int64_t* n_pinned, int64_t* table_bytes);

/*
 * For callers that time one call: the next call that the calling thread
 * makes through any device entry point above records start_event when its
 * first kernel starts executing and stop_event when its last kernel ends
 * (in the kernels' own dispatches, so the interval excludes the launch and
 * queue overheads that events recorded around a call include; a call that
 * launches two kernels, when some parameters take the fold kernel, is
 * timed from the start of the first to the end of the second).  start_event and stop_event are hipEvent_t handles
 * the caller created with timing enabled and on the launch's device; both
 * NULL cancels a pending request.  A call that launches nothing (an empty
 * bucket, an AR over one rank), or launches into a stream that is being
 * captured into a graph, leaves the request pending.
 * Errors: FSDP_EINVAL (exactly one of the two is NULL).
 */
int fsdp_time_next_launch(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* FSDP_FLAT_H */
