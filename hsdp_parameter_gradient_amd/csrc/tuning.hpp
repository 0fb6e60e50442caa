// Launch tuning of the gfx950 kernels: work-chunk sizes, grid cap and the
// store policy.  Read once per process; the defaults are the measured best on
// MI355X, and FSDP_COPY_CHUNK_SHIFT, FSDP_REDUCE_CHUNK_SHIFT, FSDP_MAX_GRID
// and FSDP_CACHED_STORE_MAX_MIB override them for experiments.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <cstdlib>

namespace fsdp {

struct Tuning {
  uint32_t copy_shift = 14;    // 16 KiB of destination per chunk
  uint32_t reduce_shift = 13;  // 8 KiB of destination per chunk
  // One workgroup per chunk up to 4 Mi workgroups (64 GiB of copy, 32 GiB of
  // reduce output); larger calls walk the chunks grid-stride.  Measured on a
  // 51.8 GB RS copy-in (3.16 M chunks): a 2^22 cap 1-2 % faster than 2^20,
  // 2^18 5-7 % slower.
  uint32_t max_grid = 1u << 22;
  // Store policy.  An output that the next step of the path reads back (the
  // AG buffer read by copy-out, the RS input read by the RS, the RS output
  // read by the fused AR) keeps normal stores while it is at most this many
  // bytes, so that part of it is still in the 256 MB MALL when it is read;
  // larger outputs, and the path's final outputs (the full parameters, the
  // AR result), use nontemporal stores.  Measured on MI355X: streaming stores
  // are 3-5% faster on multi-GB buckets and 8% slower on a 0.4 GB one.
  uint64_t cached_store_max = uint64_t(512) << 20;
};

inline const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning x;
    if (const char* e = std::getenv("FSDP_COPY_CHUNK_SHIFT"))
      x.copy_shift = (uint32_t)std::max(9, std::min(24, std::atoi(e)));
    if (const char* e = std::getenv("FSDP_REDUCE_CHUNK_SHIFT"))
      x.reduce_shift = (uint32_t)std::max(9, std::min(24, std::atoi(e)));
    if (const char* e = std::getenv("FSDP_MAX_GRID")) x.max_grid = (uint32_t)std::max(1, std::atoi(e));
    if (const char* e = std::getenv("FSDP_CACHED_STORE_MAX_MIB"))
      x.cached_store_max = uint64_t(std::max(0, std::atoi(e))) << 20;
    return x;
  }();
  return t;
}

}  // namespace fsdp
