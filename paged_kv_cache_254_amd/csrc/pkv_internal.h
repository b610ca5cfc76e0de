// Internal helpers shared by the host and device translation units of libpkv.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "pkv.h"

namespace pkv {

// Records the detail string returned by pkv_last_error() and returns status.
int fail(int status, const std::string& detail);
// Clears the thread's last error and returns PKV_OK.
int ok();

constexpr int kBlock = 16;          // tokens per page (the only size built)
constexpr int kWave = 64;           // CDNA wavefront
constexpr int kWavesPerGroup = 4;   // wavefronts per workgroup of the decode kernels
constexpr int kMaxBatch = 16000;    // keeps the per-workgroup length prefix in 64 KiB of LDS
constexpr int kMaxGroup = 64;       // query heads per KV head
constexpr int kDefaultMinChunk = 8; // pages
constexpr int kMaxItems = 1 << 22;  // work items per decode launch

__host__ __device__ inline int pages_of_len(int64_t len, int64_t max_blocks) {
  if (len <= 0 || len > max_blocks * kBlock) return 0;
  return static_cast<int>((len + kBlock - 1) / kBlock);
}

// Wavefronts that share one chunk: one per 16 query heads, rounded up to a power of two.
__host__ __device__ inline int waves_per_chunk(int group) {
  int gb = (group + 15) / 16;
  return gb <= 1 ? 1 : (gb == 2 ? 2 : 4);
}

__host__ __device__ inline int chunk_pages(int64_t total, int64_t n_items, int64_t min_chunk) {
  int64_t c = (total + n_items - 1) / n_items;
  return static_cast<int>(c < min_chunk ? min_chunk : c);
}

__host__ __device__ inline int64_t decode_slots(int64_t batch, int64_t n_kv, int64_t n_items) {
  return n_items + batch * n_kv;
}

}  // namespace pkv
