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
constexpr int kMaxBatch = 15000;    // keeps a decode workgroup's LDS (length prefix, held tokens) in 64 KiB
constexpr int kMaxGroup = 64;       // query heads per KV head
// Default lower bound on pages per chunk.  Chunks are otherwise sized to
// give one per resident group of wavefronts; on long sequences that makes
// them short, and each chunk pays a start-up latency and one partial per
// query head.  Measured on MI355X: 64 pages for groups <= 16 (131072-token
// GQA layer: 1024 chunks of 64 pages beat 2048 of 32 by 10%), 32 for larger
// groups (131072-token MQA: one chunk per CU is best).  The 8-bit cache's
// pages are half the bytes, and 32 pages is best there at every group size
// (131072-token GQA layer: 2048 chunks of 32 pages beat 1024 of 64 by 27%).
__host__ __device__ inline int default_min_chunk(int group, bool q8 = false) {
  return (q8 || group > 16) ? 32 : 64;
}
constexpr int kMaxItems = 1 << 22;  // work items per decode launch
constexpr size_t kMaxLdsBytes = 64 * 1024;  // LDS one decode workgroup may use
// The wide kernel runs one workgroup per CU and may take the whole LDS of a
// gfx950 CU for its merge slots.
constexpr size_t kMaxLdsBytesWide = 160 * 1024;

__host__ __device__ inline int pages_of_len(int64_t len, int64_t max_blocks) {
  if (len <= 0 || len > max_blocks * kBlock) return 0;
  return static_cast<int>((len + kBlock - 1) / kBlock);
}

// Several query tokens per sequence (the last q_len cached tokens, each
// attending causally, optionally only to the last `window` keys): the first
// block any of them attends, and the pages from there to the sequence's end.
// A length below q_len is invalid (no pages; the rows become NaN).
__host__ __device__ inline int first_block(int64_t len, int64_t q_len, int64_t window) {
  if (window <= 0) return 0;
  const int64_t lo = len - q_len + 1 - window;   // window start of the first query token
  return lo <= 0 ? 0 : static_cast<int>(lo / kBlock);
}
__host__ __device__ inline int pages_of_range(int64_t len, int64_t max_blocks, int64_t q_len, int64_t window) {
  if (len < q_len) return 0;
  const int n = pages_of_len(len, max_blocks);
  return n == 0 ? 0 : n - first_block(len, q_len, window);
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

// Pairs whose pages span at most this many chunks are merged by the chunk
// that finishes last, inside the decode kernel; longer ones by the combine
// kernel (one wavefront would read all their partials).
constexpr int kFuseMaxParts = 96;
// The wide kernel (33 to 64 columns per KV head) merges 64 columns per pair,
// four partials per round trip, in the one wavefront per 16-column block of
// the pair's last workgroup, while the rest of the chip has finished: at 32
// partials a pair (the 8-token 70B layer) that tail cost about 30 % of the
// launch against the combine kernel.  So when a pair may span more than
// kWideFuseMaxParts chunks the combine kernel runs, and only pairs of at most
// kWideFuseSmallParts chunks are merged inside the wide kernel.
constexpr int kWideFuseMaxParts = 24;
constexpr int kWideFuseSmallParts = 8;
// The largest pair (in chunks) merged inside the decode kernel, given the
// bound max_parts on a pair's chunks; the combine kernel runs for the rest
// when max_parts exceeds it.
inline int fuse_limit(bool wide, int64_t max_parts) {
  return wide && max_parts > kWideFuseMaxParts ? kWideFuseSmallParts : kFuseMaxParts;
}
constexpr int kMaxWavesPerChunk = 4;

// Workspace layout: partial outputs [slots][group][head_dim] f32, partial
// lse [slots][group] f32, then (256-byte aligned) the per-sequence page
// prefix [batch + 1] int32 that the split kernel stores for the combine
// kernel.  The counters sit at the END of the workspace, counted backwards
// from its last int32 word: that word is the dynamic schedule's chunk
// counter, and the words before it hold one arrival counter per (sequence,
// KV head, head block), (b, h, gb) at word -(2 + (b * n_kv + h) * 4 + gb).
// Their place depends only on the workspace's size, never on the batch, so
// a workspace sized for batch B serves later calls with any batch <= B:
// every call leaves its counters zero, and no call's partials or prefix
// reach a word another call uses as a counter.
__host__ __device__ inline int64_t decode_prefix_offset(int64_t batch, int64_t group, int64_t n_kv,
                                                        int64_t head_dim, int64_t n_items) {
  const int64_t parts = decode_slots(batch, n_kv, n_items) * group * (head_dim + 1) * 4;
  return (parts + 255) & ~int64_t{255};
}
__host__ __device__ inline int64_t decode_counters_count(int64_t batch, int64_t n_kv) {
  return batch * n_kv * kMaxWavesPerChunk;
}
// Bytes of the counters at the workspace's end (arrival counters and the chunk counter).
__host__ __device__ inline int64_t decode_tail_bytes(int64_t batch, int64_t n_kv) {
  return (decode_counters_count(batch, n_kv) + 1) * 4;
}
__host__ __device__ inline int64_t decode_workspace_end(int64_t batch, int64_t group, int64_t n_kv,
                                                        int64_t head_dim, int64_t n_items) {
  return decode_prefix_offset(batch, group, n_kv, head_dim, n_items) + (batch + 1) * 4 +
         decode_tail_bytes(batch, n_kv);
}

// Dynamic schedule (pkv_decode_opts.schedule): one workgroup per CU; by
// default kDynChunksPerWave chunks per wavefront of at least kDynMinChunk
// pages, so that wavefronts that run faster can take more of them.
constexpr int kDynChunksPerWave = 8;
constexpr int kDynMinChunk = 16;
// Pairs a wavefront of the dynamic kernel lists before counting their arrivals.
constexpr int kMaxPending = 64;
// LDS of the decode kernels (int32 units): the prefix [batch + 1] and the
// per-wave sums, then, 16-byte aligned, each wavefront's held tokens of a
// fused append (K row and V row of head_dim <= 128 elements and the token's
// destination: at most kHeldWords words each) and (split kernel, one
// wavefront per chunk) its held results, then (dynamic kernel) each
// wavefront's list of pending pairs (kMaxPending int4 entries).
constexpr int kHeldWords = 128 * 4 / 4 + 128 + 8;
// Row stride (floats) of a block of output rows [rows][head_dim] held in
// LDS.  A 16-byte LDS access by lanes (c, n) touches row n at feature 4c
// (+16 nb); with an unpadded stride of 128 or 64 floats every row starts in
// the same bank and the 16 rows of one access serialise.  Four floats of
// padding move row n by 4n banks, so the 16 rows of an access fall in
// disjoint banks.
__host__ __device__ constexpr int lds_row(int head_dim) { return head_dim + 4; }
// Result and token slots per wavefront of the split kernel, at most.
constexpr int kMaxHeldSlots = 8;
__host__ __device__ inline int held_offset(int batch) { return (batch + 1 + kWavesPerGroup + 3) & ~3; }
__host__ __device__ inline int dyn_pending_offset(int batch) {
  return held_offset(batch) + kWavesPerGroup * kHeldWords;
}

}  // namespace pkv
