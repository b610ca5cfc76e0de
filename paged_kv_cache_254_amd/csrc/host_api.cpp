// Host side of libpkv: status strings, byte accounting, the page pool and
// block tables, and the host mirror of the decode split plan.
//
// Page pool: on-demand allocation of fixed-size blocks from a free list, with
// a per-request block table from logical to physical block ("Inference
// Engines", chapter 17, "The Breakthrough"; CS336 lecture 10 notes,
// "PagedAttention (vLLM)", which also describes sharing blocks between
// sequences with copy-on-write).
#include <algorithm>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

int fail(int status, const std::string& detail) {
  g_last_error = detail;
  return status;
}

int ok() {
  g_last_error.clear();
  return PKV_OK;
}

}  // namespace pkv

struct pkv_pool {
  int32_t num_pages = 0;
  std::deque<int32_t> free_list;
  std::unordered_map<int64_t, std::vector<int32_t>> seqs;
  std::vector<int32_t> refs;
};

using pkv::fail;
using pkv::ok;

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_OUT_OF_PAGES: return "out of pages";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_NOT_FOUND: return "unknown sequence";
    case PKV_ERR_EXISTS: return "sequence already exists";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }

// Chapter 17 "The Mathematics", equation M_kv: 2 * L * n_kv * d_h * s * b * p.
uint64_t pkv_kv_cache_bytes(int64_t n_layers, int64_t n_kv_heads, int64_t head_dim,
                            int64_t seq_len, int64_t batch, int64_t elem_bytes) {
  if (n_layers < 0 || n_kv_heads < 0 || head_dim < 0 || seq_len < 0 || batch < 0 ||
      elem_bytes < 0)
    return 0;
  return 2ull * static_cast<uint64_t>(n_layers) * static_cast<uint64_t>(n_kv_heads) *
         static_cast<uint64_t>(head_dim) * static_cast<uint64_t>(seq_len) *
         static_cast<uint64_t>(batch) * static_cast<uint64_t>(elem_bytes);
}

uint64_t pkv_kv_bytes_per_token(int64_t n_layers, int64_t n_kv_heads, int64_t head_dim,
                                int64_t elem_bytes) {
  return pkv_kv_cache_bytes(n_layers, n_kv_heads, head_dim, 1, 1, elem_bytes);
}

int pkv_pool_create(int32_t num_pages, const int32_t* free_order, pkv_pool** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: out is NULL");
  *out = nullptr;
  if (num_pages < 1) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: num_pages < 1");
  auto* pool = new (std::nothrow) pkv_pool;
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_create: allocation failed");
  pool->num_pages = num_pages;
  pool->refs.assign(num_pages, 0);
  if (free_order) {
    std::vector<char> seen(num_pages, 0);
    for (int32_t i = 0; i < num_pages; ++i) {
      int32_t p = free_order[i];
      if (p < 0 || p >= num_pages || seen[p]) {
        delete pool;
        return fail(PKV_ERR_INVALID_ARG,
                    "pkv_pool_create: free_order is not a permutation of 0..num_pages-1");
      }
      seen[p] = 1;
      pool->free_list.push_back(p);
    }
  } else {
    for (int32_t i = 0; i < num_pages; ++i) pool->free_list.push_back(i);
  }
  *out = pool;
  return ok();
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int32_t pkv_pool_num_free(const pkv_pool* pool) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_pool_num_free: pool is NULL");
  return static_cast<int32_t>(pool->free_list.size());
}

int pkv_seq_reserve(pkv_pool* pool, int64_t seq_id, int64_t n_tokens, int32_t block_size,
                    int32_t* n_new_pages) {
  if (n_new_pages) *n_new_pages = 0;
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve: pool is NULL");
  if (n_tokens < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve: negative length or bad block size");
  auto it = pool->seqs.find(seq_id);
  int64_t have = it == pool->seqs.end() ? 0 : static_cast<int64_t>(it->second.size());
  int64_t need = (n_tokens + block_size - 1) / block_size - have;
  if (need > static_cast<int64_t>(pool->free_list.size()))
    return fail(PKV_ERR_OUT_OF_PAGES, "pkv_seq_reserve: need " + std::to_string(need) +
                                          " pages, " + std::to_string(pool->free_list.size()) +
                                          " free");
  std::vector<int32_t>& pages = pool->seqs[seq_id];
  for (int64_t i = 0; i < need; ++i) {
    int32_t p = pool->free_list.front();
    pool->free_list.pop_front();
    pool->refs[p] = 1;
    pages.push_back(p);
  }
  if (n_new_pages) *n_new_pages = need > 0 ? static_cast<int32_t>(need) : 0;
  return ok();
}

int pkv_seq_release(pkv_pool* pool, int64_t seq_id) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_release: pool is NULL");
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NOT_FOUND, "pkv_seq_release: unknown sequence " + std::to_string(seq_id));
  for (int32_t p : it->second) {
    if (--pool->refs[p] == 0) pool->free_list.push_back(p);
  }
  pool->seqs.erase(it);
  return ok();
}

int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_fork: pool is NULL");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NOT_FOUND, "pkv_seq_fork: unknown parent " + std::to_string(parent));
  if (pool->seqs.count(child))
    return fail(PKV_ERR_EXISTS, "pkv_seq_fork: child exists " + std::to_string(child));
  std::vector<int32_t> pages = it->second;
  for (int32_t p : pages) ++pool->refs[p];
  pool->seqs.emplace(child, std::move(pages));
  return ok();
}

int pkv_seq_reserve_for_write(pkv_pool* pool, int64_t seq_id, int64_t position,
                              int32_t block_size, int32_t* copy_src, int32_t* copy_dst) {
  if (copy_src) *copy_src = -1;
  if (copy_dst) *copy_dst = -1;
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve_for_write: pool is NULL");
  if (position < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_seq_reserve_for_write: bad position or block size");
  // A copy-on-write may need one page beyond the growth itself; check both up
  // front so that a failure leaves the pool unchanged.
  auto it = pool->seqs.find(seq_id);
  int64_t have = it == pool->seqs.end() ? 0 : static_cast<int64_t>(it->second.size());
  int64_t blk = position / block_size;
  int64_t grow = std::max<int64_t>(0, blk + 1 - have);
  bool shared = blk < have && pool->refs[it->second[blk]] > 1;
  if (grow + (shared ? 1 : 0) > static_cast<int64_t>(pool->free_list.size()))
    return fail(PKV_ERR_OUT_OF_PAGES, "pkv_seq_reserve_for_write: out of pages");
  int st = pkv_seq_reserve(pool, seq_id, position + 1, block_size, nullptr);
  if (st != PKV_OK) return st;
  if (!shared) return ok();
  std::vector<int32_t>& pages = pool->seqs[seq_id];
  int32_t old_page = pages[blk];
  int32_t new_page = pool->free_list.front();
  pool->free_list.pop_front();
  pool->refs[new_page] = 1;
  --pool->refs[old_page];
  pages[blk] = new_page;
  if (copy_src) *copy_src = old_page;
  if (copy_dst) *copy_dst = new_page;
  return ok();
}

int pkv_seq_num_blocks(const pkv_pool* pool, int64_t seq_id, int32_t* out) {
  if (!pool || !out) return fail(PKV_ERR_INVALID_ARG, "pkv_seq_num_blocks: NULL argument");
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end())
    return fail(PKV_ERR_NOT_FOUND, "pkv_seq_num_blocks: unknown sequence " + std::to_string(seq_id));
  *out = static_cast<int32_t>(it->second.size());
  return ok();
}

int pkv_build_block_table(const pkv_pool* pool, const int64_t* seq_ids, int32_t batch,
                          int32_t max_blocks_per_seq, int32_t* out) {
  if (!pool || (batch > 0 && (!seq_ids || !out)))
    return fail(PKV_ERR_INVALID_ARG, "pkv_build_block_table: NULL argument");
  if (batch < 0 || max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARG, "pkv_build_block_table: bad batch or max_blocks_per_seq");
  for (int32_t b = 0; b < batch; ++b) {
    auto it = pool->seqs.find(seq_ids[b]);
    if (it != pool->seqs.end() && static_cast<int64_t>(it->second.size()) > max_blocks_per_seq)
      return fail(PKV_ERR_INVALID_ARG, "pkv_build_block_table: sequence " +
                                           std::to_string(seq_ids[b]) +
                                           " has more blocks than max_blocks_per_seq");
  }
  for (int32_t b = 0; b < batch; ++b) {
    int32_t* row = out + static_cast<int64_t>(b) * max_blocks_per_seq;
    std::fill(row, row + max_blocks_per_seq, -1);
    auto it = pool->seqs.find(seq_ids[b]);
    if (it != pool->seqs.end()) std::copy(it->second.begin(), it->second.end(), row);
  }
  return ok();
}

int64_t pkv_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t n_items) {
  if (batch < 0 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1 || n_items < 1 ||
      n_q_heads % n_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_workspace_bytes: bad argument");
  const int64_t group = n_q_heads / n_kv_heads;
  return pkv::decode_workspace_end(batch, group, n_kv_heads, head_dim, n_items);
}

int pkv_decode_plan(const int32_t* seq_lens, int32_t batch, int32_t n_kv_heads,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t n_items,
                    int32_t min_chunk_pages, int32_t* chunk_pages, int32_t* first_chunk,
                    int32_t* last_chunk) {
  if ((batch > 0 && !seq_lens) || !chunk_pages || batch < 0 || n_kv_heads < 1 ||
      max_blocks_per_seq < 1 || n_items < 1)
    return fail(PKV_ERR_INVALID_ARG, "pkv_decode_plan: bad argument");
  if (block_size != pkv::kBlock)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_decode_plan: block_size must be 16");
  int min_chunk = min_chunk_pages;
  if (min_chunk < 1) return fail(PKV_ERR_INVALID_ARG, "pkv_decode_plan: min_chunk_pages must be resolved (>= 1)");
  std::vector<int64_t> prefix(batch + 1, 0);
  for (int32_t b = 0; b < batch; ++b)
    prefix[b + 1] = prefix[b] + pkv::pages_of_len(seq_lens[b], max_blocks_per_seq);
  int64_t total = static_cast<int64_t>(n_kv_heads) * prefix[batch];
  int C = pkv::chunk_pages(total, n_items, min_chunk);
  *chunk_pages = C;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t n = prefix[b + 1] - prefix[b];
    for (int32_t h = 0; h < n_kv_heads; ++h) {
      int64_t idx = static_cast<int64_t>(b) * n_kv_heads + h;
      int64_t start = n_kv_heads * prefix[b] + h * n;
      int32_t f = n ? static_cast<int32_t>(start / C) : -1;
      int32_t l = n ? static_cast<int32_t>((start + n - 1) / C) : -1;
      if (first_chunk) first_chunk[idx] = f;
      if (last_chunk) last_chunk[idx] = l;
    }
  }
  return ok();
}

}  // extern "C"
