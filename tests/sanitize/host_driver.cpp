// Host-only driver for the library's host code (page pool, block tables,
// byte accounting, split plan), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Exercises the
// error paths and a seeded random schedule of reserve / fork / copy-on-write /
// release against a shadow model of the pool kept here, and exits non-zero
// on the first mismatch; the sanitizers abort on any memory or UB error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <map>
#include <random>
#include <vector>

#include "pkv.h"

static int g_checks = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, #cond, pkv_last_error()); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

static void status_and_bytes() {
  const int codes[] = {PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_OUT_OF_PAGES,
                       PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_ERR_NOT_FOUND, PKV_ERR_EXISTS, 12345};
  for (int c : codes) CHECK(pkv_status_string(c) != nullptr && std::strlen(pkv_status_string(c)) > 0);
  CHECK(std::strlen(pkv_version()) > 0);
  // 2 (K and V) x 32 layers x 32 heads x 128 features x 2 bytes per token
  CHECK(pkv_kv_bytes_per_token(32, 32, 128, 2) == 524288u);
  CHECK(pkv_kv_cache_bytes(32, 8, 128, 4096, 16, 2) == 2ull * 32 * 8 * 128 * 4096 * 16 * 2);
  CHECK(pkv_kv_cache_bytes(-1, 8, 128, 1, 1, 2) == 0u);
}

static void pool_errors() {
  pkv_pool* p = reinterpret_cast<pkv_pool*>(0x1);
  CHECK(pkv_pool_create(4, nullptr, nullptr) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_pool_create(0, nullptr, &p) == PKV_ERR_INVALID_ARG && p == nullptr);
  CHECK(std::strlen(pkv_last_error()) > 0);
  const int32_t dup[4] = {0, 1, 1, 3}, out_of_range[4] = {0, 1, 2, 4};
  CHECK(pkv_pool_create(4, dup, &p) == PKV_ERR_INVALID_ARG && p == nullptr);
  CHECK(pkv_pool_create(4, out_of_range, &p) == PKV_ERR_INVALID_ARG && p == nullptr);
  const int32_t order[4] = {3, 1, 0, 2};
  CHECK(pkv_pool_create(4, order, &p) == PKV_OK && p != nullptr);
  CHECK(std::strlen(pkv_last_error()) == 0);
  int32_t n_new = -7;
  CHECK(pkv_seq_reserve(p, 10, 33, 16, &n_new) == PKV_OK && n_new == 3);
  int32_t row[4];
  const int64_t id = 10;
  CHECK(pkv_build_block_table(p, &id, 1, 4, row) == PKV_OK);
  CHECK(row[0] == 3 && row[1] == 1 && row[2] == 0 && row[3] == -1);   // pages taken in free order
  CHECK(pkv_seq_reserve(p, 11, 40, 16, &n_new) == PKV_ERR_OUT_OF_PAGES && n_new == 0);
  CHECK(pkv_pool_num_free(p) == 1);                                    // a failed reserve takes nothing
  CHECK(pkv_seq_reserve(p, 10, -1, 16, nullptr) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_seq_reserve(p, 10, 1, 0, nullptr) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_seq_reserve(nullptr, 10, 1, 16, nullptr) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_seq_release(p, 99) == PKV_ERR_NOT_FOUND);
  CHECK(pkv_seq_fork(p, 99, 100) == PKV_ERR_NOT_FOUND);
  CHECK(pkv_seq_fork(p, 10, 10) == PKV_ERR_EXISTS);
  int32_t nb = -1;
  CHECK(pkv_seq_num_blocks(p, 99, &nb) == PKV_ERR_NOT_FOUND);
  CHECK(pkv_seq_num_blocks(p, 10, &nb) == PKV_OK && nb == 3);
  CHECK(pkv_build_block_table(p, &id, 1, 2, row) == PKV_ERR_INVALID_ARG);   // 3 blocks do not fit 2
  CHECK(pkv_build_block_table(p, &id, -1, 4, row) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_build_block_table(p, nullptr, 0, 4, nullptr) == PKV_OK);
  int32_t src = 5, dst = 5;
  CHECK(pkv_seq_reserve_for_write(p, 10, -1, 16, &src, &dst) == PKV_ERR_INVALID_ARG && src == -1 && dst == -1);
  // copy-on-write of a shared block with one page free, then none left
  CHECK(pkv_seq_fork(p, 10, 20) == PKV_OK);
  CHECK(pkv_seq_reserve_for_write(p, 20, 20, 16, &src, &dst) == PKV_OK && src == 1 && dst == 2);
  CHECK(pkv_pool_num_free(p) == 0);
  CHECK(pkv_seq_reserve_for_write(p, 20, 5, 16, &src, &dst) == PKV_ERR_OUT_OF_PAGES && src == -1);
  CHECK(pkv_seq_release(p, 10) == PKV_OK);                   // pages 3 and 0 still held by 20, 1 freed
  CHECK(pkv_pool_num_free(p) == 1);
  CHECK(pkv_seq_release(p, 20) == PKV_OK);
  CHECK(pkv_pool_num_free(p) == 4);
  pkv_pool_destroy(p);
  pkv_pool_destroy(nullptr);
}

// Seeded schedule of pool calls against a shadow model of each sequence's
// token count: after every call, each sequence has exactly the blocks its
// tokens need, its block table row lists valid pages (then -1), and the free
// pages are exactly those no sequence's table holds.
static void pool_random(uint32_t seed) {
  const int32_t kPages = 64, kBs = 16;
  std::mt19937 rng(seed);
  std::vector<int32_t> order(kPages);
  for (int32_t i = 0; i < kPages; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_pool* p = nullptr;
  CHECK(pkv_pool_create(kPages, order.data(), &p) == PKV_OK);
  std::map<int64_t, int64_t> tokens;
  int64_t next_id = 1;
  for (int step = 0; step < 4000; ++step) {
    const int op = static_cast<int>(rng() % 5);
    const bool have = !tokens.empty();
    auto pick = [&]() {
      auto it = tokens.begin();
      std::advance(it, rng() % tokens.size());
      return it->first;
    };
    if (op == 0 || !have) {                            // a new sequence
      const int64_t id = next_id++, n = rng() % 80;
      int32_t n_new = -1;
      const int st = pkv_seq_reserve(p, id, n, kBs, &n_new);
      if (st == PKV_OK) {
        CHECK(n_new == static_cast<int32_t>((n + kBs - 1) / kBs));
        tokens[id] = n;
      } else {
        CHECK(st == PKV_ERR_OUT_OF_PAGES && n_new == 0);
      }
    } else if (op == 1) {                              // grow by a few tokens
      const int64_t id = pick();
      const int64_t n = tokens[id] + static_cast<int64_t>(rng() % 40);
      const int st = pkv_seq_reserve(p, id, n, kBs, nullptr);
      if (st == PKV_OK) tokens[id] = std::max(tokens[id], n);
      else CHECK(st == PKV_ERR_OUT_OF_PAGES);
    } else if (op == 2) {                              // fork
      const int64_t id = pick(), child = next_id++;
      CHECK(pkv_seq_fork(p, id, child) == PKV_OK);
      tokens[child] = tokens[id];
    } else if (op == 3) {                              // write a token (copy-on-write when shared)
      const int64_t id = pick();
      const int64_t pos = tokens[id] > 0 && rng() % 2 ? static_cast<int64_t>(rng() % tokens[id]) : tokens[id];
      int32_t src = 0, dst = 0;
      const int st = pkv_seq_reserve_for_write(p, id, pos, kBs, &src, &dst);
      if (st == PKV_OK) {
        tokens[id] = std::max(tokens[id], pos + 1);
        CHECK((src == -1 && dst == -1) || (src >= 0 && dst >= 0 && src != dst));
      } else {
        CHECK(st == PKV_ERR_OUT_OF_PAGES && src == -1 && dst == -1);
      }
    } else {                                           // release
      const int64_t id = pick();
      CHECK(pkv_seq_release(p, id) == PKV_OK);
      tokens.erase(id);
    }
    // the invariants, from the block tables
    std::vector<int32_t> refs(kPages, 0);
    for (auto& kv : tokens) {
      const int64_t id = kv.first;
      int32_t nb = -1;
      CHECK(pkv_seq_num_blocks(p, id, &nb) == PKV_OK);
      CHECK(nb == static_cast<int32_t>((tokens[id] + kBs - 1) / kBs));
      std::vector<int32_t> row(static_cast<size_t>(std::max(nb, 1)));
      CHECK(pkv_build_block_table(p, &id, 1, static_cast<int32_t>(row.size()), row.data()) == PKV_OK);
      for (int32_t j = 0; j < nb; ++j) {
        CHECK(row[j] >= 0 && row[j] < kPages);
        ++refs[row[j]];
      }
      for (int32_t j = nb; j < static_cast<int32_t>(row.size()); ++j) CHECK(row[j] == -1);
    }
    int32_t used = 0;
    for (int32_t r : refs) used += r > 0;
    CHECK(pkv_pool_num_free(p) == kPages - used);
  }
  // Two sequences never share a page that one of them may write: after a
  // copy-on-write the writer's block is its own.
  for (auto& kv : tokens) {
    if (kv.second == 0) continue;
    int32_t src = 0, dst = 0;
    const int st = pkv_seq_reserve_for_write(p, kv.first, kv.second - 1, kBs, &src, &dst);
    CHECK(st == PKV_OK || st == PKV_ERR_OUT_OF_PAGES);
  }
  for (auto& kv : tokens) CHECK(pkv_seq_release(p, kv.first) == PKV_OK);
  CHECK(pkv_pool_num_free(p) == kPages);
  pkv_pool_destroy(p);
}

static void plan_checks() {
  int32_t C = -1;
  CHECK(pkv_decode_plan(nullptr, 1, 8, 16, 4, 8, 1, &C, nullptr, nullptr) == PKV_ERR_INVALID_ARG);
  const int32_t lens[5] = {0, 1, 17, 300, 64};
  CHECK(pkv_decode_plan(lens, 5, 8, 32, 32, 8, 1, &C, nullptr, nullptr) == PKV_ERR_UNSUPPORTED);
  CHECK(pkv_decode_plan(lens, 5, 8, 16, 32, 8, 0, &C, nullptr, nullptr) == PKV_ERR_INVALID_ARG);
  for (int32_t n_items : {1, 7, 64, 1000}) {
    for (int32_t min_chunk : {1, 4, 32}) {
      std::vector<int32_t> first(5 * 8), last(5 * 8);
      CHECK(pkv_decode_plan(lens, 5, 8, 16, 32, n_items, min_chunk, &C, first.data(), last.data()) == PKV_OK);
      CHECK(C >= min_chunk);
      int64_t start = 0;
      for (int b = 0; b < 5; ++b) {
        const int64_t n = (lens[b] + 15) / 16;
        for (int h = 0; h < 8; ++h) {
          const int i = b * 8 + h;
          if (n == 0) {
            CHECK(first[i] == -1 && last[i] == -1);
            continue;
          }
          CHECK(first[i] == start / C && last[i] == (start + n - 1) / C && first[i] <= last[i]);
          start += n;
        }
      }
      CHECK((start + C - 1) / C <= std::max<int64_t>(n_items, 1) || C == min_chunk);
    }
  }
  CHECK(pkv_decode_workspace_bytes(4, 32, 8, 128, 0) < 0);
  CHECK(pkv_decode_workspace_bytes(4, 30, 8, 128, 16) < 0);
  const int64_t w1 = pkv_decode_workspace_bytes(4, 32, 8, 128, 16), w2 = pkv_decode_workspace_bytes(4, 32, 8, 128, 64);
  CHECK(w1 > 0 && w2 > w1);
}

int main() {
  status_and_bytes();
  pool_errors();
  for (uint32_t seed : {1u, 2u, 3u}) pool_random(seed);
  plan_checks();
  std::printf("host driver: ok (%d checks)\n", g_checks);
  return 0;
}
