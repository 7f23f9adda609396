// Seeded operation sequence over the host block pool, built with -fsanitize=address,undefined by
// tests/test_abi.py.  Checks pool invariants after every operation; prints "ok" on success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pagedkv.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return static_cast<uint32_t>(g_state >> 33);
}

#define REQUIRE(c)                                              \
  do {                                                          \
    if (!(c)) {                                                 \
      std::printf("FAILED %s at line %d\n", #c, __LINE__);     \
      return 1;                                                 \
    }                                                           \
  } while (0)

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 10000;
  const int32_t N = 97;
  pkv_pool* pool = nullptr;
  REQUIRE(pkv_pool_create(N, 16, nullptr, &pool) == PKV_OK);
  std::vector<int32_t> live;
  std::vector<int32_t> slots(200);
  for (int it = 0; it < steps; ++it) {
    const uint32_t r = next_u32() % 100;
    if (r < 12 || live.empty()) {
      int32_t s;
      REQUIRE(pkv_seq_new(pool, &s) == PKV_OK);
      live.push_back(s);
    } else if (r < 20) {
      int32_t c;
      REQUIRE(pkv_seq_fork(pool, live[next_u32() % live.size()], &c) == PKV_OK);
      live.push_back(c);
    } else if (r < 32) {
      const size_t i = next_u32() % live.size();
      REQUIRE(pkv_seq_free(pool, live[i]) == PKV_OK);
      REQUIRE(pkv_seq_free(pool, live[i]) == PKV_EINVAL);  // double free is rejected
      live.erase(live.begin() + static_cast<long>(i));
    } else {
      const int32_t s = live[next_u32() % live.size()];
      const int32_t n = static_cast<int32_t>(next_u32() % 150);
      int32_t cow[2], ncow = 0, need = 0, free_before = 0, free_after = 0;
      REQUIRE(pkv_seq_blocks_needed(pool, s, n, &need) == PKV_OK);
      REQUIRE(pkv_pool_num_free(pool, &free_before) == PKV_OK);
      const int st = pkv_seq_append(pool, s, n, slots.data(), cow, &ncow);
      REQUIRE(pkv_pool_num_free(pool, &free_after) == PKV_OK);
      if (st == PKV_OK) {
        REQUIRE(free_before - free_after == need);
      } else {
        REQUIRE(st == PKV_ENOMEM && need > free_before && free_after == free_before);
      }
    }
    // invariants: refcounts equal table references; free list disjoint from held blocks
    std::vector<int32_t> ref(N, 0);
    int32_t maxb = 0;
    for (int32_t s : live) {
      int32_t nb;
      REQUIRE(pkv_seq_num_blocks(pool, s, &nb) == PKV_OK);
      if (nb > maxb) maxb = nb;
    }
    if (!live.empty() && maxb > 0) {
      std::vector<int32_t> tables(live.size() * static_cast<size_t>(maxb));
      REQUIRE(pkv_build_block_tables(pool, live.data(), static_cast<int32_t>(live.size()), maxb, tables.data(),
                                     nullptr) == PKV_OK);
      for (int32_t b : tables)
        if (b >= 0) ref[b] += 1;
    }
    std::vector<int32_t> fl(N);
    int32_t nfree = 0;
    REQUIRE(pkv_pool_free_list(pool, fl.data(), N, &nfree) == PKV_OK);
    std::vector<int> in_free(N, 0);
    for (int32_t i = 0; i < nfree; ++i) in_free[fl[i]] += 1;
    for (int32_t b = 0; b < N; ++b) {
      int32_t rc;
      REQUIRE(pkv_pool_refcount(pool, b, &rc) == PKV_OK);
      REQUIRE(rc == ref[b]);
      REQUIRE((rc == 0) == (in_free[b] == 1));
      REQUIRE(in_free[b] <= 1);
    }
  }
  for (int32_t s : live) REQUIRE(pkv_seq_free(pool, s) == PKV_OK);
  int32_t nfree = 0;
  REQUIRE(pkv_pool_num_free(pool, &nfree) == PKV_OK && nfree == N);
  pkv_pool_destroy(pool);
  std::printf("ok\n");
  return 0;
}
