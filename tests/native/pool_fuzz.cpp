// Seeded operation sequence over the host block pool and its prefix cache, built with
// -fsanitize=address,undefined by tests/test_abi.py.  Checks pool invariants after every
// operation; prints "ok" on success.
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

// Token of position pos of a sequence following document d (three documents), or a divergent one.
static int32_t doc_token(int32_t d, int32_t pos, bool diverge) {
  if (diverge) return 1000 + static_cast<int32_t>(next_u32() % 50);
  return static_cast<int32_t>((d * 7919u + static_cast<uint32_t>(pos) * 104729u) % 40u);
}

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 10000;
  const int32_t N = 97;
  pkv_pool* pool = nullptr;
  REQUIRE(pkv_pool_create(N, 16, nullptr, &pool) == PKV_OK);
  std::vector<int32_t> live;
  std::vector<std::vector<int32_t>> toks;  // per sequence id: its token ids
  std::vector<int32_t> doc;
  auto track = [&](int32_t s) {
    if (static_cast<size_t>(s) >= toks.size()) {
      toks.resize(s + 1);
      doc.resize(s + 1, 0);
    }
  };
  auto allocatable = [&]() {
    int32_t f = 0, e = 0;
    pkv_pool_num_free(pool, &f);
    pkv_prefix_evictable(pool, nullptr, 0, &e);  // capacity 0: reports the length (error if > 0)
    return f + e;
  };
  std::vector<int32_t> slots(200);
  int64_t hits = 0, evictions = 0;
  for (int it = 0; it < steps; ++it) {
    const uint32_t r = next_u32() % 100;
    if (r < 10 || live.empty()) {
      int32_t s;
      REQUIRE(pkv_seq_new(pool, &s) == PKV_OK);
      track(s);
      toks[s].clear();
      doc[s] = static_cast<int32_t>(next_u32() % 3);
      live.push_back(s);
    } else if (r < 22) {
      // lookup: document prefix, possibly diverging, then a few random tokens
      const int32_t d = static_cast<int32_t>(next_u32() % 3);
      const int32_t cut = static_cast<int32_t>(next_u32() % 90);
      std::vector<int32_t> t;
      for (int32_t i = 0; i < cut; ++i) t.push_back(doc_token(d, i, next_u32() % 50 == 0));
      const int32_t extra = static_cast<int32_t>(next_u32() % 20);
      for (int32_t i = 0; i < extra; ++i) t.push_back(doc_token(d, 0, true));
      int32_t s, n;
      REQUIRE(pkv_prefix_lookup(pool, t.data(), static_cast<int32_t>(t.size()), &s, &n) == PKV_OK);
      REQUIRE(n % 16 == 0 && n <= static_cast<int32_t>(t.size()));
      hits += n > 0;
      track(s);
      toks[s].assign(t.begin(), t.begin() + n);
      doc[s] = d;
      live.push_back(s);
    } else if (r < 28) {
      int32_t c;
      const int32_t par = live[next_u32() % live.size()];
      REQUIRE(pkv_seq_fork(pool, par, &c) == PKV_OK);
      track(c);
      toks[c] = toks[par];
      doc[c] = doc[par];
      live.push_back(c);
    } else if (r < 45) {
      const size_t i = next_u32() % live.size();
      const int32_t s = live[i];
      if (next_u32() % 10 < 7) {
        int32_t added = -1;
        REQUIRE(pkv_prefix_insert(pool, s, toks[s].data(), static_cast<int32_t>(toks[s].size()), &added) == PKV_OK);
        REQUIRE(added >= 0);
      }
      REQUIRE(pkv_seq_free(pool, s) == PKV_OK);
      REQUIRE(pkv_seq_free(pool, s) == PKV_EINVAL);  // double free is rejected
      REQUIRE(pkv_prefix_insert(pool, s, toks[s].data(), 0, nullptr) == PKV_EINVAL);
      live.erase(live.begin() + static_cast<long>(i));
    } else if (r < 52) {
      const int32_t s = live[next_u32() % live.size()];
      REQUIRE(pkv_prefix_insert(pool, s, toks[s].data(), static_cast<int32_t>(toks[s].size()), nullptr) == PKV_OK);
    } else {
      const int32_t s = live[next_u32() % live.size()];
      const int32_t n = static_cast<int32_t>(next_u32() % 150);
      int32_t cow[2], ncow = 0, need = 0, free_before = 0;
      REQUIRE(pkv_seq_blocks_needed(pool, s, n, &need) == PKV_OK);
      REQUIRE(pkv_pool_num_free(pool, &free_before) == PKV_OK);
      const int32_t alloc_before = allocatable();
      const int st = pkv_seq_append(pool, s, n, slots.data(), cow, &ncow);
      const int32_t alloc_after = allocatable();
      if (st == PKV_OK) {
        REQUIRE(alloc_before - alloc_after == need);
        evictions += need > free_before;
        const bool diverge = next_u32() % 4 == 0;
        for (int32_t i = 0; i < n; ++i)
          toks[s].push_back(doc_token(doc[s], static_cast<int32_t>(toks[s].size()), diverge));
      } else {
        REQUIRE(st == PKV_ENOMEM && need > alloc_before && alloc_after == alloc_before);
      }
    }
    // invariants: refcounts equal table references; every block is referenced, free or evictable
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
    std::vector<int32_t> fl(N), ev(N);
    int32_t nfree = 0, nev = 0, nreg = 0;
    REQUIRE(pkv_pool_free_list(pool, fl.data(), N, &nfree) == PKV_OK);
    REQUIRE(pkv_prefix_evictable(pool, ev.data(), N, &nev) == PKV_OK);
    REQUIRE(pkv_prefix_num_registered(pool, &nreg) == PKV_OK);
    REQUIRE(nev <= nreg && nreg <= N);
    std::vector<int> idle(N, 0);
    for (int32_t i = 0; i < nfree; ++i) idle[fl[i]] += 1;
    for (int32_t i = 0; i < nev; ++i) idle[ev[i]] += 1;
    for (int32_t b = 0; b < N; ++b) {
      int32_t rc;
      REQUIRE(pkv_pool_refcount(pool, b, &rc) == PKV_OK);
      REQUIRE(rc == ref[b]);
      REQUIRE((rc == 0) == (idle[b] == 1));
      REQUIRE(idle[b] <= 1);
    }
  }
  for (int32_t s : live) REQUIRE(pkv_seq_free(pool, s) == PKV_OK);
  REQUIRE(allocatable() == N);
  pkv_pool_destroy(pool);
  REQUIRE(hits > 0 && evictions > 0);
  std::printf("ok (%lld prefix hits, %lld appends that evicted)\n", static_cast<long long>(hits),
              static_cast<long long>(evictions));
  return 0;
}
