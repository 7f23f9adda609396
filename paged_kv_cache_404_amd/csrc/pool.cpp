// Host block pool, block-table and slot-mapping builders (host-only; builds with g++ or hipcc).
//
// [Serving] "Production Serving: Continuous Batching and PagedAttention", The Build, Step 4:
// physical block ids live on a free list; allocation takes the id at the end of the list and
// fails on an empty list; a freed id goes back on the end; a sequence owns a block table
// (logical block -> physical block) and a token count, and the token at position pos opens a
// new block when pos % block_size == 0.  Copy-on-write sharing per [Chapter] "Continuous
// batching and PagedAttention", "PagedAttention: KV cache memory" and [Notes] "Continuous
// batching and PagedAttention: serving many users from one GPU", "Fragmentation:
// PagedAttention": blocks are shared until a sequence writes into one; the writer then gets a
// private copy.  Exact rules (fork, copy-on-write trigger, all-or-nothing append, free order,
// sequence ids) are stated in include/pagedkv.h.
//
// Prefix cache per [Serving] The Build, Step 8 ("Prefix caching"): the longest block-aligned
// prefix of a request already held in blocks is shared, one reference per block.  The pages key a
// dictionary by whole token tuples (memory quadratic in the prefix length); here each registered
// full block is a node of a trie keyed by (parent node, the block's own tokens), so a lookup is
// one exact hash probe per block.  Registered blocks with no reference wait on an LRU list and
// are evicted, with every registered block below them, when the free list runs dry.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <list>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pkv::fail;

namespace {

// Trie key of a registered block: its parent's block id (-1 for a first block) and its tokens.
struct PrefixKey {
  int32_t parent;
  std::vector<int32_t> tokens;
  bool operator==(const PrefixKey& o) const { return parent == o.parent && tokens == o.tokens; }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = 1469598103934665603ull ^ static_cast<uint32_t>(k.parent);
    for (int32_t t : k.tokens) h = (h ^ static_cast<uint32_t>(t)) * 1099511628211ull;
    return static_cast<size_t>(h ^ (h >> 29));
  }
};

}  // namespace

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // next allocation takes back()
  std::vector<int32_t> refcnt;     // per physical block
  std::vector<std::vector<int32_t>> tables;
  std::vector<int32_t> lens;
  std::vector<uint8_t> live;
  // prefix cache
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> prefix;  // key -> registered block
  std::vector<uint8_t> registered;                                // per block
  std::vector<int32_t> parent;                                    // trie parent of a registered block
  std::vector<std::vector<int32_t>> key_tokens;                   // its tokens (to rebuild the key)
  std::vector<std::vector<int32_t>> children;                     // registered blocks one level below
  std::list<int32_t> lru;                                         // registered, no reference; front = oldest
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<uint8_t> in_lru;
  std::vector<int64_t> lru_stamp;  // release order of blocks on the LRU
  int64_t clock = 0;
  int32_t num_registered = 0;
};

namespace {

bool seq_ok(const pkv_pool* p, int32_t seq) {
  return p && seq >= 0 && seq < static_cast<int32_t>(p->live.size()) && p->live[seq];
}

void lru_remove(pkv_pool* p, int32_t b) {
  p->lru.erase(p->lru_pos[b]);
  p->in_lru[b] = 0;
}

// Unregister the LRU head and every registered block below it; the ones without references
// leave the LRU for the free list, least recently released first.  Returns the head.
int32_t evict(pkv_pool* p) {
  const int32_t b = p->lru.front();
  lru_remove(p, b);
  if (p->parent[b] >= 0) {
    std::vector<int32_t>& sib = p->children[p->parent[b]];
    sib.erase(std::find(sib.begin(), sib.end(), b));
  }
  std::vector<int32_t> stack{b}, dropped;
  while (!stack.empty()) {
    const int32_t x = stack.back();
    stack.pop_back();
    dropped.push_back(x);
    for (int32_t c : p->children[x]) stack.push_back(c);
    p->prefix.erase(PrefixKey{p->parent[x], p->key_tokens[x]});
    p->registered[x] = 0;
    p->parent[x] = -1;
    p->key_tokens[x].clear();
    p->children[x].clear();
    --p->num_registered;
  }
  std::vector<std::pair<int64_t, int32_t>> idle;
  for (int32_t x : dropped)
    if (p->in_lru[x]) idle.emplace_back(p->lru_stamp[x], x);
  std::sort(idle.begin(), idle.end());
  for (const auto& e : idle) {
    lru_remove(p, e.second);
    p->free_list.push_back(e.second);
  }
  return b;
}

int32_t take_block(pkv_pool* p) {
  int32_t b;
  if (!p->free_list.empty()) {
    b = p->free_list.back();
    p->free_list.pop_back();
  } else {
    b = evict(p);
  }
  p->refcnt[b] = 1;
  return b;
}

// Drop one reference; an unregistered block at zero goes back on the free list, a registered
// one is collected in `idle` for the LRU.
void drop_ref(pkv_pool* p, int32_t b, std::vector<int32_t>& idle) {
  if (--p->refcnt[b] != 0) return;
  if (p->registered[b])
    idle.push_back(b);
  else
    p->free_list.push_back(b);
}

// Blocks released together join the LRU deepest first (reverse table order), so that eviction
// shortens a registered prefix from its end.
void lru_push_released(pkv_pool* p, const std::vector<int32_t>& idle) {
  for (auto it = idle.rbegin(); it != idle.rend(); ++it) {
    const int32_t b = *it;
    p->lru.push_back(b);
    p->lru_pos[b] = std::prev(p->lru.end());
    p->in_lru[b] = 1;
    p->lru_stamp[b] = p->clock++;
  }
}

// Blocks an allocation can take: the free list plus the evictable registered blocks.
int64_t allocatable(const pkv_pool* p) {
  return static_cast<int64_t>(p->free_list.size()) + static_cast<int64_t>(p->lru.size());
}

int32_t lowest_free_id(pkv_pool* p) {
  for (size_t i = 0; i < p->live.size(); ++i)
    if (!p->live[i]) return static_cast<int32_t>(i);
  p->live.push_back(0);
  p->tables.emplace_back();
  p->lens.push_back(0);
  return static_cast<int32_t>(p->live.size() - 1);
}

// Blocks an append of n tokens takes: positions that start a block, plus one copy-on-write
// block when the first write lands in a shared, partially filled last block.
int64_t blocks_needed(const pkv_pool* p, int32_t seq, int32_t n) {
  const int64_t start = p->lens[seq];
  const int64_t bs = p->block_size;
  const int64_t end = start + n;
  // count multiples of bs in [start, end)
  int64_t need = (end + bs - 1) / bs - (start + bs - 1) / bs;
  if (n > 0 && start % bs != 0 && p->refcnt[p->tables[seq].back()] > 1) need += 1;
  return need;
}

int append_one(pkv_pool* p, int32_t seq, int32_t n, int32_t* slots_out, int32_t* cow_out, int32_t* n_cow) {
  if (!seq_ok(p, seq)) return fail(PKV_EINVAL, "pkv_seq_append: unknown sequence %d", seq);
  if (n < 0) return fail(PKV_EINVAL, "pkv_seq_append: negative token count %d", n);
  if (n > 0 && !slots_out) return fail(PKV_EINVAL, "pkv_seq_append: slots_out is NULL");
  if (static_cast<int64_t>(p->lens[seq]) + n > static_cast<int64_t>(INT32_MAX))
    return fail(PKV_EINVAL, "pkv_seq_append: sequence length overflows int32");
  const int64_t need = blocks_needed(p, seq, n);
  if (need > allocatable(p))
    return fail(PKV_ENOMEM, "pkv_seq_append: sequence %d needs %lld blocks, %lld free or evictable", seq,
                static_cast<long long>(need), static_cast<long long>(allocatable(p)));
  std::vector<int32_t>& table = p->tables[seq];
  const int32_t bs = p->block_size;
  int32_t cows = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = p->lens[seq];
    if (pos % bs == 0) {
      table.push_back(take_block(p));
    } else if (p->refcnt[table.back()] > 1) {
      const int32_t old_blk = table.back();
      const int32_t new_blk = take_block(p);
      p->refcnt[old_blk] -= 1;  // still held by another sequence, never reaches 0 here
      table.back() = new_blk;
      if (cow_out) {
        cow_out[2 * cows] = old_blk;
        cow_out[2 * cows + 1] = new_blk;
      }
      ++cows;
    }
    slots_out[i] = table[pos / bs] * bs + pos % bs;
    p->lens[seq] = pos + 1;
  }
  if (n_cow) *n_cow = cows;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_pool** out) {
  if (!out) return fail(PKV_EINVAL, "pkv_pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PKV_EINVAL, "pkv_pool_create: bad sizes num_blocks=%d block_size=%d", num_blocks, block_size);
  if (static_cast<int64_t>(num_blocks) * block_size > static_cast<int64_t>(INT32_MAX))
    return fail(PKV_EINVAL, "pkv_pool_create: num_blocks * block_size overflows int32 slots");
  pkv_pool* p = new pkv_pool;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refcnt.assign(num_blocks, 0);
  p->registered.assign(num_blocks, 0);
  p->parent.assign(num_blocks, -1);
  p->key_tokens.resize(num_blocks);
  p->children.resize(num_blocks);
  p->lru_pos.resize(num_blocks);
  p->in_lru.assign(num_blocks, 0);
  p->lru_stamp.assign(num_blocks, 0);
  p->free_list.resize(num_blocks);
  if (free_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return fail(PKV_EINVAL, "pkv_pool_create: free_order is not a permutation of 0..%d", num_blocks - 1);
      }
      seen[b] = 1;
      p->free_list[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_list[i] = i;
  }
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_pool_num_free(const pkv_pool* pool, int32_t* out) {
  if (!pool || !out) return fail(PKV_EINVAL, "pkv_pool_num_free: NULL argument");
  *out = static_cast<int32_t>(pool->free_list.size());
  return PKV_OK;
}

int pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "pkv_pool_free_list: NULL argument");
  const int32_t len = static_cast<int32_t>(pool->free_list.size());
  *n = len;
  if (len > 0 && (!out || capacity < len))
    return fail(PKV_EINVAL, "pkv_pool_free_list: capacity %d < %d", capacity, len);
  std::copy(pool->free_list.begin(), pool->free_list.end(), out);
  return PKV_OK;
}

int pkv_pool_refcount(const pkv_pool* pool, int32_t block, int32_t* out) {
  if (!pool || !out) return fail(PKV_EINVAL, "pkv_pool_refcount: NULL argument");
  if (block < 0 || block >= pool->num_blocks) return fail(PKV_EINVAL, "pkv_pool_refcount: block %d out of range", block);
  *out = pool->refcnt[block];
  return PKV_OK;
}

int pkv_seq_new(pkv_pool* pool, int32_t* seq_id) {
  if (!pool || !seq_id) return fail(PKV_EINVAL, "pkv_seq_new: NULL argument");
  const int32_t s = lowest_free_id(pool);
  pool->live[s] = 1;
  pool->tables[s].clear();
  pool->lens[s] = 0;
  *seq_id = s;
  return PKV_OK;
}

int pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* child) {
  if (!child) return fail(PKV_EINVAL, "pkv_seq_fork: child is NULL");
  if (!seq_ok(pool, parent)) return fail(PKV_EINVAL, "pkv_seq_fork: unknown sequence %d", parent);
  const int32_t c = lowest_free_id(pool);  // may grow the vectors: index, do not hold references
  pool->live[c] = 1;
  pool->tables[c] = pool->tables[parent];
  pool->lens[c] = pool->lens[parent];
  for (int32_t b : pool->tables[c]) pool->refcnt[b] += 1;
  *child = c;
  return PKV_OK;
}

int pkv_seq_blocks_needed(const pkv_pool* pool, int32_t seq, int32_t n, int32_t* out) {
  if (!out) return fail(PKV_EINVAL, "pkv_seq_blocks_needed: out is NULL");
  if (!seq_ok(pool, seq)) return fail(PKV_EINVAL, "pkv_seq_blocks_needed: unknown sequence %d", seq);
  if (n < 0) return fail(PKV_EINVAL, "pkv_seq_blocks_needed: negative token count");
  const int64_t need = blocks_needed(pool, seq, n);
  *out = need > INT32_MAX ? INT32_MAX : static_cast<int32_t>(need);
  return PKV_OK;
}

int pkv_seq_append(pkv_pool* pool, int32_t seq, int32_t n, int32_t* slots_out, int32_t* cow_src_dst_out,
                   int32_t* n_cow) {
  return append_one(pool, seq, n, slots_out, cow_src_dst_out, n_cow);
}

int pkv_seqs_append(pkv_pool* pool, const int32_t* seqs, const int32_t* counts, int32_t n, int32_t* slots_out,
                    int32_t* cow_out, int32_t* n_cow, int32_t* done) {
  if (!pool || (n > 0 && (!seqs || !counts)) || !n_cow || !done)
    return fail(PKV_EINVAL, "pkv_seqs_append: NULL argument");
  *n_cow = 0;
  *done = 0;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = 0;
    int32_t pair[2];
    const int st = append_one(pool, seqs[i], counts[i], slots_out ? slots_out + off : nullptr, pair, &c);
    if (st != PKV_OK) {
      *done = i;
      return st;
    }
    if (c) {
      if (cow_out) {
        cow_out[2 * *n_cow] = pair[0];
        cow_out[2 * *n_cow + 1] = pair[1];
      }
      *n_cow += 1;
    }
    off += counts[i];
  }
  *done = n;
  return PKV_OK;
}

int pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!seq_ok(pool, seq)) return fail(PKV_EINVAL, "pkv_seq_free: unknown sequence %d", seq);
  std::vector<int32_t> idle;
  for (int32_t b : pool->tables[seq]) drop_ref(pool, b, idle);
  lru_push_released(pool, idle);
  pool->tables[seq].clear();
  pool->lens[seq] = 0;
  pool->live[seq] = 0;
  return PKV_OK;
}

int pkv_seq_len(const pkv_pool* pool, int32_t seq, int32_t* out) {
  if (!out) return fail(PKV_EINVAL, "pkv_seq_len: out is NULL");
  if (!seq_ok(pool, seq)) return fail(PKV_EINVAL, "pkv_seq_len: unknown sequence %d", seq);
  *out = pool->lens[seq];
  return PKV_OK;
}

int pkv_seq_num_blocks(const pkv_pool* pool, int32_t seq, int32_t* out) {
  if (!out) return fail(PKV_EINVAL, "pkv_seq_num_blocks: out is NULL");
  if (!seq_ok(pool, seq)) return fail(PKV_EINVAL, "pkv_seq_num_blocks: unknown sequence %d", seq);
  *out = static_cast<int32_t>(pool->tables[seq].size());
  return PKV_OK;
}

int pkv_build_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                           int32_t* tables_out, int32_t* lens_out) {
  if (!pool || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || (max_blocks > 0 && !tables_out))))
    return fail(PKV_EINVAL, "pkv_build_block_tables: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    if (!seq_ok(pool, seqs[i])) return fail(PKV_EINVAL, "pkv_build_block_tables: unknown sequence %d", seqs[i]);
    if (static_cast<int32_t>(pool->tables[seqs[i]].size()) > max_blocks)
      return fail(PKV_EINVAL, "pkv_build_block_tables: sequence %d has %zu blocks > max_blocks %d", seqs[i],
                  pool->tables[seqs[i]].size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = pool->tables[seqs[i]];
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks, -1);
    if (lens_out) lens_out[i] = pool->lens[seqs[i]];
  }
  return PKV_OK;
}

int pkv_build_slot_mapping(const pkv_pool* pool, const int32_t* seqs, const int32_t* starts,
                           const int32_t* counts, int32_t n, int32_t* slots_out) {
  if (!pool || n < 0 || (n > 0 && (!seqs || !starts || !counts)))
    return fail(PKV_EINVAL, "pkv_build_slot_mapping: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    if (!seq_ok(pool, seqs[i])) return fail(PKV_EINVAL, "pkv_build_slot_mapping: unknown sequence %d", seqs[i]);
    if (starts[i] < 0 || counts[i] < 0 ||
        static_cast<int64_t>(starts[i]) + counts[i] > static_cast<int64_t>(pool->lens[seqs[i]]))
      return fail(PKV_EINVAL, "pkv_build_slot_mapping: positions [%d, %d) not stored in sequence %d", starts[i],
                  starts[i] + counts[i], seqs[i]);
    if (counts[i] > 0 && !slots_out) return fail(PKV_EINVAL, "pkv_build_slot_mapping: slots_out is NULL");
  }
  const int32_t bs = pool->block_size;
  int64_t off = 0;
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = pool->tables[seqs[i]];
    for (int32_t k = 0; k < counts[i]; ++k) {
      const int32_t pos = starts[i] + k;
      slots_out[off++] = t[pos / bs] * bs + pos % bs;
    }
  }
  return PKV_OK;
}

int pkv_prefix_insert(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens, int32_t* n_registered) {
  if (!seq_ok(pool, seq)) return fail(PKV_EINVAL, "pkv_prefix_insert: unknown sequence %d", seq);
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_EINVAL, "pkv_prefix_insert: bad tokens");
  const int32_t bs = pool->block_size;
  const int32_t nfull = std::min(n_tokens, pool->lens[seq]) / bs;
  int32_t par = -1, added = 0;
  for (int32_t k = 0; k < nfull; ++k) {
    PrefixKey key{par, std::vector<int32_t>(tokens + static_cast<int64_t>(k) * bs, tokens + static_cast<int64_t>(k + 1) * bs)};
    auto it = pool->prefix.find(key);
    if (it != pool->prefix.end()) {
      par = it->second;
      continue;
    }
    const int32_t b = pool->tables[seq][k];
    if (pool->registered[b]) break;  // already registered under another prefix
    pool->registered[b] = 1;
    pool->parent[b] = par;
    pool->key_tokens[b] = key.tokens;
    if (par >= 0) pool->children[par].push_back(b);
    pool->prefix.emplace(std::move(key), b);
    ++pool->num_registered;
    ++added;
    par = b;
  }
  if (n_registered) *n_registered = added;
  return PKV_OK;
}

int pkv_prefix_lookup(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* seq_out, int32_t* n_matched) {
  if (!pool || !seq_out || !n_matched) return fail(PKV_EINVAL, "pkv_prefix_lookup: NULL argument");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens)) return fail(PKV_EINVAL, "pkv_prefix_lookup: bad tokens");
  const int32_t bs = pool->block_size;
  std::vector<int32_t> match;
  PrefixKey key{-1, std::vector<int32_t>(bs)};
  for (int32_t k = 0; k < n_tokens / bs; ++k) {
    std::copy(tokens + static_cast<int64_t>(k) * bs, tokens + static_cast<int64_t>(k + 1) * bs, key.tokens.begin());
    auto it = pool->prefix.find(key);
    if (it == pool->prefix.end()) break;
    match.push_back(it->second);
    key.parent = it->second;
  }
  const int32_t s = lowest_free_id(pool);
  pool->live[s] = 1;
  for (int32_t b : match) {
    if (pool->refcnt[b] == 0) lru_remove(pool, b);
    pool->refcnt[b] += 1;
  }
  pool->tables[s] = match;
  pool->lens[s] = static_cast<int32_t>(match.size()) * bs;
  *seq_out = s;
  *n_matched = pool->lens[s];
  return PKV_OK;
}

int pkv_prefix_evictable(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "pkv_prefix_evictable: NULL argument");
  const int32_t len = static_cast<int32_t>(pool->lru.size());
  *n = len;
  if (len > 0 && (!out || capacity < len))
    return fail(PKV_EINVAL, "pkv_prefix_evictable: capacity %d < %d", capacity, len);
  std::copy(pool->lru.begin(), pool->lru.end(), out);
  return PKV_OK;
}

int pkv_prefix_num_registered(const pkv_pool* pool, int32_t* out) {
  if (!pool || !out) return fail(PKV_EINVAL, "pkv_prefix_num_registered: NULL argument");
  *out = pool->num_registered;
  return PKV_OK;
}

}  // extern "C"
