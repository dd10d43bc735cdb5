// Host block allocator for one paged KV pool (one cache group).
//
// The mlx-node paged-cache doc (component table) splits a block-paged cache
// into physical storage (the per-layer K/V pools, owned by the caller here)
// and a BlockAllocator that owns the logical lifecycle: per-block refcounts,
// LRU eviction and a prefix table for cross-request reuse, driven by the
// per-request lifecycle reset -> find cached prefix -> allocate suffix blocks
// -> record tokens -> register full blocks for reuse -> release. Only whole
// blocks are shared; a block's identity follows its parent chain (Gemma4
// sliding sidecar section); a cache salt selects the lookup/publication domain
// (cache-salt section); sliding groups null out blocks wholly outside the
// window (hybrid coordinator paragraph).
//
// Policy details the pages leave open are fixed in pagedkv.h. Everything here
// is O(1) per block except prefix lookups (one hash-map probe per block).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <stdexcept>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pagedkv::fail;
using pagedkv::ok;

namespace {

// Exact prefix key: (domain, parent chain id or 0, the block's token ids).
struct PrefixKey {
  uint64_t domain;
  uint64_t parent;
  std::vector<int32_t> tokens;
  bool operator==(const PrefixKey& o) const {
    return domain == o.domain && parent == o.parent && tokens == o.tokens;
  }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const noexcept {
    // splitmix64-style mixing of every field; equality stays exact.
    auto mix = [](uint64_t x) {
      x += 0x9e3779b97f4a7c15ull;
      x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
      x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
      return x ^ (x >> 31);
    };
    uint64_t h = mix(k.domain) ^ mix(k.parent + 0x51ull);
    for (int32_t t : k.tokens) h = mix(h ^ static_cast<uint32_t>(t));
    return static_cast<size_t>(h);
  }
};

struct Seq {
  std::vector<int32_t> blocks;  // physical ids in logical order, 0 = dropped
  std::vector<int32_t> tokens;  // committed token ids
};

}  // namespace

struct paged_alloc {
  int32_t nb = 0;
  int32_t bs = 0;
  int32_t max_nb = 0;  // grow-on-demand ceiling; the size at creation unless raised
  std::deque<int32_t> free_list;
  // Intrusive LRU of evictable published blocks (oldest at head).
  std::vector<int32_t> lru_prev, lru_next;
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;
  std::vector<int32_t> ref;
  std::vector<uint64_t> chain_id;  // 0 = unpublished
  std::vector<PrefixKey> key_of;
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> table;
  uint64_t next_chain_id = 1;
  std::unordered_map<int64_t, Seq> seqs;

  void resize_block_arrays(int32_t n) {
    lru_prev.resize(n, -1);
    lru_next.resize(n, -1);
    in_lru.resize(n, 0);
    ref.resize(n, 0);
    chain_id.resize(n, 0);
    key_of.resize(n);
  }

  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++lru_size;
  }

  void lru_remove(int32_t b) {
    int32_t p = lru_prev[b], n = lru_next[b];
    if (p >= 0) lru_next[p] = n; else lru_head = n;
    if (n >= 0) lru_prev[n] = p; else lru_tail = p;
    lru_prev[b] = lru_next[b] = -1;
    in_lru[b] = 0;
    --lru_size;
  }

  int32_t take_new() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      b = lru_head;
      lru_remove(b);
      table.erase(key_of[b]);
      key_of[b] = PrefixKey{};
      chain_id[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  // Refcount - 1; at zero the block joins the LRU (published) or free tail.
  bool unref(int32_t b) {
    if (ref[b] <= 0) return false;
    if (--ref[b] == 0) {
      if (chain_id[b]) lru_push_back(b); else free_list.push_back(b);
    }
    return true;
  }

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

static bool valid_order(const int32_t* order, int32_t count, int32_t first) {
  std::vector<uint8_t> seen(static_cast<size_t>(count), 0);
  for (int32_t i = 0; i < count; ++i) {
    int64_t v = static_cast<int64_t>(order[i]) - first;
    if (v < 0 || v >= count || seen[v]) return false;
    seen[v] = 1;
  }
  return true;
}

extern "C" {

int32_t paged_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           paged_alloc** out) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!out) return fail(PAGED_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (num_blocks < 2 || block_size < 1)
      return fail(PAGED_ERR_INVALID_ARG, "need num_blocks >= 2 and block_size >= 1 (got %d, %d)",
                  num_blocks, block_size);
    if (free_order && !valid_order(free_order, num_blocks - 1, 1))
      return fail(PAGED_ERR_INVALID_ARG, "free_order is not a permutation of 1..%d", num_blocks - 1);
    auto* a = new paged_alloc();
    a->nb = num_blocks;
    a->max_nb = num_blocks;
    a->bs = block_size;
    a->resize_block_arrays(num_blocks);
    for (int32_t i = 0; i < num_blocks - 1; ++i)
      a->free_list.push_back(free_order ? free_order[i] : i + 1);
    *out = a;
    return ok();
  });
}

int32_t paged_alloc_destroy(paged_alloc* a) {
  delete a;
  return ok();
}

int32_t paged_alloc_grow(paged_alloc* a, int32_t new_num_blocks, const int32_t* new_order) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    if (new_num_blocks < a->nb)
      return fail(PAGED_ERR_INVALID_ARG, "cannot shrink from %d to %d blocks", a->nb, new_num_blocks);
    int32_t added = new_num_blocks - a->nb;
    if (new_order && !valid_order(new_order, added, a->nb))
      return fail(PAGED_ERR_INVALID_ARG, "new_order is not a permutation of %d..%d", a->nb,
                  new_num_blocks - 1);
    a->resize_block_arrays(new_num_blocks);
    for (int32_t i = 0; i < added; ++i) a->free_list.push_back(new_order ? new_order[i] : a->nb + i);
    a->nb = new_num_blocks;
    a->max_nb = std::max(a->max_nb, new_num_blocks);
    return ok();
  });
}

int32_t paged_alloc_set_max_blocks(paged_alloc* a, int32_t max_blocks) {
  if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
  if (max_blocks < a->nb)
    return fail(PAGED_ERR_INVALID_ARG, "max_blocks %d is below the pool's %d blocks", max_blocks, a->nb);
  a->max_nb = max_blocks;
  return ok();
}

int32_t paged_alloc_num_blocks(const paged_alloc* a, int32_t* num_blocks) {
  if (!a || !num_blocks) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  *num_blocks = a->nb;
  return ok();
}

int32_t paged_alloc_num_free(const paged_alloc* a, int32_t* free_blocks, int32_t* evictable_blocks) {
  if (!a || !free_blocks || !evictable_blocks) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  *free_blocks = static_cast<int32_t>(a->free_list.size());
  *evictable_blocks = a->lru_size;
  return ok();
}

int32_t paged_seq_add(paged_alloc* a, int64_t seq_id) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    if (a->find(seq_id)) return fail(PAGED_ERR_STATE, "sequence %lld exists", (long long)seq_id);
    a->seqs.emplace(seq_id, Seq{});
    return ok();
  });
}

int32_t paged_seq_match_prefix(paged_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                               uint64_t domain, int32_t* cached_tokens) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a || !cached_tokens || n < 0 || (n > 0 && !tokens))
      return fail(PAGED_ERR_INVALID_ARG, "bad argument");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    if (!s->blocks.empty()) return fail(PAGED_ERR_STATE, "match_prefix needs an empty sequence");
    PrefixKey key{domain, 0, std::vector<int32_t>(static_cast<size_t>(a->bs))};
    for (int32_t i = 0; i < n / a->bs; ++i) {
      std::memcpy(key.tokens.data(), tokens + static_cast<size_t>(i) * a->bs,
                  sizeof(int32_t) * a->bs);
      auto it = a->table.find(key);
      if (it == a->table.end()) break;
      int32_t b = it->second;
      if (a->ref[b] == 0) a->lru_remove(b);
      ++a->ref[b];
      s->blocks.push_back(b);
      s->tokens.insert(s->tokens.end(), key.tokens.begin(), key.tokens.end());
      key.parent = a->chain_id[b];
    }
    *cached_tokens = static_cast<int32_t>(s->blocks.size()) * a->bs;
    return ok();
  });
}

int32_t paged_seq_share_prefix(paged_alloc* a, int64_t dst_seq, int64_t src_seq, int32_t num_blocks) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    Seq* d = a->find(dst_seq);
    Seq* s = a->find(src_seq);
    if (!d || !s) return fail(PAGED_ERR_STATE, "unknown sequence");
    if (!d->blocks.empty()) return fail(PAGED_ERR_STATE, "share_prefix needs an empty destination");
    if (num_blocks < 0 || num_blocks > static_cast<int32_t>(s->blocks.size()) ||
        static_cast<int64_t>(num_blocks) * a->bs > static_cast<int64_t>(s->tokens.size()))
      return fail(PAGED_ERR_STATE, "source does not hold %d full blocks", num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i)
      if (s->blocks[i] == 0) return fail(PAGED_ERR_STATE, "cannot share a dropped block");
    for (int32_t i = 0; i < num_blocks; ++i) {
      ++a->ref[s->blocks[i]];
      d->blocks.push_back(s->blocks[i]);
    }
    d->tokens.assign(s->tokens.begin(), s->tokens.begin() + static_cast<size_t>(num_blocks) * a->bs);
    return ok();
  });
}

int32_t paged_seq_reserve(paged_alloc* a, int64_t seq_id, int32_t total_tokens) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    if (total_tokens < 0) return fail(PAGED_ERR_INVALID_ARG, "negative token count");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    int64_t want = (static_cast<int64_t>(total_tokens) + a->bs - 1) / a->bs;
    int64_t need = want - static_cast<int64_t>(s->blocks.size());
    if (need <= 0) return ok();
    if (static_cast<int64_t>(a->free_list.size()) + a->lru_size < need)
      return fail(PAGED_ERR_NO_BLOCKS, "need %lld blocks, %zu free + %d evictable", (long long)need,
                  a->free_list.size(), a->lru_size);
    s->blocks.reserve(static_cast<size_t>(want));
    for (int64_t i = 0; i < need; ++i) s->blocks.push_back(a->take_new());
    return ok();
  });
}

int32_t paged_seq_reserve_or_grow(paged_alloc* a, int64_t seq_id, int32_t total_tokens,
                                  int32_t* grow_to) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a || !grow_to) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
    *grow_to = 0;
    if (total_tokens < 0) return fail(PAGED_ERR_INVALID_ARG, "negative token count");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    const int64_t needed = (static_cast<int64_t>(total_tokens) + a->bs - 1) / a->bs -
                           static_cast<int64_t>(s->blocks.size());
    const int64_t avail = static_cast<int64_t>(a->free_list.size()) + a->lru_size;
    // Fits in free + evictable blocks (or needs nothing): an ordinary reservation.
    if (needed <= avail) return paged_seq_reserve(a, seq_id, total_tokens);
    if (a->nb >= a->max_nb)
      return fail(PAGED_ERR_NO_BLOCKS, "need %lld blocks, %lld free + evictable, pool at its maximum of %d",
                  (long long)needed, (long long)avail, a->max_nb);
    const int64_t target = std::max<int64_t>(2LL * a->nb, a->nb + needed);
    *grow_to = static_cast<int32_t>(std::min<int64_t>(a->max_nb, target));
    return ok();
  });
}

int32_t paged_seq_commit_tokens(paged_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a || n < 0 || (n > 0 && !tokens)) return fail(PAGED_ERR_INVALID_ARG, "bad argument");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    if (static_cast<int64_t>(s->tokens.size()) + n > static_cast<int64_t>(s->blocks.size()) * a->bs)
      return fail(PAGED_ERR_CAPACITY, "commit beyond reserved blocks");
    s->tokens.insert(s->tokens.end(), tokens, tokens + n);
    return ok();
  });
}

int32_t paged_seq_publish_full_blocks(paged_alloc* a, int64_t seq_id, uint64_t domain) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    uint64_t parent = 0;
    const size_t full = s->tokens.size() / static_cast<size_t>(a->bs);
    for (size_t i = 0; i < full; ++i) {
      int32_t b = s->blocks[i];
      if (b == 0) break;
      if (a->chain_id[b]) {
        parent = a->chain_id[b];
        continue;
      }
      PrefixKey key{domain, parent,
                    std::vector<int32_t>(s->tokens.begin() + i * a->bs,
                                         s->tokens.begin() + (i + 1) * a->bs)};
      auto it = a->table.find(key);
      if (it != a->table.end()) {
        parent = a->chain_id[it->second];
        continue;
      }
      a->chain_id[b] = a->next_chain_id++;
      a->key_of[b] = key;
      a->table.emplace(std::move(key), b);
      parent = a->chain_id[b];
    }
    return ok();
  });
}

int32_t paged_seq_drop_outside_window(paged_alloc* a, int64_t seq_id, int32_t window) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    if (window <= 0) return fail(PAGED_ERR_INVALID_ARG, "window must be positive");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    int64_t first_needed = static_cast<int64_t>(s->tokens.size()) - window;
    for (size_t i = 0; i < s->blocks.size(); ++i) {
      int32_t b = s->blocks[i];
      if (b != 0 && static_cast<int64_t>(i + 1) * a->bs <= first_needed) {
        if (!a->unref(b)) return fail(PAGED_ERR_STATE, "refcount underflow on block %d", b);
        s->blocks[i] = 0;
      }
    }
    return ok();
  });
}

int32_t paged_seq_release(paged_alloc* a, int64_t seq_id) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a) return fail(PAGED_ERR_INVALID_ARG, "allocator is NULL");
    Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    for (auto it = s->blocks.rbegin(); it != s->blocks.rend(); ++it)
      if (*it != 0 && !a->unref(*it))
        return fail(PAGED_ERR_STATE, "refcount underflow on block %d", *it);
    a->seqs.erase(seq_id);
    return ok();
  });
}

int32_t paged_seq_num_tokens(const paged_alloc* a, int64_t seq_id, int32_t* committed_tokens,
                             int32_t* table_blocks) {
  if (!a || !committed_tokens || !table_blocks) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  const Seq* s = a->find(seq_id);
  if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
  *committed_tokens = static_cast<int32_t>(s->tokens.size());
  *table_blocks = static_cast<int32_t>(s->blocks.size());
  return ok();
}

int32_t paged_alloc_block_tables(const paged_alloc* a, const int64_t* seq_ids, int32_t batch,
                                 int32_t max_blocks, int32_t* out, int32_t* needed) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a || batch < 0 || max_blocks < 0 || (batch > 0 && (!seq_ids || !out)))
      return fail(PAGED_ERR_INVALID_ARG, "bad argument");
    int32_t widest = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const Seq* s = a->find(seq_ids[b]);
      if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_ids[b]);
      widest = std::max(widest, static_cast<int32_t>(s->blocks.size()));
    }
    if (needed) *needed = widest;
    if (widest > max_blocks)
      return fail(PAGED_ERR_CAPACITY, "a table needs %d columns, buffer has %d", widest, max_blocks);
    for (int32_t b = 0; b < batch; ++b) {
      const Seq* s = a->find(seq_ids[b]);
      int32_t* row = out + static_cast<size_t>(b) * max_blocks;
      size_t n = s->blocks.size();
      if (n) std::memcpy(row, s->blocks.data(), n * sizeof(int32_t));
      std::memset(row + n, 0, (static_cast<size_t>(max_blocks) - n) * sizeof(int32_t));
    }
    return ok();
  });
}

int32_t paged_alloc_slot_mapping(const paged_alloc* a, int64_t seq_id, int32_t start_pos, int32_t n,
                                 int64_t* out) {
  PAGEDKV_GUARD([&]() -> int32_t {
    if (!a || n < 0 || (n > 0 && !out)) return fail(PAGED_ERR_INVALID_ARG, "bad argument");
    const Seq* s = a->find(seq_id);
    if (!s) return fail(PAGED_ERR_STATE, "unknown sequence %lld", (long long)seq_id);
    // Validate every position before writing anything.
    for (int32_t j = 0; j < n; ++j) {
      int64_t p = static_cast<int64_t>(start_pos) + j;
      if (p < 0 || p / a->bs >= static_cast<int64_t>(s->blocks.size()))
        return fail(PAGED_ERR_CAPACITY, "position %lld is not reserved", (long long)p);
      if (s->blocks[static_cast<size_t>(p / a->bs)] == 0)
        return fail(PAGED_ERR_STATE, "position %lld lies in a dropped block", (long long)p);
    }
    for (int32_t j = 0; j < n; ++j) {
      int64_t p = static_cast<int64_t>(start_pos) + j;
      out[j] = static_cast<int64_t>(s->blocks[static_cast<size_t>(p / a->bs)]) * a->bs + p % a->bs;
    }
    return ok();
  });
}

int32_t paged_alloc_refcount(const paged_alloc* a, int32_t block_id, int32_t* refcount) {
  if (!a || !refcount) return fail(PAGED_ERR_INVALID_ARG, "NULL argument");
  if (block_id < 0 || block_id >= a->nb)
    return fail(PAGED_ERR_INVALID_ARG, "block id %d out of range", block_id);
  *refcount = a->ref[block_id];
  return ok();
}

}  // extern "C"
