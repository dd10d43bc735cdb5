// Host-only driver for the allocator under AddressSanitizer/UBSan: random
// lifecycle calls (including every error path) against the C ABI, checking
// the conservation invariant after each call. Built and run by
// tests/test_allocator_parity.py.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);      \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main() {
  std::mt19937 rng(7);
  for (int round = 0; round < 20; ++round) {
    const int nb = 16 + round * 3, bs = 4;
    std::vector<int32_t> order(nb - 1);
    for (int i = 0; i < nb - 1; ++i) order[i] = i + 1;
    std::shuffle(order.begin(), order.end(), rng);
    paged_alloc* a = nullptr;
    CHECK(paged_alloc_create(nb, bs, order.data(), &a) == PAGED_OK);
    std::vector<int64_t> live;
    int64_t next = 0;
    for (int op = 0; op < 400; ++op) {
      const int r = rng() % 10;
      if (r < 3 || live.empty()) {
        int64_t id = next++;
        CHECK(paged_seq_add(a, id) == PAGED_OK);
        CHECK(paged_seq_add(a, id) == PAGED_ERR_STATE);
        std::vector<int32_t> toks(1 + rng() % 20);
        for (auto& t : toks) t = rng() % 3;
        int32_t cached = -1;
        CHECK(paged_seq_match_prefix(a, id, toks.data(), (int32_t)toks.size() - 1, rng() % 2, &cached) == PAGED_OK);
        CHECK(cached % bs == 0);
        if (paged_seq_reserve(a, id, (int32_t)toks.size()) == PAGED_OK) {
          CHECK(paged_seq_commit_tokens(a, id, toks.data() + cached, (int32_t)toks.size() - cached) == PAGED_OK);
          CHECK(paged_seq_publish_full_blocks(a, id, 0) == PAGED_OK);
        }
        live.push_back(id);
      } else if (r < 5) {
        int64_t id = live[rng() % live.size()];
        int32_t t = 0, blocks = 0;
        CHECK(paged_seq_num_tokens(a, id, &t, &blocks) == PAGED_OK);
        std::vector<int32_t> toks(1 + rng() % 6, 1);
        if (paged_seq_reserve(a, id, t + (int32_t)toks.size()) == PAGED_OK)
          CHECK(paged_seq_commit_tokens(a, id, toks.data(), (int32_t)toks.size()) == PAGED_OK);
        CHECK(paged_seq_commit_tokens(a, id, toks.data(), 1 << 20) == PAGED_ERR_CAPACITY);
      } else if (r < 6) {
        int64_t id = live[rng() % live.size()];
        CHECK(paged_seq_drop_outside_window(a, id, 1 + rng() % 9) == PAGED_OK);
        CHECK(paged_seq_drop_outside_window(a, id, 0) == PAGED_ERR_INVALID_ARG);
      } else if (r < 7) {
        int64_t src = live[rng() % live.size()];
        int64_t dst = next++;
        CHECK(paged_seq_add(a, dst) == PAGED_OK);
        paged_seq_share_prefix(a, dst, src, rng() % 3);
        live.push_back(dst);
      } else if (r < 8) {
        std::vector<int32_t> tab(live.size() * 8);
        int32_t needed = 0;
        int rc = paged_alloc_block_tables(a, live.data(), (int32_t)live.size(), 8, tab.data(), &needed);
        CHECK(rc == PAGED_OK || rc == PAGED_ERR_CAPACITY);
        int64_t id = live[rng() % live.size()];
        int32_t t = 0, blocks = 0;
        CHECK(paged_seq_num_tokens(a, id, &t, &blocks) == PAGED_OK);
        std::vector<int64_t> slots(static_cast<size_t>(blocks) * bs + 1);
        rc = paged_alloc_slot_mapping(a, id, 0, t, slots.data());
        CHECK(rc == PAGED_OK || rc == PAGED_ERR_STATE);
        CHECK(paged_alloc_slot_mapping(a, id, 0, blocks * bs + 1, slots.data()) != PAGED_OK);
      } else {
        size_t k = rng() % live.size();
        CHECK(paged_seq_release(a, live[k]) == PAGED_OK);
        CHECK(paged_seq_release(a, live[k]) == PAGED_ERR_STATE);
        live.erase(live.begin() + k);
      }
      // conservation: free + evictable + referenced == nb - 1
      int32_t f = 0, e = 0, used = 0, rc = 0;
      CHECK(paged_alloc_num_free(a, &f, &e) == PAGED_OK);
      for (int b = 1; b < nb; ++b) {
        CHECK(paged_alloc_refcount(a, b, &rc) == PAGED_OK);
        used += rc > 0;
      }
      CHECK(f + e + used == nb - 1);
    }
    CHECK(paged_alloc_grow(a, nb + 5, nullptr) == PAGED_OK);
    CHECK(paged_alloc_refcount(a, nb + 5, nullptr) == PAGED_ERR_INVALID_ARG);
    for (int64_t id : live) CHECK(paged_seq_release(a, id) == PAGED_OK);
    int32_t f = 0, e = 0;
    CHECK(paged_alloc_num_free(a, &f, &e) == PAGED_OK);
    CHECK(f + e == nb + 4);
    CHECK(paged_alloc_destroy(a) == PAGED_OK);
  }
  std::printf("OK\n");
  return 0;
}
