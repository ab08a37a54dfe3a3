// Drives the host block manager through a seeded random sequence of calls
// (adds with and without prompt tokens, forks, batched appends, frees, table
// and slot queries, and calls that must fail) for a build with address and
// undefined-behaviour sanitizers.  After every call it checks what the
// manager's own contract fixes: a failed call leaves the counts unchanged,
// every table entry and slot lies in the pool, each sequence holds
// ceil(tokens / block_size) blocks, and no block is lost (free + cached +
// referenced-only blocks never exceed the pool).  Prints "all ok".
#include <algorithm>
#include <cstdint>
#include <iterator>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::printf("check failed at line %d: %s\n", __LINE__, #c);     \
      std::exit(1);                                                    \
    }                                                                  \
  } while (0)

namespace {

struct Run {
  pkv_block_manager* bm = nullptr;
  int32_t nb, bs;
  std::map<int64_t, int64_t> tokens;           // live sequences -> token count
  std::mt19937_64 rng;
  int64_t next_id = 1;

  Run(int32_t nb_, int32_t bs_, uint64_t seed) : nb(nb_), bs(bs_), rng(seed) {
    CHECK(pkv_bm_create(nb, bs, &bm) == PKV_OK);
  }
  ~Run() { pkv_bm_destroy(bm); }

  int64_t pick() {
    auto it = tokens.begin();
    std::advance(it, int(rng() % tokens.size()));
    return it->first;
  }

  void check_sequence(int64_t id) {
    std::vector<int32_t> table(4096);
    int32_t n = -1;
    int64_t t = -1;
    CHECK(pkv_bm_get_block_table(bm, id, table.data(), int32_t(table.size()), &n, &t) == PKV_OK);
    CHECK(t == tokens[id]);
    CHECK(n == int32_t((t + bs - 1) / bs));
    for (int i = 0; i < n; ++i) CHECK(table[i] >= 0 && table[i] < nb);
    if (t > 0) {
      std::vector<int64_t> slots(static_cast<size_t>(t));
      CHECK(pkv_bm_token_slots(bm, id, 0, int32_t(t), slots.data()) == PKV_OK);
      for (int64_t k = 0; k < t; ++k) CHECK(slots[k] == int64_t(table[k / bs]) * bs + k % bs);
      CHECK(pkv_bm_token_slots(bm, id, t, 1, slots.data()) == PKV_ERR_VALUE);
    }
  }

  void step() {
    const int32_t free0 = pkv_bm_num_free_blocks(bm);
    const int32_t cached0 = pkv_bm_num_cached_blocks(bm);
    CHECK(free0 >= 0 && cached0 >= 0 && free0 + cached0 <= nb);
    int op = int(rng() % 8);
    if (free0 < nb / 4 && rng() % 2 == 0 && !tokens.empty()) op = 5;   // keep the pool in use, not full
    if (op == 0 || tokens.empty()) {                       // plain add
      const int64_t id = next_id++;
      const int64_t t = int64_t(rng() % (3 * bs + 1));
      const pkv_status st = pkv_bm_add_sequence(bm, id, t);
      CHECK(st == PKV_OK || st == PKV_ERR_NO_BLOCKS);
      if (st == PKV_OK) tokens[id] = t;
      else CHECK(pkv_bm_num_free_blocks(bm) == free0 && pkv_bm_num_cached_blocks(bm) == cached0);
    } else if (op == 1) {                                  // add with prompt tokens (few ids: prefixes repeat)
      const int64_t id = next_id++;
      const int64_t t = 1 + int64_t(rng() % (4 * bs));
      std::vector<int64_t> toks(static_cast<size_t>(t));
      const int64_t family = int64_t(rng() % 3);
      for (int64_t k = 0; k < t; ++k) toks[k] = family * 1000 + (k < 2 * bs ? k : int64_t(rng() % 4));
      int64_t cached = -1;
      const pkv_status st = pkv_bm_add_sequence_cached(bm, id, toks.data(), t, &cached);
      CHECK(st == PKV_OK || st == PKV_ERR_NO_BLOCKS);
      if (st == PKV_OK) {
        tokens[id] = t;
        CHECK(cached >= 0 && cached % bs == 0 && cached <= t - 1);
      }
    } else if (op == 2) {                                  // fork
      const int64_t parent = pick(), child = next_id++;
      CHECK(pkv_bm_fork(bm, parent, child) == PKV_OK);
      tokens[child] = tokens[parent];
      CHECK(pkv_bm_num_free_blocks(bm) == free0);
    } else if (op <= 4) {                                  // batched append
      const int32_t n = 1 + int32_t(rng() % 6);
      std::vector<int64_t> ids(static_cast<size_t>(n)), slots(static_cast<size_t>(n)),
          pairs(static_cast<size_t>(2 * n));
      std::set<int64_t> seen;
      for (int32_t i = 0; i < n; ++i) {
        ids[i] = pick();
        if (!seen.insert(ids[i]).second) ids[i] = next_id + 1000000;   // an unknown id
      }
      int32_t ncopy = -1, done = -1;
      const pkv_status st = pkv_bm_append_tokens(bm, ids.data(), n, slots.data(), pairs.data(),
                                                 &ncopy, &done);
      CHECK(st == PKV_OK || st == PKV_ERR_NO_BLOCKS || st == PKV_ERR_SEQUENCE);
      CHECK(done >= 0 && done <= n && ncopy >= 0 && ncopy <= done);
      CHECK((st == PKV_OK) == (done == n));
      for (int32_t i = 0; i < done; ++i) {
        CHECK(slots[i] >= 0 && slots[i] < int64_t(nb) * bs);
        CHECK(slots[i] % bs == tokens[ids[i]] % bs);
        ++tokens[ids[i]];
      }
      for (int32_t c = 0; c < ncopy; ++c) {
        CHECK(pairs[2 * c] >= 0 && pairs[2 * c] < nb && pairs[2 * c + 1] >= 0 && pairs[2 * c + 1] < nb);
        CHECK(pairs[2 * c] != pairs[2 * c + 1]);
      }
    } else if (op == 5) {                                  // free
      const int64_t id = pick();
      CHECK(pkv_bm_free_sequence(bm, id) == PKV_OK);
      tokens.erase(id);
    } else if (op == 6) {                                  // tables for a batch
      const int32_t n = int32_t(tokens.size());
      std::vector<int64_t> ids;
      for (auto& kv : tokens) ids.push_back(kv.first);
      int32_t mb = 1;
      for (auto& kv : tokens) mb = std::max<int32_t>(mb, int32_t((kv.second + bs - 1) / bs));
      std::vector<int32_t> bt(static_cast<size_t>(n) * mb), lens(static_cast<size_t>(n));
      CHECK(pkv_bm_build_block_tables(bm, ids.data(), n, mb, bt.data(), lens.data()) == PKV_OK);
      for (int32_t i = 0; i < n; ++i) {
        CHECK(lens[i] == tokens[ids[i]]);
        for (int32_t j = 0; j < mb; ++j) {
          const int32_t e = bt[size_t(i) * mb + j];
          CHECK(j < (lens[i] + bs - 1) / bs ? (e >= 0 && e < nb) : e == -1);
        }
      }
      if (mb > 1) {                                        // too narrow: nothing written
        std::vector<int32_t> bt2(static_cast<size_t>(n) * (mb - 1), 77), lens2(static_cast<size_t>(n), 77);
        CHECK(pkv_bm_build_block_tables(bm, ids.data(), n, mb - 1, bt2.data(), lens2.data()) ==
              PKV_ERR_SHAPE);
        for (int32_t x : bt2) CHECK(x == 77);
        for (int32_t x : lens2) CHECK(x == 77);
      }
    } else {                                               // calls that must fail, changing nothing
      const int64_t id = pick();
      CHECK(pkv_bm_add_sequence(bm, id, 1) != PKV_OK);                 // id in use
      CHECK(pkv_bm_add_sequence(bm, next_id, -1) != PKV_OK);           // negative count
      CHECK(pkv_bm_fork(bm, next_id + 7, next_id + 8) != PKV_OK);      // unknown parent
      CHECK(pkv_bm_fork(bm, id, id) != PKV_OK);                        // child in use
      CHECK(pkv_bm_free_sequence(bm, next_id + 9) != PKV_OK);          // unknown
      int64_t cached = 0;
      CHECK(pkv_bm_add_sequence_cached(bm, next_id, nullptr, 3, &cached) == PKV_ERR_NULL);
      int32_t n = 0;
      int64_t t = 0;
      int32_t one = 0;
      if (tokens[id] > bs) CHECK(pkv_bm_get_block_table(bm, id, &one, 1, &n, &t) == PKV_ERR_SHAPE);
      CHECK(pkv_bm_num_free_blocks(bm) == free0 && pkv_bm_num_cached_blocks(bm) == cached0);
    }
    for (auto& kv : tokens) check_sequence(kv.first);
    // every block is free, referenced by a sequence, or cached without a
    // reference: free + referenced <= pool <= free + referenced + cached
    std::set<int32_t> referenced;
    for (auto& kv : tokens) {
      std::vector<int32_t> table(4096);
      int32_t n = 0;
      int64_t t = 0;
      CHECK(pkv_bm_get_block_table(bm, kv.first, table.data(), int32_t(table.size()), &n, &t) ==
            PKV_OK);
      referenced.insert(table.begin(), table.begin() + n);
    }
    const int32_t fr = pkv_bm_num_free_blocks(bm), ca = pkv_bm_num_cached_blocks(bm);
    CHECK(fr + int32_t(referenced.size()) <= nb);
    CHECK(fr + int32_t(referenced.size()) + ca >= nb);
  }
};

}  // namespace

int main() {
  CHECK(pkv_bm_create(0, 16, nullptr) != PKV_OK);
  pkv_block_manager* bad = nullptr;
  CHECK(pkv_bm_create(4, 0, &bad) != PKV_OK);
  const int32_t sizes[][2] = {{48, 1}, {40, 2}, {64, 16}, {24, 5}};
  for (int r = 0; r < 4; ++r) {
    Run run(sizes[r][0], sizes[r][1], 1234u + r);
    for (int s = 0; s < 3000; ++s) run.step();
  }
  std::printf("all ok\n");
  return 0;
}
