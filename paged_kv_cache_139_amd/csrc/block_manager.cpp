// Host block manager: the bookkeeping half of paged KV caching.
//
// A pool of num_blocks physical blocks, a block table and token count per
// sequence, and a reference count per block ([L3] "核心数据结构：Block Table":
// a sequence holds ceil(tokens / block_size) blocks; [CB] §3.2: allocate,
// fork -- the child shares the parent's blocks, whose counts go up -- and
// free, which returns a block when its count reaches zero; [VN] "Sharing KV
// Cache" and [L3] "共享前缀": appending into a block that another sequence
// still references first moves the appending sequence to a copy).
//
// The manager never touches device memory.  A decode step asks it for the
// new tokens' slots and the copy-on-write pairs; the caller then runs
// copy_blocks(pairs), reshape_and_cache(slots) and the decode call with the
// tables built here.
//
// Prefix cache ([TGI] §5.2-5.3: a trie from prompt tokens to blocks with a
// reference count and last access time per node, longest-prefix lookup on
// allocation, insertion of the prompt's blocks when the request is freed,
// eviction of unreferenced leaves oldest first; [VN] "Prefix Caching": a
// request whose leading blocks hold the same tokens as cached ones points
// its table at them).  One trie node per full block, keyed by that block's
// token ids, so no node ever needs splitting.  A block is free, referenced
// by sequences, or cached with no reference; cached blocks are taken for new
// allocations only when the free list is empty.
//
// Policy: free blocks are handed out lowest id first (a min-heap), evicted
// blocks least recently used first (ties: lowest id); a failed call changes
// nothing, except that a batch append keeps the appends made before the
// sequence that failed.
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <map>
#include <new>
#include <queue>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
    std::vector<int64_t> prompt;                   // token ids (cached adds only)
  };
  using Key = std::vector<int64_t>;                // one block's token ids
  static constexpr int32_t kRoot = -1;
  // trie node of a cached block, indexed by the block id
  struct Node {
    bool cached = false;
    int32_t parent = kRoot;
    int64_t access = 0;
    Key key;
    std::map<Key, int32_t> children;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free;
  std::vector<int32_t> ref;                        // per block; 0 = free or cached only
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<Node> node;                          // per block
  std::map<Key, int32_t> root_children;
  std::set<std::pair<int64_t, int32_t>> evictable; // (access, block): unreferenced leaves
  int32_t num_cached = 0;
  int64_t tick = 0;

  std::map<Key, int32_t>& children_of(int32_t parent) {
    return parent == kRoot ? root_children : node[size_t(parent)].children;
  }
  bool is_evictable(int32_t b) const {
    const Node& n = node[size_t(b)];
    return n.cached && ref[size_t(b)] == 0 && n.children.empty();
  }
  void update_evictable(int32_t b) {
    if (b == kRoot) return;
    const Node& n = node[size_t(b)];
    if (is_evictable(b)) evictable.insert({n.access, b});
  }
  void unmark(int32_t b) { evictable.erase({node[size_t(b)].access, b}); }

  // Removes the least recently used unreferenced leaf from the cache and
  // returns its block (its parent may become evictable).
  int32_t evict() {
    const int32_t b = evictable.begin()->second;
    evictable.erase(evictable.begin());
    Node& n = node[size_t(b)];
    children_of(n.parent).erase(n.key);
    const int32_t parent = n.parent;
    n = Node();
    --num_cached;
    update_evictable(parent);
    return b;
  }
  bool can_take() const { return !free.empty() || !evictable.empty(); }
  int32_t take() {
    int32_t b;
    if (!free.empty()) {
      b = free.top();
      free.pop();
    } else {
      b = evict();
    }
    ref[size_t(b)] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[size_t(b)] > 0) return;
    if (node[size_t(b)].cached) update_evictable(b);
    else free.push(b);
  }
  // Blocks that allocation can obtain now or by evicting leaves in turn: the
  // free list plus the cached blocks whose subtree no sequence references
  // (`pinned` blocks count as referenced).
  int64_t obtainable(const std::vector<int32_t>& pinned) {
    int64_t n = int64_t(free.size());
    if (evictable.empty()) return n;
    std::vector<char> pin(size_t(num_blocks), 0);
    for (int32_t b : pinned) pin[size_t(b)] = 1;
    // post-order over the trie: a node counts when it and its subtree are free of references
    std::function<bool(int32_t)> clear = [&](int32_t b) {
      bool all = ref[size_t(b)] == 0 && !pin[size_t(b)];
      for (const auto& kv : node[size_t(b)].children) all = clear(kv.second) && all;
      if (all) ++n;
      return all;
    };
    for (const auto& kv : root_children) clear(kv.second);
    return n;
  }
};

namespace {

// One token appended to `s`: its slot, and (src, dst) when the last block was
// copied.  The caller has checked that a free block exists if one is needed.
int64_t append_one(pkv_block_manager* bm, pkv_block_manager::Seq& s, int32_t* src,
                   int32_t* dst) {
  const int32_t off = static_cast<int32_t>(s.tokens % bm->block_size);
  int32_t b;
  *src = *dst = -1;
  if (off == 0) {
    b = bm->take();
    s.blocks.push_back(b);
  } else {
    b = s.blocks.back();
    if (bm->ref[b] > 1) {
      const int32_t nb = bm->take();
      --bm->ref[b];
      *src = b;
      *dst = nb;
      s.blocks.back() = nb;
      b = nb;
    }
  }
  ++s.tokens;
  return int64_t(b) * bm->block_size + off;
}

bool needs_block(const pkv_block_manager* bm, const pkv_block_manager::Seq& s) {
  const int32_t off = static_cast<int32_t>(s.tokens % bm->block_size);
  return off == 0 || bm->ref[s.blocks.back()] > 1;
}

}  // namespace

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, pkv_block_manager** out) {
  if (!out) return PKV_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PKV_ERR_SHAPE;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return PKV_ERR_NO_BLOCKS;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(size_t(num_blocks), 0);
  bm->node.assign(size_t(num_blocks), pkv_block_manager::Node());
  std::vector<int32_t> ids(static_cast<size_t>(num_blocks));
  for (int32_t i = 0; i < num_blocks; ++i) ids[size_t(i)] = i;
  bm->free = decltype(bm->free)(std::greater<int32_t>(), std::move(ids));
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
  return bm ? static_cast<int32_t>(bm->free.size()) : 0;
}

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens) {
  if (!bm) return PKV_ERR_NULL;
  if (num_tokens < 0) return PKV_ERR_VALUE;
  if (bm->seqs.count(seq_id)) return PKV_ERR_SEQUENCE;
  const int64_t need = (num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > int64_t(bm->free.size()) && need > bm->obtainable({})) return PKV_ERR_NO_BLOCKS;
  pkv_block_manager::Seq s;
  s.blocks.reserve(size_t(need));
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  s.tokens = num_tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->seqs.count(child_id)) return PKV_ERR_SEQUENCE;
  pkv_block_manager::Seq child = it->second;       // copy before the map may rehash
  for (int32_t b : child.blocks) ++bm->ref[b];
  bm->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
  const pkv_block_manager::Seq& s = it->second;
  ++bm->tick;
  if (!s.prompt.empty()) {
    // the prompt's full blocks enter the cache: follow the nodes that hold
    // the same tokens, add this sequence's blocks below where they end
    const int64_t full = int64_t(s.prompt.size()) / bm->block_size;
    int32_t at = pkv_block_manager::kRoot;
    for (int64_t j = 0; j < full; ++j) {
      pkv_block_manager::Key key(s.prompt.begin() + j * bm->block_size,
                                 s.prompt.begin() + (j + 1) * bm->block_size);
      auto& kids = bm->children_of(at);
      auto found = kids.find(key);
      int32_t b;
      if (found != kids.end()) {
        b = found->second;
        bm->unmark(b);
      } else {
        b = s.blocks[size_t(j)];
        if (at != pkv_block_manager::kRoot) bm->unmark(at);   // no longer a leaf
        pkv_block_manager::Node& n = bm->node[size_t(b)];
        n.cached = true;
        n.parent = at;
        n.key = key;
        kids.emplace(std::move(key), b);
        ++bm->num_cached;
      }
      bm->node[size_t(b)].access = bm->tick;
      bm->update_evictable(b);
      at = b;
    }
  }
  for (int32_t b : s.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_add_sequence_cached(pkv_block_manager* bm, int64_t seq_id,
                                      const int64_t* tokens, int64_t num_tokens,
                                      int64_t* cached_tokens) {
  if (!bm || !cached_tokens) return PKV_ERR_NULL;
  *cached_tokens = 0;
  if (num_tokens < 0) return PKV_ERR_VALUE;
  if (num_tokens > 0 && !tokens) return PKV_ERR_NULL;
  if (bm->seqs.count(seq_id)) return PKV_ERR_SEQUENCE;
  const int32_t bs = bm->block_size;
  // cached blocks matching the prompt's leading full blocks, within its
  // first num_tokens - 1 tokens (the last token is always computed)
  std::vector<int32_t> hits;
  const int64_t matchable = num_tokens > 0 ? (num_tokens - 1) / bs : 0;
  int32_t at = pkv_block_manager::kRoot;
  for (int64_t j = 0; j < matchable; ++j) {
    const pkv_block_manager::Key key(tokens + j * bs, tokens + (j + 1) * bs);
    auto& kids = bm->children_of(at);
    auto found = kids.find(key);
    if (found == kids.end()) break;
    at = found->second;
    hits.push_back(at);
  }
  const int64_t need = (num_tokens + bs - 1) / bs - int64_t(hits.size());
  if (need > int64_t(bm->free.size()) && need > bm->obtainable(hits)) return PKV_ERR_NO_BLOCKS;
  ++bm->tick;
  pkv_block_manager::Seq s;
  s.blocks.reserve(size_t(need) + hits.size());
  for (int32_t b : hits) {                        // shared: referenced, recently used
    bm->unmark(b);
    ++bm->ref[size_t(b)];
    bm->node[size_t(b)].access = bm->tick;
    s.blocks.push_back(b);
  }
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  s.tokens = num_tokens;
  s.prompt.assign(tokens, tokens + num_tokens);
  bm->seqs.emplace(seq_id, std::move(s));
  *cached_tokens = int64_t(hits.size()) * bs;
  return PKV_OK;
}

int32_t pkv_bm_num_cached_blocks(const pkv_block_manager* bm) {
  return bm ? bm->num_cached : 0;
}

pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                                int64_t* slots, int64_t* copy_pairs, int32_t* num_copies,
                                int32_t* num_done) {
  if (!bm || !num_copies || !num_done) return PKV_ERR_NULL;
  *num_copies = 0;
  *num_done = 0;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!seq_ids || !slots || !copy_pairs) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
    if (needs_block(bm, it->second) && !bm->can_take()) return PKV_ERR_NO_BLOCKS;
    int32_t src, dst;
    slots[i] = append_one(bm, it->second, &src, &dst);
    if (src >= 0) {
      copy_pairs[2 * *num_copies] = src;
      copy_pairs[2 * *num_copies + 1] = dst;
      ++*num_copies;
    }
    ++*num_done;
  }
  return PKV_OK;
}

pkv_status pkv_bm_get_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table,
                                  int32_t capacity, int32_t* num_blocks, int64_t* num_tokens) {
  if (!bm || !num_blocks || !num_tokens) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
  const auto& s = it->second;
  *num_blocks = static_cast<int32_t>(s.blocks.size());
  *num_tokens = s.tokens;
  if (capacity < *num_blocks) return PKV_ERR_SHAPE;
  if (*num_blocks > 0 && !table) return PKV_ERR_NULL;
  std::copy(s.blocks.begin(), s.blocks.end(), table);
  return PKV_OK;
}

pkv_status pkv_bm_token_slots(const pkv_block_manager* bm, int64_t seq_id, int64_t first,
                              int32_t count, int64_t* slots) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
  const auto& s = it->second;
  if (first < 0 || count < 0 || first + count > s.tokens) return PKV_ERR_VALUE;
  if (count > 0 && !slots) return PKV_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t t = first + i;
    slots[i] = int64_t(s.blocks[size_t(t / bm->block_size)]) * bm->block_size +
               t % bm->block_size;
  }
  return PKV_OK;
}

pkv_status pkv_bm_build_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids,
                                     int32_t n, int32_t max_blocks_per_seq,
                                     int32_t* block_tables, int32_t* context_lens) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0 || max_blocks_per_seq < 1) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!seq_ids || !block_tables || !context_lens) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {                // check everything before writing
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_ERR_SEQUENCE;
    if (int64_t(it->second.blocks.size()) > max_blocks_per_seq) return PKV_ERR_SHAPE;
    if (it->second.tokens > 0x7fffffff) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + size_t(i) * max_blocks_per_seq;
    std::fill(row, row + max_blocks_per_seq, -1);
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    context_lens[i] = static_cast<int32_t>(s.tokens);
  }
  return PKV_OK;
}

}  // extern "C"
