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
// Policy: free blocks are handed out lowest id first (a min-heap); a failed
// call changes nothing, except that a batch append keeps the appends made
// before the sequence that failed.
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free;
  std::vector<int32_t> ref;                        // per block; 0 = free
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free.top();
    free.pop();
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) free.push(b);
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
  if (need > int64_t(bm->free.size())) return PKV_ERR_NO_BLOCKS;
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
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
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
    if (needs_block(bm, it->second) && bm->free.empty()) return PKV_ERR_NO_BLOCKS;
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
