// Host block manager of the paged KV cache (declared in pkv_blocks.h).
//
// The pool is allocated once; the manager only moves block indices around:
// a FIFO free queue, a reference count per block, and per sequence its block
// list and token count. Blocks are handed out as sequences grow, shared
// between a parent and its forks, copied before a shared block is written,
// and returned last block first when a sequence ends (vLLM paper page,
// "PagedAttention" core idea and the OS-paging table: on-demand blocks, fork
// and copy-on-write; vLLM notes page, "KV Cache and PagedAttention":
// ref_count sharing and the free-block queue; same page, "Prefix Caching"
// eviction paragraph: reverse-order release).
#include <stdint.h>

#include <deque>
#include <mutex>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_blocks.h"
#include "status.h"

struct pkv_block_manager {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_queue;  // front = next block handed out
  std::vector<int32_t> refcount;   // per block; 0 while in the free queue
  struct Sequence {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  std::unordered_map<int64_t, Sequence> seqs;
  std::mutex mu;

  int32_t take() {
    const int32_t b = free_queue.front();
    free_queue.pop_front();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) free_queue.push_back(b);
  }
};

namespace {

using pkv::clear_error;
using pkv::set_error;

int64_t blocks_for(int64_t tokens, int32_t block_size) { return (tokens + block_size - 1) / block_size; }

}  // namespace

extern "C" {

int pkv_bm_create(int64_t num_blocks, int32_t block_size, pkv_block_manager **out) {
  if (!out) return set_error(PKV_ERR_INVALID, "out is null");
  *out = nullptr;
  if (block_size < 1) return set_error(PKV_ERR_INVALID, "block_size %d < 1", block_size);
  if (num_blocks < 1 || num_blocks > INT32_MAX / block_size)
    return set_error(PKV_ERR_INVALID, "num_blocks %lld outside [1, 2^31 / block_size)",
                     (long long)num_blocks);
  pkv_block_manager *bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return set_error(PKV_ERR_INVALID, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign((size_t)num_blocks, 0);
  for (int64_t b = 0; b < num_blocks; ++b) bm->free_queue.push_back((int32_t)b);
  *out = bm;
  return clear_error();
}

int pkv_bm_destroy(pkv_block_manager *bm) {
  delete bm;
  return clear_error();
}

int pkv_bm_add_sequence(pkv_block_manager *bm, int64_t seq_id, int32_t num_tokens) {
  if (!bm) return set_error(PKV_ERR_INVALID, "manager is null");
  if (num_tokens < 0) return set_error(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  std::lock_guard<std::mutex> lock(bm->mu);
  if (bm->seqs.count(seq_id)) return set_error(PKV_ERR_INVALID, "sequence %lld exists", (long long)seq_id);
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if ((int64_t)bm->free_queue.size() < need)
    return set_error(PKV_ERR_NO_BLOCKS, "sequence %lld needs %lld blocks, %zu free", (long long)seq_id,
                     (long long)need, bm->free_queue.size());
  pkv_block_manager::Sequence &sq = bm->seqs[seq_id];
  sq.tokens = num_tokens;
  sq.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) sq.blocks.push_back(bm->take());
  return clear_error();
}

int pkv_bm_fork(pkv_block_manager *bm, int64_t parent, int64_t child) {
  if (!bm) return set_error(PKV_ERR_INVALID, "manager is null");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "unknown sequence %lld", (long long)parent);
  if (bm->seqs.count(child)) return set_error(PKV_ERR_INVALID, "sequence %lld exists", (long long)child);
  pkv_block_manager::Sequence copy = it->second;
  for (int32_t b : copy.blocks) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(copy));
  return clear_error();
}

int pkv_bm_append_slots(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n, int32_t *slots,
                        int32_t *copies, int32_t *num_copies) {
  if (!bm) return set_error(PKV_ERR_INVALID, "manager is null");
  if (n < 0) return set_error(PKV_ERR_INVALID, "n %d < 0", n);
  if (n > 0 && (!seq_ids || !slots || !copies))
    return set_error(PKV_ERR_INVALID, "seq_ids, slots and copies must be non-null");
  if (!num_copies) return set_error(PKV_ERR_INVALID, "num_copies is null");
  std::lock_guard<std::mutex> lock(bm->mu);
  // Validate and count the blocks needed before changing anything. A last
  // block shared among several sequences of this call is copied for all of
  // them but the last one in the list, which then holds it alone: the count
  // follows the reference counts as the loop below will change them.
  std::unordered_set<int64_t> seen;
  std::unordered_map<int32_t, int32_t> count_after;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq_ids[i]);
    if (!seen.insert(seq_ids[i]).second)
      return set_error(PKV_ERR_INVALID, "sequence %lld appears twice", (long long)seq_ids[i]);
    const pkv_block_manager::Sequence &sq = it->second;
    if (sq.tokens + 1 > (int64_t)INT32_MAX) return set_error(PKV_ERR_INVALID, "sequence too long");
    if (sq.tokens % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t b = sq.blocks.back();
      auto c = count_after.find(b);
      const int32_t refs = c == count_after.end() ? bm->refcount[b] : c->second;
      if (refs > 1) {
        ++need;
        count_after[b] = refs - 1;
      }
    }
  }
  if ((int64_t)bm->free_queue.size() < need)
    return set_error(PKV_ERR_NO_BLOCKS, "%lld blocks needed, %zu free", (long long)need, bm->free_queue.size());
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_block_manager::Sequence &sq = bm->seqs[seq_ids[i]];
    const int64_t pos = sq.tokens;
    if (pos % bm->block_size == 0) {
      sq.blocks.push_back(bm->take());
    } else if (bm->refcount[sq.blocks.back()] > 1) {
      const int32_t src = sq.blocks.back();
      const int32_t dst = bm->take();
      bm->release(src);  // still referenced elsewhere: count > 0 after this
      sq.blocks.back() = dst;
      copies[2 * nc] = src;
      copies[2 * nc + 1] = dst;
      ++nc;
    }
    slots[i] = (int32_t)((int64_t)sq.blocks[(size_t)(pos / bm->block_size)] * bm->block_size +
                         pos % bm->block_size);
    sq.tokens = pos + 1;
  }
  *num_copies = nc;
  return clear_error();
}

int pkv_bm_free_sequence(pkv_block_manager *bm, int64_t seq_id) {
  if (!bm) return set_error(PKV_ERR_INVALID, "manager is null");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq_id);
  const std::vector<int32_t> &blocks = it->second.blocks;
  for (size_t i = blocks.size(); i-- > 0;) bm->release(blocks[i]);
  bm->seqs.erase(it);
  return clear_error();
}

int pkv_bm_num_free(pkv_block_manager *bm, int64_t *num_free) {
  if (!bm || !num_free) return set_error(PKV_ERR_INVALID, "null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  *num_free = (int64_t)bm->free_queue.size();
  return clear_error();
}

int pkv_bm_refcount(pkv_block_manager *bm, int32_t block, int32_t *count) {
  if (!bm || !count) return set_error(PKV_ERR_INVALID, "null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  if (block < 0 || block >= bm->num_blocks) return set_error(PKV_ERR_INVALID, "block %d outside the pool", block);
  *count = bm->refcount[(size_t)block];
  return clear_error();
}

int pkv_bm_sequence(pkv_block_manager *bm, int64_t seq_id, int32_t *num_tokens, int32_t *num_blocks,
                    int32_t *blocks, int32_t capacity) {
  if (!bm || !num_tokens || !num_blocks || capacity < 0 || (capacity > 0 && !blocks))
    return set_error(PKV_ERR_INVALID, "null argument or negative capacity");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq_id);
  const pkv_block_manager::Sequence &sq = it->second;
  *num_tokens = (int32_t)sq.tokens;
  *num_blocks = (int32_t)sq.blocks.size();
  for (int32_t i = 0; i < capacity && i < (int32_t)sq.blocks.size(); ++i) blocks[i] = sq.blocks[(size_t)i];
  return clear_error();
}

int pkv_bm_build_tables(pkv_block_manager *bm, const int64_t *seq_ids, int32_t n, int32_t max_blocks,
                        int32_t *block_tables, int32_t *seq_lens) {
  if (!bm || n < 0 || max_blocks < 1) return set_error(PKV_ERR_INVALID, "bad manager, n or max_blocks");
  if (n > 0 && (!seq_ids || !block_tables || !seq_lens)) return set_error(PKV_ERR_INVALID, "null array");
  std::lock_guard<std::mutex> lock(bm->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return set_error(PKV_ERR_INVALID, "unknown sequence %lld", (long long)seq_ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return set_error(PKV_ERR_INVALID, "sequence %lld has %zu blocks > max_blocks %d", (long long)seq_ids[i],
                       it->second.blocks.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_block_manager::Sequence &sq = bm->seqs[seq_ids[i]];
    int32_t *row = block_tables + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)sq.blocks.size() ? sq.blocks[(size_t)j] : -1;
    seq_lens[i] = (int32_t)sq.tokens;
  }
  return clear_error();
}

int pkv_bm_free_queue(pkv_block_manager *bm, int32_t *blocks, int64_t capacity) {
  if (!bm || capacity < 0 || (capacity > 0 && !blocks)) return set_error(PKV_ERR_INVALID, "bad argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  int64_t i = 0;
  for (auto it = bm->free_queue.begin(); it != bm->free_queue.end() && i < capacity; ++it) blocks[i++] = *it;
  return clear_error();
}

}  // extern "C"
