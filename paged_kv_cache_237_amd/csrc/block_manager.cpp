// Host block manager of the paged KV cache: the bookkeeping that feeds the
// store and attention calls with block tables and slot mappings.
//
// What it implements (nano-vllm hub page, "KV Cache block management": the
// cache is cut into blocks of a fixed 256 tokens whose allocation and release
// are managed with reference counts; CSDN essay comparing nanoVLLM and vLLM,
// first section: a per-sequence block table maps logical blocks to physical
// ones, allocated on demand -- a sequence takes a new block each time its
// length reaches 256k+1):
//   * allocate(seq, n): a new sequence of n tokens owns ceil(n/256) blocks;
//   * append(seq): one more token; a new block when the new length is 256k+1,
//     and a private copy of the last block first if another sequence shares
//     it (copy-on-write: the caller copies the block with pa_copy_blocks);
//   * append_batch(seqs): append for a whole decode batch in one call, all
//     or nothing, returning the slot mapping and the copy pairs of the step;
//   * fork(parent, child): the child shares every block of the parent
//     (reference counts + 1), e.g. for parallel samples of one prompt;
//   * free(seq): reference counts - 1; blocks at zero return to the pool.
// Free blocks are handed out first-in first-out, starting from block 0.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.hpp"

namespace {

int bm_fail(int code, const std::string& msg) { return pa::report_error(code, msg); }

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;  // per physical block
  struct Seq {
    int64_t len = 0;
    std::vector<int32_t> blocks;
    uint64_t batch = 0;  // last append_batch call that listed it
  };
  std::unordered_map<int64_t, Seq> seqs;
  std::mutex mu;
  uint64_t batch_counter = 0;
  std::vector<Seq*> batch_rows;  // reused across append_batch calls

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  // One more token for s, with a free block guaranteed to be there when one
  // is needed; returns the token's slot, sets pair to (shared, fresh) when the
  // last block was copied.
  int32_t append_one(Seq& s, int32_t* pair) {
    const int64_t pos = s.len;  // 0-based position of the new token
    pair[0] = pair[1] = -1;
    if (pos % block_size == 0) {
      // the sequence reaches 256k+1 tokens: a new block
      s.blocks.push_back(take());
    } else {
      int32_t& last = s.blocks.back();
      if (ref[last] > 1) {
        // shared last block: take a private copy before writing into it
        const int32_t fresh = take();
        pair[0] = last;
        pair[1] = fresh;
        release(last);
        last = fresh;
      }
    }
    s.len = pos + 1;
    return int32_t(int64_t(s.blocks.back()) * block_size + pos % block_size);
  }
  // Blocks one append of s takes.
  bool needs_block(const Seq& s) const {
    return s.len % block_size == 0 || ref[s.blocks.back()] > 1;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size) {
  try {
    if (num_blocks <= 0 || block_size <= 0 || num_blocks * int64_t(block_size) > int64_t(INT32_MAX) + 1) {
      pa::report_error(PA_ERR_BAD_SHAPE,
                       "num_blocks and block_size must be positive, with every slot an int32");
      return nullptr;
    }
    auto* bm = new pa_block_manager;
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign(size_t(num_blocks), 0);
    for (int64_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(int32_t(b));
    pa::report_error(PA_OK, "");
    return bm;
  } catch (...) {
    pa::report_error(PA_ERR_BAD_SHAPE, "host allocation failed");
    return nullptr;
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int64_t pa_bm_num_free(pa_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return int64_t(bm->free_list.size());
}

int pa_bm_allocate(pa_block_manager* bm, int64_t seq, int64_t num_tokens) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  try {
    std::lock_guard<std::mutex> lock(bm->mu);
    if (num_tokens < 0) return bm_fail(PA_ERR_BAD_SHAPE, "num_tokens < 0");
    if (bm->seqs.count(seq)) return bm_fail(PA_ERR_BAD_SHAPE, "sequence " + std::to_string(seq) + " exists");
    const int64_t need = (num_tokens + bm->block_size - 1) / bm->block_size;
    if (need > int64_t(bm->free_list.size()))
      return bm_fail(PA_ERR_NO_BLOCKS, "sequence " + std::to_string(seq) + " needs " + std::to_string(need) +
                                           " blocks, " + std::to_string(bm->free_list.size()) + " free");
    pa_block_manager::Seq s;
    s.len = num_tokens;
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    bm->seqs.emplace(seq, std::move(s));
    pa::report_error(PA_OK, "");
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t* slot_out, int32_t* copy_pair_out) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  if (!slot_out || !copy_pair_out) return bm_fail(PA_ERR_NULL_PTR, "output pointer is NULL");
  try {
    std::lock_guard<std::mutex> lock(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(seq));
    if (bm->needs_block(it->second) && bm->free_list.empty())
      return bm_fail(PA_ERR_NO_BLOCKS, "no free block");
    *slot_out = bm->append_one(it->second, copy_pair_out);
    pa::report_error(PA_OK, "");
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                       int32_t* pairs_out, int32_t* n_pairs_out) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  if (!n_pairs_out) return bm_fail(PA_ERR_NULL_PTR, "n_pairs_out is NULL");
  if (n < 0) return bm_fail(PA_ERR_BAD_SHAPE, "n < 0");
  *n_pairs_out = 0;
  if (n == 0) return PA_OK;
  if (!seqs || !slots_out || !pairs_out) return bm_fail(PA_ERR_NULL_PTR, "seqs, slots_out or pairs_out is NULL");
  try {
    std::lock_guard<std::mutex> lock(bm->mu);
    auto& rows = bm->batch_rows;
    rows.assign(size_t(n), nullptr);
    const uint64_t stamp = ++bm->batch_counter;
    // Blocks the whole batch takes, counted before anything changes: one per
    // sequence that opens a block, and one per holder of a shared partial
    // last block that still shares it when its turn comes -- every holder in
    // the batch, except the last one when all holders are in it.
    int64_t need = 0;
    std::unordered_map<int32_t, int64_t> holders;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seqs[i]);
      if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(seqs[i]));
      auto& s = it->second;
      if (s.batch == stamp)
        return bm_fail(PA_ERR_BAD_SHAPE, "sequence " + std::to_string(seqs[i]) + " appears twice");
      s.batch = stamp;
      rows[size_t(i)] = &s;
      if (s.len % bm->block_size == 0) ++need;
      else if (bm->ref[s.blocks.back()] > 1) ++holders[s.blocks.back()];
    }
    for (const auto& h : holders) need += h.second == bm->ref[h.first] ? h.second - 1 : h.second;
    if (need > int64_t(bm->free_list.size()))
      return bm_fail(PA_ERR_NO_BLOCKS, "the batch needs " + std::to_string(need) + " blocks, " +
                                           std::to_string(bm->free_list.size()) + " free");
    int32_t n_pairs = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t pair[2];
      slots_out[i] = bm->append_one(*rows[size_t(i)], pair);
      if (pair[0] >= 0) {
        pairs_out[2 * n_pairs] = pair[0];
        pairs_out[2 * n_pairs + 1] = pair[1];
        ++n_pairs;
      }
    }
    *n_pairs_out = n_pairs;
    pa::report_error(PA_OK, "");
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  try {
    std::lock_guard<std::mutex> lock(bm->mu);
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(parent));
    if (bm->seqs.count(child)) return bm_fail(PA_ERR_BAD_SHAPE, "sequence " + std::to_string(child) + " exists");
    pa_block_manager::Seq s = it->second;
    for (int32_t b : s.blocks) ++bm->ref[b];
    bm->seqs.emplace(child, std::move(s));
    pa::report_error(PA_OK, "");
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(seq));
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  pa::report_error(PA_OK, "");
  return PA_OK;
}

int64_t pa_bm_seq_len(pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int pa_bm_block_table(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* table_out,
                      int32_t max_blocks_per_seq) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  if (n < 0 || max_blocks_per_seq <= 0) return bm_fail(PA_ERR_BAD_SHAPE, "bad table shape");
  if (n == 0) return PA_OK;
  if (!seqs || !table_out) return bm_fail(PA_ERR_NULL_PTR, "seqs or table_out is NULL");
  try {
    std::lock_guard<std::mutex> lock(bm->mu);
    auto& rows = bm->batch_rows;
    rows.assign(size_t(n), nullptr);
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seqs[i]);
      if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(seqs[i]));
      if (int64_t(it->second.blocks.size()) > max_blocks_per_seq)
        return bm_fail(PA_ERR_BAD_SHAPE, "sequence " + std::to_string(seqs[i]) + " has more than " +
                                             std::to_string(max_blocks_per_seq) + " blocks");
      rows[size_t(i)] = &it->second;
    }
    for (int32_t i = 0; i < n; ++i) {
      const auto& blocks = rows[size_t(i)]->blocks;
      int32_t* row = table_out + int64_t(i) * max_blocks_per_seq;
      std::copy(blocks.begin(), blocks.end(), row);
      std::fill(row + blocks.size(), row + max_blocks_per_seq, -1);
    }
    pa::report_error(PA_OK, "");
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_BAD_SHAPE, "host allocation failed");
  }
}

int pa_bm_slot_mapping(pa_block_manager* bm, int64_t seq, int64_t first_pos, int64_t count,
                       int32_t* slots_out) {
  if (!bm) return bm_fail(PA_ERR_NULL_PTR, "block manager is NULL");
  if (count < 0 || first_pos < 0) return bm_fail(PA_ERR_BAD_SHAPE, "negative position or count");
  if (count == 0) return PA_OK;
  if (!slots_out) return bm_fail(PA_ERR_NULL_PTR, "slots_out is NULL");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bm_fail(PA_ERR_BAD_SHAPE, "no sequence " + std::to_string(seq));
  const auto& s = it->second;
  if (first_pos + count > s.len) return bm_fail(PA_ERR_BAD_SHAPE, "positions past the sequence");
  for (int64_t i = 0; i < count; ++i) {
    const int64_t p = first_pos + i;
    slots_out[i] = int32_t(int64_t(s.blocks[size_t(p / bm->block_size)]) * bm->block_size +
                           p % bm->block_size);
  }
  pa::report_error(PA_OK, "");
  return PA_OK;
}

}  // extern "C"
