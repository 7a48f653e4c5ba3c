// Block manager of the paged KV cache (host bookkeeping; C ABI in
// include/pagedkv_blocks.h).
//
// "LLM Engineering (5)", "Block manager: how paging works": a pool of
// fixed-size physical blocks with a free list; a growing sequence takes a
// block off the free list when its tail block is full; reference counts let
// sequences share blocks (a forked sequence shares all of its parent's), and
// a write into a shared tail block first moves the sequence to a private
// copy (copy-on-write); a preempted sequence's blocks go to host memory and
// come back later.  Every call checks its arguments and its block needs
// before changing anything, so a failed call leaves the manager as it was.
//
// Free blocks are handed out last-released-first from a stack whose initial
// order is the caller's `order` (first element first).

#include <cstdint>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv_blocks.h"
#include "pkv_host.hpp"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;  // device blocks, or host blocks when swapped out
    int64_t length = 0;
    bool swapped = false;
  };
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_dev;   // stack: back() is handed out next
  std::vector<int32_t> free_host;
  std::vector<int32_t> refcount;   // device blocks
  std::unordered_map<int64_t, Seq> seqs;
  int64_t next_id = 0;

  int32_t pop_dev() {
    const int32_t b = free_dev.back();
    free_dev.pop_back();
    refcount[b] = 1;
    return b;
  }
  void release_dev(int32_t b) {
    if (--refcount[b] == 0) free_dev.push_back(b);
  }
  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

using pkv::fail;
using pkv::ok;

extern "C" {

pkv_status pkv_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks,
                         const int32_t* order, pkv_block_manager** out) {
  if (!out) return fail(PKV_ERR_INVALID, "bm_create: null out");
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0)
    return fail(PKV_ERR_INVALID, "bm_create: num_blocks must be in [1, 2^31) and block_size > 0");
  if (num_host_blocks < 0 || num_host_blocks > INT32_MAX)
    return fail(PKV_ERR_INVALID, "bm_create: num_host_blocks must be in [0, 2^31)");
  auto* bm = new pkv_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(static_cast<size_t>(num_blocks), 0);
  bm->free_dev.resize(static_cast<size_t>(num_blocks));
  std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
  for (int64_t i = 0; i < num_blocks; ++i) {
    const int32_t b = order ? order[i] : static_cast<int32_t>(i);
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return fail(PKV_ERR_INVALID, "bm_create: order is not a permutation of the block ids");
    }
    seen[b] = 1;
    bm->free_dev[static_cast<size_t>(num_blocks - 1 - i)] = b;  // order[0] on top
  }
  bm->free_host.resize(static_cast<size_t>(num_host_blocks));
  for (int64_t i = 0; i < num_host_blocks; ++i)
    bm->free_host[static_cast<size_t>(i)] = static_cast<int32_t>(num_host_blocks - 1 - i);
  *out = bm;
  return ok();
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int64_t pkv_bm_num_free(const pkv_block_manager* bm) {
  return bm ? static_cast<int64_t>(bm->free_dev.size()) : -1;
}

int64_t pkv_bm_num_free_host(const pkv_block_manager* bm) {
  return bm ? static_cast<int64_t>(bm->free_host.size()) : -1;
}

pkv_status pkv_bm_new_sequence(pkv_block_manager* bm, int64_t* seq) {
  if (!bm || !seq) return fail(PKV_ERR_INVALID, "bm_new_sequence: null argument");
  *seq = bm->next_id++;
  bm->seqs[*seq] = pkv_block_manager::Seq();
  return ok();
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t* child) {
  if (!bm || !child) return fail(PKV_ERR_INVALID, "bm_fork: null argument");
  const auto* p = bm->find(parent);
  if (!p) return fail(PKV_ERR_INVALID, "bm_fork: unknown sequence %lld", static_cast<long long>(parent));
  if (p->swapped) return fail(PKV_ERR_INVALID, "bm_fork: sequence is swapped out");
  pkv_block_manager::Seq c;
  c.table = p->table;
  c.length = p->length;
  for (int32_t b : c.table) ++bm->refcount[b];
  *child = bm->next_id++;
  bm->seqs[*child] = std::move(c);
  return ok();
}

pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PKV_ERR_INVALID, "bm_free_sequence: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end())
    return fail(PKV_ERR_INVALID, "bm_free_sequence: unknown sequence %lld", static_cast<long long>(seq));
  if (it->second.swapped) {
    for (int32_t h : it->second.table) bm->free_host.push_back(h);
  } else {
    for (int32_t b : it->second.table) bm->release_dev(b);
  }
  bm->seqs.erase(it);
  return ok();
}

pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int64_t n, int64_t* slots,
                         int32_t* copies, int32_t max_copies, int32_t* num_copies) {
  if (!bm || !num_copies || (n > 0 && !slots))
    return fail(PKV_ERR_INVALID, "bm_append: null argument");
  auto* s = bm->find(seq);
  if (!s) return fail(PKV_ERR_INVALID, "bm_append: unknown sequence %lld", static_cast<long long>(seq));
  if (s->swapped) return fail(PKV_ERR_INVALID, "bm_append: sequence is swapped out");
  if (n < 0) return fail(PKV_ERR_INVALID, "bm_append: n must be >= 0");
  *num_copies = 0;
  if (n == 0) return ok();
  const int64_t bs = bm->block_size;
  const int64_t row = s->length % bs;
  // blocks this call takes: a private copy of a shared, partly written tail,
  // then one per block boundary the new tokens cross
  const bool cow = row != 0 && bm->refcount[s->table.back()] > 1;
  const int64_t first = row == 0 ? 0 : (n < bs - row ? n : bs - row);
  const int64_t need = (cow ? 1 : 0) + (n - first + bs - 1) / bs;
  if (cow && (max_copies < 1 || !copies))
    return fail(PKV_ERR_INVALID, "bm_append: a copy-on-write needs room for one copy");
  if (need > static_cast<int64_t>(bm->free_dev.size()))
    return fail(PKV_ERR_NO_BLOCKS, "bm_append: %lld free blocks, %lld needed",
                static_cast<long long>(bm->free_dev.size()), static_cast<long long>(need));
  if (cow) {
    const int32_t tail = s->table.back();
    const int32_t fresh = bm->pop_dev();
    copies[0] = tail;
    copies[1] = fresh;
    copies[2] = static_cast<int32_t>(row);
    *num_copies = 1;
    bm->release_dev(tail);
    s->table.back() = fresh;
  }
  for (int64_t done = 0; done < n;) {
    const int64_t r = s->length % bs;
    if (r == 0) s->table.push_back(bm->pop_dev());
    const int64_t blk = s->table.back();
    const int64_t take = (n - done < bs - r) ? n - done : bs - r;
    for (int64_t i = 0; i < take; ++i) slots[done + i] = blk * bs + r + i;
    s->length += take;
    done += take;
  }
  return ok();
}

int64_t pkv_bm_length(const pkv_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.length;
}

pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table,
                              int32_t max_blocks, int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_INVALID, "bm_block_table: null argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end())
    return fail(PKV_ERR_INVALID, "bm_block_table: unknown sequence %lld", static_cast<long long>(seq));
  if (it->second.swapped) return fail(PKV_ERR_INVALID, "bm_block_table: sequence is swapped out");
  const auto& t = it->second.table;
  if (static_cast<int64_t>(t.size()) > max_blocks || (!t.empty() && !table))
    return fail(PKV_ERR_INVALID, "bm_block_table: table of %zu blocks, room for %d", t.size(), max_blocks);
  for (size_t i = 0; i < t.size(); ++i) table[i] = t[i];
  *n = static_cast<int32_t>(t.size());
  return ok();
}

pkv_status pkv_bm_refcounts(const pkv_block_manager* bm, int32_t* refcounts) {
  if (!bm || !refcounts) return fail(PKV_ERR_INVALID, "bm_refcounts: null argument");
  for (size_t i = 0; i < bm->refcount.size(); ++i) refcounts[i] = bm->refcount[i];
  return ok();
}

pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                           int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_INVALID, "bm_swap_out: null argument");
  auto* s = bm->find(seq);
  if (!s) return fail(PKV_ERR_INVALID, "bm_swap_out: unknown sequence %lld", static_cast<long long>(seq));
  if (s->swapped) return fail(PKV_ERR_INVALID, "bm_swap_out: sequence is already swapped out");
  const int64_t cnt = static_cast<int64_t>(s->table.size());
  if (cnt > max_pairs || (cnt > 0 && !pairs))
    return fail(PKV_ERR_INVALID, "bm_swap_out: %lld pairs, room for %d", static_cast<long long>(cnt), max_pairs);
  if (cnt > static_cast<int64_t>(bm->free_host.size()))
    return fail(PKV_ERR_NO_BLOCKS, "bm_swap_out: %zu free host blocks, %lld needed",
                bm->free_host.size(), static_cast<long long>(cnt));
  for (int64_t i = 0; i < cnt; ++i) {
    const int32_t h = bm->free_host.back();
    bm->free_host.pop_back();
    pairs[2 * i] = s->table[i];
    pairs[2 * i + 1] = h;
    bm->release_dev(s->table[i]);
    s->table[i] = h;
  }
  s->swapped = true;
  *n = static_cast<int32_t>(cnt);
  return ok();
}

pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                          int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_INVALID, "bm_swap_in: null argument");
  auto* s = bm->find(seq);
  if (!s) return fail(PKV_ERR_INVALID, "bm_swap_in: unknown sequence %lld", static_cast<long long>(seq));
  if (!s->swapped) return fail(PKV_ERR_INVALID, "bm_swap_in: sequence is not swapped out");
  const int64_t cnt = static_cast<int64_t>(s->table.size());
  if (cnt > max_pairs || (cnt > 0 && !pairs))
    return fail(PKV_ERR_INVALID, "bm_swap_in: %lld pairs, room for %d", static_cast<long long>(cnt), max_pairs);
  if (cnt > static_cast<int64_t>(bm->free_dev.size()))
    return fail(PKV_ERR_NO_BLOCKS, "bm_swap_in: %zu free blocks, %lld needed", bm->free_dev.size(),
                static_cast<long long>(cnt));
  for (int64_t i = 0; i < cnt; ++i) {
    const int32_t b = bm->pop_dev();
    pairs[2 * i] = s->table[i];
    pairs[2 * i + 1] = b;
    bm->free_host.push_back(s->table[i]);
    s->table[i] = b;
  }
  s->swapped = false;
  *n = static_cast<int32_t>(cnt);
  return ok();
}

}  // extern "C"
