// Host checks of the device-data preconditions (include/pagedkv_debug.h),
// and the PKV_DEBUG=1 mode that runs them inside every call.
//
// The arrays they check define paged addressing ("LLM Engineering (5)",
// "Paged attention": token t of a sequence lives in row t % bs of block
// block_tables[b][t / bs]; "Block manager: how paging works": a new token is
// written to a slot of its sequence's tail block).

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/pagedkv_debug.h"
#include "pkv_debug.hpp"
#include "pkv_host.hpp"

using pkv::fail;
using pkv::ok;

extern "C" {

pkv_status pkv_check_block_tables(const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t max_blocks_per_seq,
                                  int32_t block_size, int64_t num_blocks) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "check_block_tables: invalid sizes");
  if (num_seqs > 0 && (!block_tables || !context_lens))
    return fail(PKV_ERR_INVALID, "check_block_tables: null array");
  const int64_t max_len = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t L = context_lens[b];
    if (L < 0 || L > max_len)
      return fail(PKV_ERR_INVALID, "context_lens[%d] = %lld outside [0, %lld]", b,
                  static_cast<long long>(L), static_cast<long long>(max_len));
    const int64_t n = (L + block_size - 1) / block_size;
    const int32_t* row = block_tables + static_cast<int64_t>(b) * max_blocks_per_seq;
    for (int64_t j = 0; j < n; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(PKV_ERR_INVALID, "block_tables[%d][%lld] = %d outside [0, %lld)", b,
                    static_cast<long long>(j), row[j], static_cast<long long>(num_blocks));
  }
  return ok();
}

pkv_status pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens,
                                  int32_t block_size, int64_t num_blocks) {
  if (num_tokens < 0 || block_size < 1 || num_blocks < 1)
    return fail(PKV_ERR_INVALID, "check_slot_mapping: invalid sizes");
  if (num_tokens > 0 && !slot_mapping) return fail(PKV_ERR_INVALID, "check_slot_mapping: null array");
  const int64_t slots = num_blocks * block_size;
  std::vector<std::pair<int64_t, int64_t>> used;  // (slot, token)
  used.reserve(static_cast<size_t>(num_tokens));
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= slots)
      return fail(PKV_ERR_INVALID, "slot_mapping[%lld] = %lld outside [0, %lld)", static_cast<long long>(t),
                  static_cast<long long>(s), static_cast<long long>(slots));
    used.emplace_back(s, t);
  }
  std::sort(used.begin(), used.end());
  for (size_t i = 1; i < used.size(); ++i)
    if (used[i].first == used[i - 1].first)
      return fail(PKV_ERR_INVALID, "tokens %lld and %lld share slot %lld", static_cast<long long>(used[i - 1].second),
                  static_cast<long long>(used[i].second), static_cast<long long>(used[i].first));
  return ok();
}

pkv_status pkv_check_query_start(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_queries_per_seq) {
  if (num_seqs < 0 || num_query_tokens < 0)
    return fail(PKV_ERR_INVALID, "check_query_start: invalid sizes");
  if (!query_start || (num_seqs > 0 && !context_lens))
    return fail(PKV_ERR_INVALID, "check_query_start: null array");
  if (query_start[0] != 0) return fail(PKV_ERR_INVALID, "query_start[0] = %d, not 0", query_start[0]);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = static_cast<int64_t>(query_start[b + 1]) - query_start[b];
    if (n < 0) return fail(PKV_ERR_INVALID, "query_start decreases at %d", b + 1);
    if (n > max_queries_per_seq)
      return fail(PKV_ERR_INVALID, "sequence %d has %lld new tokens, max_queries_per_seq is %d", b,
                  static_cast<long long>(n), max_queries_per_seq);
    if (n > context_lens[b])
      return fail(PKV_ERR_INVALID, "sequence %d has %lld new tokens in a context of %d", b,
                  static_cast<long long>(n), context_lens[b]);
  }
  if (query_start[num_seqs] != num_query_tokens)
    return fail(PKV_ERR_INVALID, "query_start[%d] = %d, not num_query_tokens = %d", num_seqs,
                query_start[num_seqs], num_query_tokens);
  return ok();
}

pkv_status pkv_check_groups(const int32_t* group_start, const int32_t* group_shared_blocks,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                            int32_t num_groups, int32_t max_group_size, int32_t max_shared_blocks) {
  if (num_seqs < 0 || num_groups < 0 || max_blocks_per_seq < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID, "check_groups: invalid sizes");
  if (!group_start || (num_groups > 0 && !group_shared_blocks) ||
      (num_seqs > 0 && (!block_tables || !context_lens)))
    return fail(PKV_ERR_INVALID, "check_groups: null array");
  if (group_start[0] != 0) return fail(PKV_ERR_INVALID, "group_start[0] = %d, not 0", group_start[0]);
  if (group_start[num_groups] != num_seqs)
    return fail(PKV_ERR_INVALID, "group_start[%d] = %d, not num_seqs = %d", num_groups,
                group_start[num_groups], num_seqs);
  // non-decreasing from 0 to num_seqs: every member index below is in range
  for (int32_t g = 0; g < num_groups; ++g)
    if (group_start[g + 1] < group_start[g])
      return fail(PKV_ERR_INVALID, "group_start decreases at %d", g + 1);
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t a = group_start[g], e = group_start[g + 1];
    if (e - a > max_group_size)
      return fail(PKV_ERR_INVALID, "group %d has %d sequences, max_group_size is %d", g, e - a,
                  max_group_size);
    if (e == a) continue;
    // the group's shared span in blocks, as the kernels compute it
    const int32_t nb = std::min(std::min(std::max(group_shared_blocks[g], 0), max_shared_blocks),
                                context_lens[a] / block_size);
    const int32_t* lead = block_tables + static_cast<int64_t>(a) * max_blocks_per_seq;
    for (int32_t m = a + 1; m < e; ++m) {
      if (context_lens[m] < static_cast<int64_t>(nb) * block_size)
        return fail(PKV_ERR_INVALID, "sequence %d of group %d has %d tokens, fewer than the %d shared", m, g,
                    context_lens[m], nb * block_size);
      const int32_t* row = block_tables + static_cast<int64_t>(m) * max_blocks_per_seq;
      for (int32_t j = 0; j < nb; ++j)
        if (row[j] != lead[j])
          return fail(PKV_ERR_INVALID, "sequence %d of group %d: block_tables[%d][%d] = %d, the first member's is %d",
                      m, g, m, j, row[j], lead[j]);
    }
  }
  return ok();
}

}  // extern "C"

namespace pkv {

bool debug_checks_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("PKV_DEBUG");
    return e != nullptr && std::strcmp(e, "1") == 0;
  }();
  return on;
}

namespace {

// n elements of a device array -> host (synchronises the stream).
template <typename T>
pkv_status fetch(const T* dev, size_t n, hipStream_t s, std::vector<T>* out) {
  out->resize(n);
  if (n == 0) return PKV_OK;
  hipError_t e = hipMemcpyAsync(out->data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "PKV_DEBUG copy of device data failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace

pkv_status debug_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                              hipStream_t s, std::vector<int32_t>* tables, std::vector<int32_t>* lens) {
  pkv_status st = fetch(block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, s, tables);
  if (st == PKV_OK) st = fetch(context_lens, static_cast<size_t>(num_seqs), s, lens);
  if (st != PKV_OK) return st;
  return pkv_check_block_tables(tables->data(), lens->data(), num_seqs, max_blocks_per_seq, block_size,
                                num_blocks);
}

pkv_status debug_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int32_t block_size,
                             int64_t num_blocks, hipStream_t s) {
  std::vector<int64_t> slots;
  const pkv_status st = fetch(slot_mapping, static_cast<size_t>(num_tokens), s, &slots);
  if (st != PKV_OK) return st;
  return pkv_check_slot_mapping(slots.data(), num_tokens, block_size, num_blocks);
}

pkv_status debug_check_query_start(const int32_t* query_start, const std::vector<int32_t>& lens,
                                   int32_t num_seqs, int32_t num_query_tokens, int32_t max_queries,
                                   hipStream_t s) {
  std::vector<int32_t> qs;
  const pkv_status st = fetch(query_start, static_cast<size_t>(num_seqs) + 1, s, &qs);
  if (st != PKV_OK) return st;
  return pkv_check_query_start(qs.data(), lens.data(), num_seqs, num_query_tokens, max_queries);
}

pkv_status debug_check_groups(const int32_t* group_start, const int32_t* group_shared_blocks,
                              const std::vector<int32_t>& tables, const std::vector<int32_t>& lens,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                              int32_t num_groups, int32_t max_group_size, int32_t max_shared_blocks,
                              hipStream_t s, bool step) {
  std::vector<int32_t> gs, gsb;
  pkv_status st = fetch(group_start, static_cast<size_t>(num_groups) + 1, s, &gs);
  if (st == PKV_OK) st = fetch(group_shared_blocks, static_cast<size_t>(num_groups), s, &gsb);
  if (st != PKV_OK) return st;
  st = pkv_check_groups(gs.data(), gsb.data(), tables.data(), lens.data(), num_seqs, max_blocks_per_seq,
                        block_size, num_groups, max_group_size, max_shared_blocks);
  if (st != PKV_OK || !step) return st;
  // the fused step writes each member's new token at L - 1: never inside
  // the span its group shares
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t lead = gs[g];
    if (lead >= gs[g + 1]) continue;
    const int64_t span =
        static_cast<int64_t>(std::min(std::min(std::max(gsb[g], 0), max_shared_blocks), lens[lead] / block_size)) *
        block_size;
    for (int32_t b = lead; b < gs[g + 1]; ++b)
      if (lens[b] > 0 && lens[b] - 1 < span)
        return fail(PKV_ERR_INVALID, "sequence %d: new token at %d lies in its group's shared span of %lld tokens",
                    b, lens[b] - 1, static_cast<long long>(span));
  }
  return ok();
}

}  // namespace pkv
