// PKV_DEBUG=1 mode: the C ABI's calls copy their device arrays to the host
// and check the device-data preconditions before launching anything.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/pagedkv.h"

namespace pkv {

// True when the environment variable PKV_DEBUG is "1" (read once).
bool debug_checks_enabled();

// Each copies the arrays it checks to the host (synchronising s) and
// returns PKV_OK, PKV_ERR_INVALID (a violated precondition) or PKV_ERR_HIP
// (the copy failed), with the message set.  The table check leaves its host
// copies in tables / lens for the group and query checks.
pkv_status debug_check_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                              hipStream_t s, std::vector<int32_t>* tables, std::vector<int32_t>* lens);
pkv_status debug_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int32_t block_size,
                             int64_t num_blocks, hipStream_t s);
pkv_status debug_check_query_start(const int32_t* query_start, const std::vector<int32_t>& lens,
                                   int32_t num_seqs, int32_t num_query_tokens, int32_t max_queries,
                                   hipStream_t s);
pkv_status debug_check_groups(const int32_t* group_start, const int32_t* group_shared_blocks,
                              const std::vector<int32_t>& tables, const std::vector<int32_t>& lens,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                              int32_t num_groups, int32_t max_group_size, int32_t max_shared_blocks,
                              hipStream_t s, bool step = false);

}  // namespace pkv
