/*
 * pagedkv_debug — checks of the device-data preconditions of libpagedkv.so.
 *
 * The attention and cache-write calls take block tables, context lengths,
 * slot mappings, query ranges and group arrays in device memory and do not
 * read them on the host: a block id outside the pool, a context longer than
 * its table or two tokens written to one slot is undefined behaviour there
 * (pagedkv.h lists the preconditions).  The functions below check those
 * preconditions on host copies of the arrays, for callers that want to
 * validate what they are about to pass.
 *
 * With the environment variable PKV_DEBUG set to 1 (read once per process),
 * every attention and cache-write call of pagedkv.h copies its device
 * arrays to the host on its stream, synchronises the stream and runs these
 * checks before launching anything; a violation returns PKV_ERR_INVALID
 * (pkv_last_error() names the first offending entry) and launches nothing.
 * Without it, no call synchronises.  The mode is for eager debugging runs:
 * under stream capture the copies fail and the call returns PKV_ERR_HIP.
 *
 * Every function returns PKV_OK or PKV_ERR_INVALID; all pointers are host
 * memory.
 */
#ifndef PAGEDKV_DEBUG_H
#define PAGEDKV_DEBUG_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Paged addressing ("LLM Engineering (5)", "Paged attention": a sequence's
 * token t lives in row t % bs of block block_tables[b][t / bs]).
 *   block_tables [num_seqs][max_blocks_per_seq], context_lens [num_seqs].
 * Checks 0 <= context_lens[b] <= max_blocks_per_seq * block_size and that
 * every entry a context uses (the first ceil(L / block_size) of its row) is
 * in [0, num_blocks); entries past those are never read and not checked.
 */
pkv_status pkv_check_block_tables(const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t max_blocks_per_seq,
                                  int32_t block_size, int64_t num_blocks);

/*
 * A cache write's slots ("LLM Engineering (5)", "Block manager: how paging
 * works": a new token goes to a row of its sequence's tail block).
 *   slot_mapping [num_tokens]; a negative slot is skipped.
 * Checks every other slot is < num_blocks * block_size and that no two
 * tokens share a slot (their writes would race).
 */
pkv_status pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens,
                                  int32_t block_size, int64_t num_blocks);

/*
 * Multi-query ranges (pkv_paged_attention_multi_query).
 *   query_start [num_seqs + 1], context_lens [num_seqs].
 * Checks query_start[0] = 0, non-decreasing, query_start[num_seqs] =
 * num_query_tokens, and for every sequence n_b = query_start[b + 1] -
 * query_start[b] <= max_queries_per_seq and n_b <= context_lens[b] (its new
 * tokens are the last n_b positions of its context).
 */
pkv_status pkv_check_query_start(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_query_tokens,
                                 int32_t max_queries_per_seq);

/*
 * Shared-prefix groups (pkv_paged_attention_decode_cascade).
 *   group_start [num_groups + 1], group_shared_blocks [num_groups],
 *   block_tables and context_lens as above (already checked by
 *   pkv_check_block_tables).
 * Checks group_start[0] = 0, non-decreasing, group_start[num_groups] =
 * num_seqs, every group at most max_group_size sequences, and, with the
 * group's shared span S_g as pagedkv.h defines it, every member's context
 * holds at least S_g tokens and its first S_g / block_size table entries
 * equal the group's first member's.
 */
pkv_status pkv_check_groups(const int32_t* group_start, const int32_t* group_shared_blocks,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                            int32_t num_groups, int32_t max_group_size, int32_t max_shared_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_DEBUG_H */
