/*
 * pagedkv_blocks — the block manager of a paged KV cache, and the kernel
 * that moves whole blocks, in libpagedkv.so.
 *
 * [ENG5] "LLM Engineering (5)", "Block manager: how paging works": a pool of
 * fixed-size physical blocks with a free list; a growing request takes a
 * block off the free list and appends its id to its block table when its
 * tail block is full; blocks are reference-counted so requests can share
 * them, and a request about to write into a shared block first copies it
 * (copy-on-write); under memory pressure a victim request's blocks are
 * copied to pinned host memory over PCIe and its GPU blocks freed, to be
 * copied back when memory frees up.  [ENG5] "Paged attention": requests
 * with a common prefix share physical blocks.
 *
 * The manager is host bookkeeping only (no device calls); the data moves
 * with pkv_copy_blocks, from the (src, dst) pairs the manager returns.
 * Slots follow pagedkv.h: slot = physical_block * block_size + row.
 */
#ifndef PAGEDKV_BLOCKS_H
#define PAGEDKV_BLOCKS_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

/*
 * A manager over num_blocks device blocks of block_size tokens, and
 * num_host_blocks host blocks (the swap space; may be 0).  order
 * (host int32 [num_blocks], or NULL for 0, 1, 2, ...) is the order in which
 * free device blocks are handed out first; it must be a permutation of
 * 0 .. num_blocks-1.  *out receives the manager (the caller owns it; free
 * it with pkv_bm_destroy).  PKV_ERR_INVALID for non-positive sizes, a
 * negative host pool, a bad order or a null out.
 */
pkv_status pkv_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks,
                         const int32_t* order, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Free device blocks / free host blocks (-1 for a null manager). */
int64_t pkv_bm_num_free(const pkv_block_manager* bm);
int64_t pkv_bm_num_free_host(const pkv_block_manager* bm);

/* A new, empty sequence; its id goes to *seq (ids are never reused). */
pkv_status pkv_bm_new_sequence(pkv_block_manager* bm, int64_t* seq);

/*
 * A new sequence sharing every block of `parent` (each block's refcount
 * + 1), with the parent's length.  PKV_ERR_INVALID for an unknown or
 * swapped-out parent.
 */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t* child);

/*
 * Drop the sequence: one reference per block (device, or host if it is
 * swapped out); a block returns to its free list when its count reaches 0.
 */
pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq);

/*
 * Append n >= 0 tokens to `seq`; slots[0 .. n-1] (host int64) receive their
 * slots in order.  A full tail block gets a fresh block appended; a tail
 * block shared with another sequence (refcount > 1) that still has room is
 * first replaced by a fresh private block, and the copy that must happen
 * before the new tokens are written is reported as (src block, dst block,
 * rows already written) in copies (host int32 [max_copies][3]; at most one
 * per call), *num_copies receiving the count.  All-or-nothing: when the
 * free list cannot supply every block the call needs, PKV_ERR_NO_BLOCKS is
 * returned and nothing changes.  PKV_ERR_INVALID for an unknown or
 * swapped-out sequence, n < 0, null outputs, or max_copies < 1 when a copy
 * is needed.
 */
pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int64_t n, int64_t* slots,
                         int32_t* copies, int32_t max_copies, int32_t* num_copies);

/* Tokens held by `seq` (-1 for an unknown sequence). */
int64_t pkv_bm_length(const pkv_block_manager* bm, int64_t seq);

/*
 * The sequence's block table (device block ids, host int32 [max_blocks]);
 * *n receives its length.  PKV_ERR_INVALID for an unknown or swapped-out
 * sequence or a table longer than max_blocks.
 */
pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table,
                              int32_t max_blocks, int32_t* n);

/* Reference counts of all device blocks (host int32 [num_blocks]). */
pkv_status pkv_bm_refcounts(const pkv_block_manager* bm, int32_t* refcounts);

/*
 * Swap `seq` out: every one of its device blocks gets a host block; pairs
 * (host int32 [max_pairs][2]) receive (device block, host block) in table
 * order, *n the count; then its device references are dropped (blocks it
 * shared stay with their other owners) and it holds host blocks only.
 * Copy the pairs with pkv_copy_blocks (device pool -> host pool) before any
 * freed block is reused.  All-or-nothing: PKV_ERR_NO_BLOCKS when the host
 * pool is short.  PKV_ERR_INVALID for an unknown or already swapped-out
 * sequence, or max_pairs below its block count.
 */
pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                           int32_t* n);

/*
 * Swap `seq` back in: fresh private device blocks for its host blocks;
 * pairs receive (host block, device block) in table order, *n the count;
 * the host blocks return to the host pool.  Copy the pairs with
 * pkv_copy_blocks (host pool -> device pool) before attending.
 * All-or-nothing: PKV_ERR_NO_BLOCKS when the device pool is short.
 */
pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                          int32_t* n);

/*
 * Copy whole blocks between two pools of the layout in pagedkv.h: for each
 * pair i, block pairs[2i] of the source pool goes to block pairs[2i+1] of
 * the destination pool — its K tile rows [Hkv][bs][D], V tiles
 * [Hkv][bs/4][D][4] (INT4: [Hkv][bs][D/2] and [Hkv][bs/4][D/2][4] bytes)
 * and, for int8 / FP8 / INT4 caches, its k_scale / v_scale rows [Hkv][bs].
 * Pools may be the same (copy-on-write) or one of them pinned host memory
 * the device can address (swapping; e.g. hipHostMalloc'd, the kernel reads
 * or writes it over the host link).  pairs: device int32 [n][2].
 *   dtype: PKV_F32, PKV_BF16, PKV_I8, PKV_FP8, PKV_FP8_E5M2 or PKV_I4;
 *   scale pointers required for the coded kinds and NULL otherwise.  n >= 0 (0: no launch).
 * Not checked (device data): block ids inside their pools; no destination
 * block written twice, none both read and written by one call.
 */
pkv_status pkv_copy_blocks(void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                           const void* src_k, const void* src_v, const float* src_k_scale,
                           const float* src_v_scale, const int32_t* pairs, int32_t n,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_BLOCKS_H */
