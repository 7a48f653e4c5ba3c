/*
 * pagedkv — paged KV cache decode attention for AMD MI355X (gfx950).
 *
 * C ABI of libpagedkv.so.  Every pointer argument is device memory owned by
 * the caller unless stated otherwise; the library never allocates or frees
 * device memory and retains no pointer after a call returns (the only
 * resources it creates are, on the first cascade decode on a device, one
 * stream and two events for that device, kept until the process ends).
 * Every call is asynchronous on the
 * given HIP stream (a hipStream_t passed as void*, NULL = the default stream)
 * and never synchronises it (except in the PKV_DEBUG=1 checking mode of
 * pagedkv_debug.h).  A non-OK return launches nothing and has no
 * side effects, except PKV_ERR_HIP, which reports a failed launch.  Errors
 * that happen while a kernel runs surface at the caller's next
 * synchronisation.  pkv_last_error() gives the text of the last failure on
 * the calling thread.
 *
 * Sources the operations follow (web pages, cited by title and section):
 *   [ENG5]   "LLM Engineering (5): core techniques of inference
 *            optimization" (chenk.top): "Two phases with very different
 *            characteristics" (decode reads the whole KV cache each step),
 *            "Paged attention" (fixed 16-token blocks, per-sequence block
 *            tables, 47 tokens -> 16+16+15), "Block manager: how paging
 *            works" (append a block to the table, copy-on-write sharing),
 *            "KV-cache quantization" (per-token-per-head scales computed
 *            online), "INT8 weight-only quantization" (q = round(x / s)),
 *            "SGLang and RadixAttention" (the longest shared prefix is
 *            reused, only the rest is computed per request), "Orca's
 *            iteration-level scheduling" (chunked prefill) and
 *            "Speculative decoding" (k + 1 positions in one pass).
 *   [LAYERS] four-layer inference-optimization article
 *            (gsyq.cn/news/366077), 2.2 (block size 16 or 32) and 2.3
 *            (per-token scales; K and V quantized separately).
 *
 * Data layout (shared by all entry points).  Notation: NB = num_blocks,
 * Hkv = num_kv_heads, bs = block_size, D = head_dim, H = num_heads,
 * G = H / Hkv, B = num_seqs, MB = max_blocks_per_seq, T = num_tokens.
 *   k_cache      [NB][Hkv][bs][D]   one row of D elements per token
 *   v_cache      [NB][Hkv][bs/4][D][4]  each (block, kv-head) tile in groups
 *                                   of 4 consecutive tokens, dim-major inside
 *                                   a group: element (token row r, dim d) at
 *                                   ((r / 4) * D + d) * 4 + r % 4
 *   k_scale,
 *   v_scale      [NB][Hkv][bs] fp32 (int8, FP8 and INT4 caches only)
 *   FP8 caches hold E4M3 codes (PKV_FP8) or E5M2 codes (PKV_FP8_E5M2).
 *   INT4 caches hold two codes per byte, two consecutive head dims of one
 *   token (dim 2j in the low nibble, 2j + 1 in the high nibble, 4-bit two's
 *   complement), so their tiles are k_cache [NB][Hkv][bs][D/2] and
 *   v_cache [NB][Hkv][bs/4][D/2][4] (byte ((r / 4) * D/2 + j) * 4 + r % 4:
 *   dims 2j, 2j + 1 of token r).
 *   block_tables [B][MB] int32      logical block j of sequence b lives in
 *                                   physical block block_tables[b*MB + j];
 *                                   entries past the sequence's last block
 *                                   are never read
 *   context_lens [B] int32          tokens to attend, including the newest
 *   slot_mapping [T] int64          slot = physical_block * bs + row; < 0: skip
 *   q, out       [B][H][D]          query head h reads kv-head h / G
 *   new k, v     [T][Hkv][D]
 * All arrays are dense and row-major with exactly these shapes.
 *
 * Device-data preconditions that are NOT checked by default (a violation is
 * undefined behaviour, typically a memory fault): every block id a sequence
 * uses is in [0, NB); context_lens[b] <= MB * bs; every slot is < NB * bs;
 * no two tokens of one write call share a slot (they would race).  With the
 * environment variable PKV_DEBUG=1 every attention and cache-write call
 * checks them, and the group and query arrays below, on host copies before
 * launching (synchronising its stream); pagedkv_debug.h declares the same
 * checks for callers to run on host arrays.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,      /* bad pointer, size or scalar argument        */
  PKV_ERR_UNSUPPORTED = 2,  /* valid, but not a built variant              */
  PKV_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required  */
  PKV_ERR_HIP = 4,          /* the HIP runtime refused a launch            */
  PKV_ERR_NO_BLOCKS = 5     /* block manager: a pool is out of free blocks */
} pkv_status;

typedef enum {
  PKV_F32 = 0,   /* IEEE binary32                         */
  PKV_BF16 = 1,  /* bfloat16, 16-bit patterns             */
  PKV_I8 = 2,    /* int8 codes with an fp32 per-row scale */
  PKV_FP8 = 3,   /* FP8 E4M3 codes (OCP: bias 7, largest finite 448, no
                    infinities) with an fp32 per-row scale              */
  PKV_I4 = 4,    /* INT4 codes in [-7, 7], two per byte (layout above),
                    with an fp32 per-row scale                          */
  PKV_FP8_E5M2 = 5 /* FP8 E5M2 codes (bias 15, largest finite 57344) with
                      an fp32 per-row scale                             */
} pkv_dtype;

/*
 * Slot-scatter cache write ([ENG5] "Block manager: how paging works": a new
 * token goes to the next slot of its sequence's tail block).
 *   For every token t with s = slot_mapping[t] >= 0, row r = s % bs and
 *   every kv-head h:
 *     k_cache[s / bs][h][r][:] = k[t][h][:]
 *     v_cache[s / bs][h][r / 4][:][r % 4] = v[t][h][:]
 *   The copy is bit-exact.  dtype is PKV_F32 or PKV_BF16 (the element type of
 *   k, v and both caches).  head_dim in {64, 128}; block_size in {16, 32};
 *   num_tokens >= 0 (0: no-op).  Errors: PKV_ERR_INVALID for null pointers
 *   or non-positive sizes, PKV_ERR_UNSUPPORTED for other dtypes or sizes.
 */
pkv_status pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, pkv_dtype dtype, void* stream);

/*
 * Quantising cache write for an int8 KV cache ([ENG5] "KV-cache
 * quantization", [LAYERS] 2.3, [ENG5] "INT8 weight-only quantization").
 *   Each (token, kv-head) row x of k (and, separately, of v), fp32, becomes
 *     a = max_d |x_d|;  s = a / 127 (IEEE fp32 division);
 *     code_d = clamp(rint(x_d / s), -127, 127)  (round half to even);
 *     s == 0 (a == 0, or a / 127 underflows) gives all codes 0.
 *   Codes go to the slot as in pkv_kv_cache_write; s goes to
 *   k_scale[s_slot / bs][h][s_slot % bs] (v_scale likewise).  Inputs must be
 *   finite.  Bit-exact: identical codes and scales for identical inputs.
 */
pkv_status pkv_kv_cache_write_int8(const float* k, const float* v, int8_t* k_cache,
                                   int8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, void* stream);

/*
 * Quantising cache write for an FP8 KV cache ([ENG5] "KV-cache
 * quantization": FP8 KV caches with per-token scales computed online;
 * [LAYERS] 2.3: K and V quantized separately).
 *   Each (token, kv-head) row x of k (and, separately, of v), fp32, becomes
 *     a = max_d |x_d|;  s = a / 448 (IEEE fp32 division);
 *     code_d = the E4M3 code nearest to x_d / s (ties to the even code;
 *              |x_d / s| above 448, possible only through the rounding of
 *              s, gives +-448; the sign of a zero is kept);
 *     s == 0 (a == 0, or a / 448 underflows) gives all codes 0.
 *   Codes and scales go to the slots as in pkv_kv_cache_write_int8.  Inputs
 *   must be finite.  Bit-exact: identical codes and scales for identical
 *   inputs.  Errors as for pkv_kv_cache_write_int8.
 */
pkv_status pkv_kv_cache_write_fp8(const float* k, const float* v, uint8_t* k_cache,
                                  uint8_t* v_cache, float* k_scale, float* v_scale,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int64_t num_blocks, void* stream);

/*
 * Quantising cache write for an FP8 KV cache in the E5M2 format (the other
 * common FP8 encoding; [ENG5] "KV-cache quantization").
 *   As pkv_kv_cache_write_fp8 with s = a / 57344 (IEEE fp32 division) and
 *   code_d = the finite E5M2 code nearest to x_d / s (ties to the even
 *   code; +-57344 at most, never an infinity; the sign of a zero is kept).
 *   Bit-exact.  Errors as for pkv_kv_cache_write_int8.
 */
pkv_status pkv_kv_cache_write_fp8_e5m2(const float* k, const float* v, uint8_t* k_cache,
                                       uint8_t* v_cache, float* k_scale, float* v_scale,
                                       const int64_t* slot_mapping, int64_t num_tokens,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int64_t num_blocks, void* stream);

/*
 * Quantising cache write for an INT4 KV cache ([ENG5] "KV-cache
 * quantization": INT4 KV caches calibrated per token, with per-token-per-
 * head scales; [LAYERS] 2.3: K and V quantized separately).
 *   Each (token, kv-head) row x of k (and, separately, of v), fp32, becomes
 *     a = max_d |x_d|;  s = a / 7 (IEEE fp32 division);
 *     code_d = clamp(rint(x_d / s), -7, 7)  (round half to even);
 *     s == 0 (a == 0, or a / 7 underflows) gives all codes 0.
 *   Codes are packed two per byte into the INT4 tiles (layout above): the
 *   token's K row is k_cache[s_slot / bs][h][r][0 .. D/2-1], its V codes
 *   v_cache[s_slot / bs][h][r / 4][0 .. D/2-1][r % 4] (r = s_slot % bs);
 *   scales as for
 *   pkv_kv_cache_write_int8.  No byte is shared by two tokens, so any set of
 *   distinct slots may be written in one call.  Inputs must be finite.
 *   Bit-exact.  Errors as for pkv_kv_cache_write_int8.
 */
pkv_status pkv_kv_cache_write_int4(const float* k, const float* v, uint8_t* k_cache,
                                   uint8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these
 * sizes (0 when every sequence fits one partition, in which case the
 * workspace pointer may be NULL).  partition_tokens as for decode.  The
 * cache kind is not an argument, so the size covers both ways decode may
 * split contexts (fixed partitions for fp32 caches, balanced shares for the
 * others).  Returns 0 also for invalid sizes (decode then reports the
 * error).
 */
size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq,
                                          int32_t partition_tokens);

/*
 * Token count per context partition the library would use for these sizes
 * when partition_tokens is 0 (the automatic choice); 0 for invalid sizes.
 * With balanced shares (below) this is the fixed-partition length that
 * decides between the two: contexts up to it are attended whole.
 */
int32_t pkv_paged_attention_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t block_size, int32_t max_blocks_per_seq,
                                             int32_t partition_tokens);

/*
 * Number of balanced shares decode (and the fused step) use for these sizes
 * and cache kind, or 0 when they use fixed partitions (see
 * pkv_paged_attention_decode: partition_tokens); 0 also for invalid sizes.
 */
int32_t pkv_paged_attention_shares(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t partition_tokens,
                                   pkv_dtype kv_dtype);

/*
 * 1 if one-query decode (pkv_paged_attention_decode, the fused step and the
 * no-allocation variant) reads a cache pool of these sizes with the
 * non-temporal load hint, else 0; 0 also for invalid sizes.  The pool is
 * num_blocks blocks of num_kv_heads x block_size tokens, each token holding
 * K and V of head_dim elements of kv_dtype (half a byte for I4) plus, for
 * the coded caches, two fp32 scales.  The hint is taken when the pool is
 * larger than 512 MiB, twice the GPU's memory-side cache: a step then reads
 * more than that cache can keep until the next step, and loads that skip
 * it sustain a higher rate.  A smaller pool keeps the default policy, so
 * that blocks read again (the next step, or by the sequences that share
 * them) can be served from that cache.  The cascade and multi-query calls
 * always use the default policy.  The results are the same either way.
 */
int32_t pkv_paged_attention_streams_cache(int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                                          int32_t head_dim, pkv_dtype kv_dtype);

/*
 * Single-token decode attention over the paged cache ([ENG5] "Two phases
 * with very different characteristics": each decode step attends the new
 * token over the whole cached context; [ENG5] "Paged attention").
 *   For each sequence b with L = context_lens[b] and query head h (kv-head
 *   g = h / G), with K_b, V_b the L tokens gathered through the block table:
 *     out[b][h][:] = softmax(scale * K_b q[b][h]) V_b,  accumulated in fp32;
 *   L == 0 gives zeros.  For an int8, FP8 (E4M3 or E5M2) or INT4 cache each
 *   K/V element's value is its code times the token's scale.
 * Supported: (q_dtype, kv_dtype) in {(F32, F32), (BF16, BF16), (BF16, I8),
 * (BF16, FP8), (BF16, FP8_E5M2), (BF16, I4)};
 * out has q's dtype; head_dim in {64, 128}; block_size in {16, 32};
 * G in {1, 2, 4, 8, 16}.  k_scale and v_scale are required for the coded
 * caches (I8, FP8, FP8_E5M2, I4) and must be NULL otherwise.  num_seqs == 0 is a no-op.  scale must be finite.
 * partition_tokens: a multiple of 32 in [32, 128 * block_size]: long
 * contexts are split into partitions of that many tokens, one workgroup
 * each, whose partial results a second kernel combines.  0: the automatic
 * choice.  If every context fits the automatic partition length (as
 * max_blocks_per_seq * block_size bounds it), one workgroup per (sequence,
 * kv-head) attends it whole and no second kernel runs.  Otherwise, for
 * bf16, int8 and FP8 caches, the work is balanced: the 32-token chunks of
 * all (sequence, kv-head) pairs, laid end to end, are cut into equal
 * contiguous shares, one per workgroup of a grid sized to the GPU
 * (pkv_paged_attention_shares), so that ragged context lengths leave no
 * tail of idle CUs; pairs split between shares are combined by the second
 * kernel.  fp32 and INT4 caches keep fixed partitions; for INT4 the
 * automatic length may be longer than the query above reports (never
 * giving more partitions, so the workspace size holds), chosen so that
 * the partitions fill whole rounds of the GPU's workgroup slots.  The
 * result is the same softmax in every case, up to rounding.
 * workspace / workspace_bytes: device scratch of at least
 * pkv_paged_attention_workspace_size(...) bytes, 256-byte aligned.
 */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const float* k_scale,
                                      const float* v_scale, const int32_t* block_tables,
                                      const int32_t* context_lens, float scale,
                                      int32_t num_seqs, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, pkv_dtype q_dtype,
                                      pkv_dtype kv_dtype, int32_t partition_tokens,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two launches pkv_paged_attention_decode is made of, for callers that
 * schedule or time them separately.  Same arguments and preconditions.
 * _partitions: attends each context partition; a sequence that fits one
 * partition gets its final output here, longer ones leave per-partition
 * (max, sum, unnormalised output) partials in the workspace.
 * _reduce: combines those partials into out (nothing to do, and no launch,
 * when every sequence fits one partition).  Call _partitions first, on the
 * same stream.
 */
pkv_status pkv_paged_attention_decode_partitions(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream);

pkv_status pkv_paged_attention_decode_reduce(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * Fused decode step: append each sequence's new token, then attend.
 *   For every sequence b with L = context_lens[b] >= 1, the token at
 *   position L - 1 (its block is block_tables[b][(L-1) / bs], row
 *   (L-1) % bs) receives k_new[b][h][:] and v_new[b][h][:] for every
 *   kv-head h, exactly as pkv_kv_cache_write or the quantising write of the
 *   cache's kind (int8, FP8, INT4) with that slot would write it; then out is computed as by
 *   pkv_paged_attention_decode over the updated cache.  One launch does
 *   both (plus the reduce launch when a context spans several partitions):
 *   the workgroups of the partition holding position L - 1 write the token
 *   before attending, and nothing else reads it.
 *   k_new, v_new: [B][Hkv][D], the cache element type (fp32 or bf16), or
 *   fp32 for a coded cache (quantised in the kernel).  The block holding
 *   position L - 1 must belong to this sequence alone (copy it on write
 *   first if it is shared).  Other arguments, errors and the workspace as
 *   for pkv_paged_attention_decode; the caches (and int8 scales) are
 *   written.
 * _partitions: the first launch only (append + attend per partition); the
 *   second is pkv_paged_attention_decode_reduce with the same arguments.
 */
pkv_status pkv_paged_attention_decode_step(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream);

pkv_status pkv_paged_attention_decode_step_partitions(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * Shared-prefix ("cascade") decode: the same attention as
 * pkv_paged_attention_decode, with the blocks a group of sequences shares
 * read once for the whole group ([ENG5] "Paged attention": requests with a
 * common prefix share physical blocks, the basis of prompt caching; [ENG5]
 * "SGLang and RadixAttention": the longest shared prefix is reused and only
 * the rest is computed per request).
 *   Groups are contiguous ranges of sequences: group g is sequences
 *   group_start[g] .. group_start[g+1]-1, with group_start[0] = 0,
 *   non-decreasing, group_start[num_groups] = num_seqs (device int32
 *   [num_groups + 1]).  group_shared_blocks[g] (device int32 [num_groups])
 *   is how many leading block-table entries every member of group g has in
 *   common with the group's first member.  The group's shared span is
 *     S_g = min(group_shared_blocks[g], max_shared_blocks,
 *               context_lens[first member] / block_size) * block_size
 *   tokens; they are attended once per group (queries of all members
 *   together), each member's remaining tokens S_g .. L-1 as in decode, and
 *   the partials are merged per (sequence, head) by the split-context
 *   combine, so out equals pkv_paged_attention_decode's result up to
 *   rounding.  Groups of one sequence or with no shared blocks are plain
 *   decode.
 *   Host-side bounds (the grid is sized from them): num_groups in
 *   [1, num_seqs]; max_group_size >= every group's size, <= num_seqs;
 *   max_shared_blocks in [0, max_blocks_per_seq].
 *   prefix_partition_tokens: tokens of the shared span per workgroup; 0 for
 *   the automatic choice, else a multiple of 32 in [32, 128 * block_size].
 *   partition_tokens as for decode (for the remaining tokens).
 * Supported: (BF16, BF16), (BF16, I8), (BF16, FP8), (BF16, FP8_E5M2) and
 * (BF16, I4) with the sizes of decode; an fp32 cache returns
 * PKV_ERR_UNSUPPORTED.  The workspace size comes from
 * pkv_paged_attention_cascade_workspace_size with the same sizes and is
 * needed whenever num_seqs > 0.  Launches: for bf16 and byte-code caches,
 * one kernel on `stream` holds the shared-prefix workgroups and the
 * workgroups of the sequences' own tokens, then the reduce follows on
 * `stream`.  INT4: the prefix kernel (skipped when max_shared_blocks is 0)
 * on a second stream of the library's (one per device, created on first
 * use, default priority), the partition kernel on `stream` beside it, then
 * the reduce on `stream` after both (the second stream is forked from and
 * joined back into `stream` by events, so the call orders like launches on
 * `stream`, also under graph capture).
 * Not checked unless PKV_DEBUG=1 (device data): the group arrays as stated
 * above; every member's context_lens >= S_g; the shared entries really are
 * equal (if not, the first member's blocks are used for the whole group).
 */
pkv_status pkv_paged_attention_decode_cascade(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_start, const int32_t* group_shared_blocks, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,
    int32_t prefix_partition_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused shared-prefix decode step: append each sequence's new token, then
 * attend as pkv_paged_attention_decode_cascade.
 *   The token at position L - 1 of every sequence with L = context_lens[b]
 *   >= 1 receives k_new[b][h][:] and v_new[b][h][:] exactly as in
 *   pkv_paged_attention_decode_step (same formats: [B][Hkv][D], the cache
 *   element type, fp32 for a coded cache), and out is then computed as by
 *   pkv_paged_attention_decode_cascade over the updated cache: the
 *   workgroups that attend a sequence's own tokens write its token first.
 *   out and the caches equal those of the write followed by the cascade
 *   call, bit for bit.
 *   The new token must lie past its group's shared span (L - 1 >= S_g, in
 *   a block of this sequence alone): shared blocks are never written.  A
 *   block manager that copies a shared tail block on write gives every
 *   sequence such a block; PKV_DEBUG=1 checks it.
 *   Other arguments, errors and the workspace as for
 *   pkv_paged_attention_decode_cascade; the caches (and scales) are written.
 */
pkv_status pkv_paged_attention_decode_cascade_step(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_start, const int32_t* group_shared_blocks, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,
    int32_t prefix_partition_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of pkv_paged_attention_decode_cascade (and of the fused
 * step) for these sizes (0 for invalid sizes, or num_seqs == 0).
 */
size_t pkv_paged_attention_cascade_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, int32_t partition_tokens, int32_t prefix_partition_tokens);

/*
 * Causal multi-query attention over the paged cache: several new tokens per
 * sequence in one call, as a speculative-decoding verification (k + 1
 * proposed positions scored in one pass, [ENG5] "Speculative decoding") or
 * a prefill chunk interleaved with decode ([ENG5] "Orca's iteration-level
 * scheduling", chunked prefill) needs.
 *   Sequence b's new tokens are query rows query_start[b] ..
 *   query_start[b+1]-1 of q and out ([T][H][D], T = num_query_tokens); with
 *   n_b of them and L = context_lens[b], they are the last n_b positions of
 *   its context (their K/V already written), and row query_start[b] + i
 *   attends to tokens 0 .. L - n_b + i:
 *     out[r][h][:] = softmax(scale * K_b[0..pos] q[r][h]) V_b[0..pos].
 *   One query per sequence is exactly pkv_paged_attention_decode.
 * query_start: device int32 [num_seqs + 1], query_start[0] = 0,
 * non-decreasing, query_start[num_seqs] = num_query_tokens.
 * max_queries_per_seq: host bound on every n_b, in [1, num_query_tokens].
 * Supported: (BF16, BF16), (BF16, I8), (BF16, FP8), (BF16, FP8_E5M2) and
 * (BF16, I4) with decode's sizes; an fp32 cache returns
 * PKV_ERR_UNSUPPORTED.  Up to 48 (new token, head) pairs per sequence and
 * kv-head (max_queries_per_seq * G <= 48) the partition kernel computes the
 * partials (its waves split a partition's chunks), beyond that an
 * LDS-staged kernel (its waves split the columns, 64 or 128 per workgroup,
 * and share each chunk).
 * partition_tokens: 0 for the automatic choice, else as for decode.
 * Workspace: pkv_paged_attention_multi_query_workspace_size(...) bytes,
 * 256-byte aligned, whenever num_query_tokens > 0.  Two launches (partials
 * of every context partition, then the combine).
 * Not checked unless PKV_DEBUG=1 (device data): query_start as stated;
 * n_b <= context_lens[b]; n_b <= max_queries_per_seq.
 */
pkv_status pkv_paged_attention_multi_query(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start, float scale, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t num_query_tokens, int32_t max_queries_per_seq, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream);

/* Workspace bytes of pkv_paged_attention_multi_query (0 for invalid sizes
 * or no query tokens). */
size_t pkv_paged_attention_multi_query_workspace_size(
    int32_t num_seqs, int32_t num_query_tokens, int32_t max_queries_per_seq, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t partition_tokens);

/*
 * pkv_paged_attention_decode without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocating routine.
 *   Arguments, result and errors as pkv_paged_attention_decode with
 *   partition_tokens 0 (the automatic choice); the split-context partials
 *   go to a scratch array inside the library instead of a workspace:
 *   PKV_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the
 *   library's loading until the process ends.  Sizes whose partials need
 *   more (pkv_paged_attention_workspace_size bounds them; with balanced
 *   shares they do not grow with context length) return PKV_ERR_WORKSPACE
 *   and launch nothing.
 *   Every call on one GPU uses that GPU's one scratch array, and it keeps
 *   the last call's contents: calls that overlap on one GPU (on different
 *   streams, or from several threads without ordering) race and give wrong
 *   results; calls ordered on one stream are safe.  Nothing in the scratch
 *   needs to start at zero.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                              const void* v_cache, const float* k_scale,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* context_lens, float scale,
                                              int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t block_size, int32_t max_blocks_per_seq,
                                              int64_t num_blocks, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, void* stream);

/* Text of the last failure on this thread ("" after a successful call).
 * The pointer stays valid until the next call on the same thread. */
const char* pkv_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
