// Kernel parameter blocks and launchers of libpagedkv (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// One decode launch.  Partials of sequences longer than one partition go to
// the workspace:
//   ws_acc [B][H][P][D]  unnormalised sum_t p_t v_t of the partition
//   ws_m   [B][H][P]     max over the partition of scale*log2(e)*score
//   ws_l   [B][H][P]     sum_t p_t,  p_t = exp2(scaled score - ws_m)
// where P = num_parts = ceil(max_blocks_per_seq * block_size / part_tokens).
struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;
  float* ws_m;
  float* ws_l;
  // Optional new token per sequence, [B][Hkv][D] (cache element type; fp32
  // for a coded cache): when non-null, the partition holding position L-1
  // writes it there through the block table before attending.
  const void* k_new;
  const void* v_new;
  // Shared-prefix (cascade) decode, or nullptr.  Sequences
  // [group_start[g], group_start[g+1]) form group g and share their first
  // group_shared_blocks[g] blocks; group_shared_tokens() gives the tokens
  // attended once for the whole group.  Their partials fill workspace slots
  // [0, prefix_parts) (partitions of prefix_part_tokens); the partition
  // kernel attends each sequence's remaining tokens into slots
  // prefix_parts + part, and the reduce always runs.
  const int32_t* group_start;
  const int32_t* group_shared_blocks;
  int32_t num_groups;
  int32_t max_shared_blocks;
  int32_t prefix_part_tokens;
  int32_t prefix_parts;
  // Multi-query (causal) attention, or nullptr: sequence b's query rows are
  // query_start[b] .. query_start[b+1]-1 of q and out ([T][H][D]), for the
  // last n_b positions of its context; row query_start[b] + i attends to
  // tokens 0 .. L_b - n_b + i.  Partials of every partition go to the
  // workspace ([T][H][P]) and the reduce always runs.
  const int32_t* query_start;
  int32_t num_query_rows;  // T (multi-query)
  // Multi-query in the partition kernel: column tiles of 16 (new token,
  // head) pairs per (sequence, kv-head); 0 otherwise.
  int32_t mq_tiles;
  float scale_log2;  // scale * log2(e)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t part_tokens;
  int32_t num_parts;
  // Balanced shares (plain decode and the fused step with the automatic
  // choice, when contexts span several partitions), or 0.  The partition
  // kernel's grid is bal_shares workgroups; each takes an equal contiguous
  // share of all (sequence, kv-head) units' 32-token chunks.  Partials of
  // split units go to share slots instead of per-partition slots:
  //   ws_acc [2 * bal_shares][G][D], ws_m / ws_l [2 * bal_shares][G]
  //   ws_unit [B * Hkv][2]: first slot of unit b * Hkv + kvh, and its
  //                          number of splits (1: written whole)
  // where split j >= 1 of a unit whose first slot is f lives in slot
  // 2 * (f / 2 + j).  Share slot r is workspace row bal_row0 + r * G + head
  // (of D floats in ws_acc, of one float in ws_m / ws_l).  Shared-prefix
  // decode: the units cover each sequence's tokens past its group's shared
  // ones, every unit leaves partials (records count 1 too: a whole unit u
  // uses slot 2 * bal_shares + u), and the shared tokens' partials come
  // first, rows [0, bal_row0) = [B][H][num_parts] (num_parts = prefix_parts
  // then).
  int32_t bal_shares;
  int32_t* ws_unit;
  int64_t bal_row0;
  // One-launch shared-prefix decode (set by its launcher): the number of
  // leading workgroups that attend shared tokens, their query tiles per
  // (group, kv-head) and their column tiles per wave.
  int32_t fused_prefix_wgs;
  int32_t fused_prefix_qtiles;
  int32_t fused_prefix_tiles;
  // One-query decode and the fused step: load the K/V tiles with the
  // non-temporal hint (set by the host when the pool is too large to stay
  // in the memory-side cache between steps).
  int32_t stream_loads;
};

struct WriteParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
};

// FP8: E4M3 codes; E5M2: the other FP8 format.  I4: two 4-bit codes per
// byte, two consecutive head dims of one token (K tiles [bs][D/2], V tiles
// [bs/4][D/2][4]).
enum class KvKind { F32 = 0, BF16 = 1, I8 = 2, FP8 = 3, I4 = 4, E5M2 = 5 };

// Whole-block copies between two pools: parts 0..3 are the K tiles, the V
// tiles, the K scale rows and the V scale rows of a block (tile_bytes,
// tile_bytes, scale_bytes, scale_bytes each; scale_bytes 0 without scales).
struct CopyParams {
  const void* src[4];
  void* dst[4];
  const int32_t* pairs;  // [num_pairs][2]: source block, destination block
  int32_t num_pairs;
  int64_t tile_bytes;
  int64_t scale_bytes;
};

// Waves per workgroup of the partition kernels.
constexpr int kDecodeWaves = 4;
// Tokens a wave takes per step (one matrix-core chunk); partition lengths
// are multiples of it.
constexpr int kChunk = 32;
// Block ids one partition may span (its length / block_size): the kernels
// stage them in LDS arrays of this size, and the host rejects longer
// partitions.
constexpr int kMaxPartBlocks = 128;
// Query-column tiles (16 queries each) per wave of the shared-prefix
// kernel: two (128 columns per workgroup), or one when a unit's columns fit
// 64, so that no wave of the workgroup sits idle beside the others.
constexpr int kPrefixTiles = 2;
__host__ __device__ constexpr int prefix_tiles_for(int64_t columns) {
  return columns <= 16 * kDecodeWaves ? 1 : kPrefixTiles;
}
// Queries per workgroup for a unit of `columns` query columns.
__host__ __device__ constexpr int prefix_queries_for(int64_t columns) {
  return 16 * prefix_tiles_for(columns) * kDecodeWaves;
}

// Tokens of group g attended by the shared-prefix kernel: its shared
// blocks, capped at the whole blocks of its first sequence's context (so
// the span is block-aligned and every table entry it reads is in use) and at
// max_shared_blocks (so its partials fit the prefix_parts slots).
__device__ __forceinline__ int group_shared_tokens(const DecodeParams& p, int g) {
  const int lead = p.group_start[g];
  const int full = p.context_lens[lead] / p.block_size;
  const int nb = min(min(max(p.group_shared_blocks[g], 0), full), p.max_shared_blocks);
  return nb * p.block_size;
}

// Index i in [0, n) with start[i] <= x < start[i + 1] of a non-decreasing
// array (x uniform, so the search runs on scalar loads).
__device__ __forceinline__ int range_of(const int32_t* start, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Group of sequence b (groups are contiguous ranges).
__device__ __forceinline__ int group_of(const DecodeParams& p, int b) {
  return range_of(p.group_start, p.num_groups, b);
}

hipError_t launch_decode_mfma(const DecodeParams& p, KvKind kv, hipStream_t s);
// Workgroups of the partition kernel one CU holds at once for cache kind kv
// (its waves per SIMD: 4-wave workgroups on 4 SIMDs).
int balanced_slots_per_cu(KvKind kv);
hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_reduce(const DecodeParams& p, bool out_bf16, hipStream_t s);
hipError_t launch_cascade_prefix(const DecodeParams& p, KvKind kv, int max_group_size, hipStream_t s);
// Shared-prefix decode in one launch (balanced shares for the sequences'
// own tokens, bal_shares set): the shared-prefix workgroups, then the shares.
hipError_t launch_cascade_fused(DecodeParams p, KvKind kv, int max_group_size, hipStream_t s);
// Multi-query attention partials (query_start set): every partition of every
// sequence's context for up to max_queries new tokens per sequence.
hipError_t launch_multi_query(const DecodeParams& p, KvKind kv, int max_queries, hipStream_t s);
// The same partials from the partition kernel (few new tokens per sequence:
// p.mq_tiles column tiles of 16 per (sequence, kv-head); waves split the
// chunks of a partition instead of its columns, each wave carrying every
// tile of its workgroup: all of them, or one for INT4).
hipError_t launch_multi_query_decode(const DecodeParams& p, KvKind kv, hipStream_t s);
// Column tiles up to which the partition kernel runs multi-query attention
// (70B GQA shape, 50 sequences, bf16, measured per call against the
// LDS-staged kernel: 1 tile 373 us vs 508, 2 tiles 415 vs 668, 3 tiles 446
// vs 673; four tiles' states do not fit two waves' registers per SIMD).
constexpr int kMqDecodeMaxTiles = 3;
hipError_t launch_cache_write(const WriteParams& p, KvKind kind, hipStream_t s);
// Quantising write of fp32 rows into an int8, FP8 or INT4 cache.
hipError_t launch_cache_write_codes(const WriteParams& p, KvKind kind, hipStream_t s);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t s);
hipError_t launch_tile_read(const void* pool, const int32_t* ids, int64_t ntiles, int grid, bool streaming,
                            uint32_t* sink, hipStream_t s);

}  // namespace pkv
