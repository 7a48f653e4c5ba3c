// C ABI of libpagedkv: argument validation, variant dispatch, partition
// sizing and error reporting.  Every check here runs before any HIP call, so
// an invalid call launches nothing and has no side effect.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pagedkv.h"
#include "../../include/pagedkv_blocks.h"
#include "../../include/pagedkv_probe.h"
#include "pkv_debug.hpp"
#include "pkv_host.hpp"
#include "pkv_kernels.hpp"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace pkv {

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::ok;

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }
bool block_size_ok(int32_t bs) { return bs == 16 || bs == 32; }
bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// A second stream per device for the shared-prefix kernel of cascade
// decode: that kernel is bound by its contractions and softmax, the
// partition kernel over each sequence's own tokens by HBM, and they write
// disjoint workspace slots, so they run side by side; the caller's stream
// waits for it (an event) before the reduce.  Created on first use with the
// default priority and kept until the process ends.  The fork / join
// sequence is enqueued under g_side_mutex so that concurrent callers never
// re-record each other's events in between.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mutex;
SideStream g_side[kMaxDevices];

// The current device's side stream (caller holds g_side_mutex).
hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr) {
    SideStream n;
    e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
      return e;
    }
    ss = n;
  }
  *out = &ss;
  return hipSuccess;
}

// Scratch of pkv_paged_attention_decode_noalloc: the split-context
// partials of a decode call, in device memory the library never allocates.
// One copy per GPU, loaded with the library's code and held until the
// process ends.  Host code reaches it only through the device address
// hipGetSymbolAddress returns for the current device (the array's name on
// the host is a stand-in, not a device address); the address is looked up
// once per device, on that device's first call, and kept.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];

// The current device's scratch address.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

using pkv::kChunk;          // tokens per wave iteration
using pkv::kMaxPartBlocks;  // block ids of one partition staged in LDS

// Automatic partition length: the longest of 2048 / 1024 / 512 / 256 tokens
// (at most kMaxPartBlocks blocks) that still gives the launch about two full
// rounds of workgroups on the GPU (two 256-thread workgroups per CU, 256
// CUs).  Longer partitions amortise each workgroup's fixed cost (query load,
// block-id staging, the final merge) and leave fewer partials to reduce.
int32_t auto_part_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_blocks_per_seq) {
  const int64_t ctx = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  constexpr int64_t kTargetWorkgroups = 1024;
  int32_t pt = 256;
  for (int32_t cand : {2048, 1024, 512}) {
    if (cand > kMaxPartBlocks * block_size) continue;
    if (units * ((ctx + cand - 1) / cand) >= kTargetWorkgroups) {
      pt = cand;
      break;
    }
  }
  return pt;
}

// Among partition lengths no shorter than pt (never more partitions, hence
// never a larger workspace), the one whose workgroups fill `slots`
// workgroup slots in whole rounds best: the fewest rounds x tokens per
// workgroup, for contexts of ctx tokens.  (64 x 8192-token contexts, 8
// kv-heads, 768 slots: 3 partitions of 2752 tokens, two full rounds,
// instead of 4 of 2048 in 2.67 rounds.)
int32_t refine_part_tokens(int32_t pt, int64_t units, int64_t ctx, int64_t slots) {
  auto cost = [&](int64_t t) {
    const int64_t w = units * ((ctx + t - 1) / t);
    return ((w + slots - 1) / slots) * t;
  };
  int64_t best = pt, best_cost = cost(pt);
  for (int64_t parts = (ctx + pt - 1) / pt - 1; parts >= 1; --parts) {
    const int64_t t = ((ctx + parts - 1) / parts + kChunk - 1) / kChunk * kChunk;
    const int64_t c = cost(t);
    if (c < best_cost) {
      best = t;
      best_cost = c;
    }
  }
  return static_cast<int32_t>(best);
}

// Validated partition length, or 0 if `requested` is not acceptable.
int32_t part_tokens_for(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                        int32_t max_blocks_per_seq, int32_t requested) {
  if (requested == 0) return auto_part_tokens(num_seqs, num_kv_heads, block_size, max_blocks_per_seq);
  if (requested < kChunk || requested % kChunk != 0 || requested > kMaxPartBlocks * block_size)
    return 0;
  return requested;
}

int32_t num_parts_for(int32_t block_size, int32_t max_blocks_per_seq, int32_t pt) {
  const int64_t ctx = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  return static_cast<int32_t>((ctx + pt - 1) / pt);
}

// Balanced shares (DecodeParams::bal_shares).  The partition kernel's grid
// is one workgroup per share, sized to the workgroups all CUs hold at once
// (MI355X: 256 CUs) times kShareRounds.
constexpr int32_t kNumCUs = 256;
constexpr int32_t kShareRounds = 1;

int32_t shares_for(pkv::KvKind kv) { return kShareRounds * kNumCUs * pkv::balanced_slots_per_cu(kv); }
int32_t max_shares() {
  int32_t s = 0;
  for (pkv::KvKind kv : {pkv::KvKind::BF16, pkv::KvKind::I8, pkv::KvKind::FP8, pkv::KvKind::E5M2})
    s = std::max(s, shares_for(kv));
  return s;
}

// Does a call with these sizes run in balanced shares?  The automatic
// choice, a bf16 or byte-code cache, and contexts that may span more than
// one partition (otherwise one workgroup per (sequence, kv-head) attends
// it whole and no reduce runs); chunk counts must stay far inside 64-bit
// arithmetic.  fp32 caches have their own kernel.  INT4 keeps fixed
// partitions: its kernel runs three workgroups per CU only within 168
// VGPRs, which the share walk exceeds (spills); at two per CU, or with the
// spills, its step measured 134-166 us against 131-133 us on fixed
// partitions (70B-shaped INT4 workload, one box).
bool balanced_for(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size, int32_t max_blocks_per_seq,
                  int32_t partition_tokens, pkv::KvKind kv) {
  if (partition_tokens != 0 || num_seqs <= 0) return false;
  if (kv != pkv::KvKind::BF16 && kv != pkv::KvKind::I8 && kv != pkv::KvKind::FP8 && kv != pkv::KvKind::E5M2)
    return false;
  const int32_t pt = auto_part_tokens(num_seqs, num_kv_heads, block_size, max_blocks_per_seq);
  const int64_t ctx = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  if (ctx <= pt) return false;
  const int64_t chunks = static_cast<int64_t>(num_seqs) * num_kv_heads * ((ctx + kChunk - 1) / kChunk);
  return chunks < (int64_t(1) << 40);
}

// Workspace of balanced shares: ws_acc [2S][G][D], ws_m and ws_l [2S][G],
// ws_unit [B * Hkv][2] int32, each 256-byte aligned.
struct BalancedLayout {
  size_t acc, ml, unit;
  size_t total() const { return acc + 2 * ml + unit; }
};
BalancedLayout balanced_layout(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t shares) {
  const size_t rows = static_cast<size_t>(2) * shares * (num_heads / num_kv_heads);
  BalancedLayout l;
  l.acc = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  l.ml = (rows * sizeof(float) + 255) & ~size_t(255);
  l.unit = (static_cast<size_t>(num_seqs) * num_kv_heads * 2 * sizeof(int32_t) + 255) & ~size_t(255);
  return l;
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t nparts) {
  if (nparts <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * nparts;
  size_t acc = rows * head_dim * sizeof(float);
  acc = (acc + 255) & ~size_t(255);
  size_t ml = rows * sizeof(float);
  ml = (ml + 255) & ~size_t(255);
  return acc + 2 * ml;
}

// The K/V loads of one-query decode take the non-temporal hint when the
// cache pool holds more than twice the GPU's memory-side cache (256 MiB on
// MI355X): then the KV a step reads cannot stay cached until the next step,
// and streaming it past that cache reads faster (7B MHA step 184.1 -> 168.7
// us, 70B GQA bf16 361 -> 323 us, int8 202 -> 184 us, one box).  A smaller
// pool may be served from that cache step after step, and so may blocks
// that many sequences share (the 256-sequence shared-prefix workload, 338
// MiB of pool: plain step 196 -> 342 us with the hint), so those keep the
// default policy; shared prefixes have the cascade call, which always does.
constexpr int64_t kMemorySideCacheBytes = int64_t(256) << 20;
bool stream_loads_for(pkv::KvKind kv, int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                      int32_t head_dim) {
  // K + V bytes per dim, and per token and kv-head (with the two scales)
  const int64_t kv_bytes = kv == pkv::KvKind::F32 ? 8 : kv == pkv::KvKind::BF16 ? 4 : kv == pkv::KvKind::I4 ? 1 : 2;
  const int64_t scales = kv == pkv::KvKind::F32 || kv == pkv::KvKind::BF16 ? 0 : 8;
  const int64_t per_token = kv_bytes * head_dim + scales;
  return num_blocks * num_kv_heads * block_size * per_token > 2 * kMemorySideCacheBytes;
}

struct DecodeSetup {
  pkv::DecodeParams p;
  pkv::KvKind kv;
  bool out_bf16;
  size_t need;  // workspace bytes this call uses (plain decode / step layout)
};

pkv_status validate_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int64_t num_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           const void* k_new, const void* v_new, bool step, DecodeSetup* st,
                           bool check_workspace = true, bool allow_balanced = false) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID, "num_heads and num_kv_heads must be positive");
  if (num_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_heads (%d) must be a multiple of num_kv_heads (%d)",
                num_heads, num_kv_heads);
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID, "max_blocks_per_seq must be positive");
  if (num_blocks <= 0) return fail(PKV_ERR_INVALID, "num_blocks must be positive");
  if (head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID, "head_dim and block_size must be positive");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID, "scale must be finite");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > (int64_t(1) << 30))
    return fail(PKV_ERR_INVALID, "max_blocks_per_seq * block_size too large");
  if (!head_dim_ok(head_dim)) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (!block_size_ok(block_size))
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
  if (!group_ok(num_heads / num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "num_heads / num_kv_heads = %d not in {1, 2, 4, 8, 16}",
                num_heads / num_kv_heads);
  pkv::KvKind kv;
  if (q_dtype == PKV_F32 && kv_dtype == PKV_F32) {
    kv = pkv::KvKind::F32;
  } else if (q_dtype == PKV_BF16 && kv_dtype == PKV_BF16) {
    kv = pkv::KvKind::BF16;
  } else if (q_dtype == PKV_BF16 && kv_dtype == PKV_I8) {
    kv = pkv::KvKind::I8;
  } else if (q_dtype == PKV_BF16 && kv_dtype == PKV_FP8) {
    kv = pkv::KvKind::FP8;
  } else if (q_dtype == PKV_BF16 && kv_dtype == PKV_I4) {
    kv = pkv::KvKind::I4;
  } else if (q_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E5M2) {
    kv = pkv::KvKind::E5M2;
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "(q_dtype, kv_dtype) = (%d, %d) is not supported",
                static_cast<int>(q_dtype), static_cast<int>(kv_dtype));
  }
  const int32_t pt0 = part_tokens_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq,
                                      partition_tokens);
  if (pt0 == 0)
    return fail(PKV_ERR_INVALID,
                "partition_tokens %d must be 0 or a multiple of %d in [%d, %d]",
                partition_tokens, kChunk, kChunk, kMaxPartBlocks * block_size);
  const bool bal = allow_balanced && balanced_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq,
                                                  partition_tokens, kv);
  // INT4 keeps fixed partitions: their automatic length is refined to fill
  // whole rounds of the GPU's workgroup slots
  const int32_t pt = allow_balanced && partition_tokens == 0 && kv == pkv::KvKind::I4
                         ? refine_part_tokens(pt0, static_cast<int64_t>(num_seqs) * num_kv_heads,
                                              static_cast<int64_t>(max_blocks_per_seq) * block_size,
                                              static_cast<int64_t>(kNumCUs) * pkv::balanced_slots_per_cu(kv))
                         : pt0;
  const int32_t nparts = num_parts_for(block_size, max_blocks_per_seq, pt);
  if (nparts > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many context partitions (%d)", nparts);
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > 0x7fffffff)
    return fail(PKV_ERR_UNSUPPORTED, "num_seqs * num_kv_heads too large");
  if (num_seqs > 0) {
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
      return fail(PKV_ERR_INVALID, "null pointer among out, q, k_cache, v_cache, block_tables, context_lens");
  }
  if (step && num_seqs > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID, "decode step needs k_new and v_new");
  if (kv != pkv::KvKind::F32 && kv != pkv::KvKind::BF16) {
    if (num_seqs > 0 && (!k_scale || !v_scale))
      return fail(PKV_ERR_INVALID, "int8 / FP8 / INT4 cache needs k_scale and v_scale");
  } else if (k_scale || v_scale) {
    return fail(PKV_ERR_INVALID, "k_scale / v_scale must be NULL for fp32 and bf16 caches");
  }
  const int32_t shares = bal ? shares_for(kv) : 0;
  const BalancedLayout bl = balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim, shares);
  const size_t need = !check_workspace ? 0
                      : bal          ? bl.total()
                                     : workspace_bytes_for(num_seqs, num_heads, head_dim, nparts);
  st->need = bal ? bl.total() : workspace_bytes_for(num_seqs, num_heads, head_dim, nparts);
  if (need > 0 && num_seqs > 0) {
    if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  pkv::DecodeParams& p = st->p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * nparts;
  size_t acc_bytes = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  size_t ml_bytes = (rows * sizeof(float) + 255) & ~size_t(255);
  char* ws = static_cast<char*>(workspace);
  p.ws_acc = need ? reinterpret_cast<float*>(ws) : nullptr;
  p.ws_m = need ? reinterpret_cast<float*>(ws + acc_bytes) : nullptr;
  p.ws_l = need ? reinterpret_cast<float*>(ws + acc_bytes + ml_bytes) : nullptr;
  p.bal_shares = shares;
  p.ws_unit = nullptr;
  p.bal_row0 = 0;
  p.fused_prefix_wgs = p.fused_prefix_qtiles = p.fused_prefix_tiles = 0;
  p.stream_loads = stream_loads_for(kv, num_blocks, num_kv_heads, block_size, head_dim) ? 1 : 0;
  if (bal && need) {
    p.ws_acc = reinterpret_cast<float*>(ws);
    p.ws_m = reinterpret_cast<float*>(ws + bl.acc);
    p.ws_l = reinterpret_cast<float*>(ws + bl.acc + bl.ml);
    p.ws_unit = reinterpret_cast<int32_t*>(ws + bl.acc + 2 * bl.ml);
  }
  p.k_new = step ? k_new : nullptr;
  p.v_new = step ? v_new : nullptr;
  p.group_start = nullptr;  // plain decode; the cascade entry point sets these
  p.group_shared_blocks = nullptr;
  p.num_groups = 0;
  p.max_shared_blocks = 0;
  p.prefix_part_tokens = 0;
  p.prefix_parts = 0;
  p.query_start = nullptr;  // plain decode; the multi-query entry point sets it
  p.num_query_rows = 0;
  p.mq_tiles = 0;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.part_tokens = pt;
  p.num_parts = nparts;
  st->kv = kv;
  st->out_bf16 = q_dtype == PKV_BF16;
  return PKV_OK;
}

pkv_status launch_partitions(const DecodeSetup& st, hipStream_t stream) {
  hipError_t e = st.kv == pkv::KvKind::F32 ? pkv::launch_decode_f32(st.p, stream)
                                           : pkv::launch_decode_mfma(st.p, st.kv, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "partition kernel launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

pkv_status launch_reduce(const DecodeSetup& st, hipStream_t stream) {
  if (st.p.num_parts <= 1 && st.p.bal_shares == 0) return PKV_OK;
  hipError_t e = pkv::launch_decode_reduce(st.p, st.out_bf16, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "reduce kernel launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Shared-prefix partition length: the longest of 2048 ... 32 tokens that
// still gives at least 128 shared-prefix workgroups, half a workgroup per
// CU (at most kMaxPartBlocks blocks; a multiple of 32, hence of the block
// size).  The rest of the GPU's workgroup slots go to the sequences' own
// tokens, attended beside them; longer partitions also leave fewer
// partials to merge.  Shared-prefix workload (256 x 2000 shared + 50..500
// own tokens, one launch): 88-93 us per step at 128 workgroups (1024
// tokens), 94-98 us at 256, 109-113 us at 512, 115-122 us at 64.
int32_t auto_prefix_part_tokens(int64_t prefix_units, int32_t block_size, int32_t max_shared_blocks) {
  const int64_t span = static_cast<int64_t>(max_shared_blocks) * block_size;
  int32_t pt = 32;
  for (int32_t cand : {2048, 1024, 512, 256, 128, 64}) {
    if (cand > kMaxPartBlocks * block_size) continue;
    if (prefix_units * ((span + cand - 1) / cand) >= 128) {
      pt = cand;
      break;
    }
  }
  return pt;
}

using pkv::prefix_queries_for;  // queries per prefix workgroup

struct CascadeSizes {
  int32_t ppt, pparts, spt, sparts, qtiles;
};

// Validated cascade sizes (returns PKV_OK and fills cs) for the calls below.
pkv_status cascade_sizes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_groups,
                         int32_t max_group_size, int32_t max_shared_blocks,
                         int32_t partition_tokens, int32_t prefix_partition_tokens,
                         CascadeSizes* cs) {
  if (num_groups < 0 || (num_seqs > 0 && num_groups < 1))
    return fail(PKV_ERR_INVALID, "num_groups must be >= 1 when num_seqs > 0 (got %d)", num_groups);
  if (num_groups > num_seqs)
    return fail(PKV_ERR_INVALID, "num_groups (%d) exceeds num_seqs (%d)", num_groups, num_seqs);
  if (max_group_size < 0 || max_group_size > num_seqs || (num_seqs > 0 && max_group_size < 1))
    return fail(PKV_ERR_INVALID, "max_group_size must be in [1, num_seqs] (got %d)", max_group_size);
  if (max_shared_blocks < 0 || max_shared_blocks > max_blocks_per_seq)
    return fail(PKV_ERR_INVALID, "max_shared_blocks must be in [0, max_blocks_per_seq] (got %d)",
                max_shared_blocks);
  const int32_t G = num_heads / num_kv_heads;
  const int64_t cols = static_cast<int64_t>(max_group_size) * G;
  const int64_t qtiles = (cols + prefix_queries_for(cols) - 1) / prefix_queries_for(cols);
  if (qtiles > 65535) return fail(PKV_ERR_UNSUPPORTED, "max_group_size * G too large");
  if (static_cast<int64_t>(num_groups) * num_kv_heads > 0x7fffffff)
    return fail(PKV_ERR_UNSUPPORTED, "num_groups * num_kv_heads too large");
  int32_t ppt = prefix_partition_tokens;
  if (ppt == 0) {
    ppt = auto_prefix_part_tokens(static_cast<int64_t>(num_groups) * num_kv_heads * qtiles,
                                  block_size, max_shared_blocks);
  } else if (ppt < kChunk || ppt % kChunk != 0 || ppt > kMaxPartBlocks * block_size) {
    return fail(PKV_ERR_INVALID, "prefix_partition_tokens %d must be 0 or a multiple of %d in [%d, %d]",
                ppt, kChunk, kChunk, kMaxPartBlocks * block_size);
  }
  const int32_t spt = part_tokens_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq,
                                      partition_tokens);
  if (spt == 0)
    return fail(PKV_ERR_INVALID, "partition_tokens %d must be 0 or a multiple of %d in [%d, %d]",
                partition_tokens, kChunk, kChunk, kMaxPartBlocks * block_size);
  const int64_t span = static_cast<int64_t>(max_shared_blocks) * block_size;
  cs->ppt = ppt;
  cs->pparts = static_cast<int32_t>((span + ppt - 1) / ppt);
  cs->spt = spt;
  cs->sparts = num_parts_for(block_size, max_blocks_per_seq, spt);
  cs->qtiles = static_cast<int32_t>(qtiles);
  if (static_cast<int64_t>(cs->pparts) + cs->sparts > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "too many partitions (%d + %d)", cs->pparts, cs->sparts);
  return PKV_OK;
}

// Multi-query partition length: as auto_part_tokens, counting the query
// tiles of the prefix-style kernel among the units of work.
int32_t auto_mq_part_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t qtiles, int32_t block_size,
                            int32_t max_blocks_per_seq) {
  const int64_t ctx = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads * qtiles;
  int32_t pt = 256;
  for (int32_t cand : {2048, 1024, 512}) {
    if (cand > kMaxPartBlocks * block_size) continue;
    if (units * ((ctx + cand - 1) / cand) >= 1024) {
      pt = cand;
      break;
    }
  }
  return pt;
}

// Multi-query sizing.  Up to kMqDecodeMaxTiles column tiles of 16 (new
// token, head) pairs per (sequence, kv-head), the partition kernel runs it
// (its waves split a partition's chunks, each carrying all the columns of
// its workgroup);
// beyond, the LDS-staged kernel (its waves split 128 columns and share each
// chunk).  qtiles counts the chosen kernel's column tiles.
struct MqSizes {
  int32_t pt, parts, qtiles;
  bool decode_style;
};

pkv_status mq_sizes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t num_query_tokens, int32_t max_queries,
                    int32_t partition_tokens, MqSizes* ms) {
  if (num_query_tokens < 0) return fail(PKV_ERR_INVALID, "num_query_tokens must be >= 0");
  if (num_query_tokens > 0 && (max_queries < 1 || max_queries > num_query_tokens))
    return fail(PKV_ERR_INVALID, "max_queries_per_seq must be in [1, num_query_tokens] (got %d)", max_queries);
  if (static_cast<int64_t>(num_query_tokens) * num_heads > 0x7fffffff)
    return fail(PKV_ERR_UNSUPPORTED, "num_query_tokens * num_heads too large");
  const int32_t G = num_heads / num_kv_heads;
  const int64_t cols = static_cast<int64_t>(max_queries > 0 ? max_queries : 1) * G;
  const bool decode_style = cols <= 16 * pkv::kMqDecodeMaxTiles;
  const int64_t qtiles = decode_style ? (cols + 15) / 16 : (cols + prefix_queries_for(cols) - 1) / prefix_queries_for(cols);
  if (qtiles > 65535) return fail(PKV_ERR_UNSUPPORTED, "max_queries_per_seq * G too large");
  int32_t pt = partition_tokens;
  if (pt == 0) {
    pt = auto_mq_part_tokens(num_seqs, num_kv_heads, static_cast<int32_t>(qtiles), block_size,
                             max_blocks_per_seq);
  } else if (pt < kChunk || pt % kChunk != 0 || pt > kMaxPartBlocks * block_size) {
    return fail(PKV_ERR_INVALID, "partition_tokens %d must be 0 or a multiple of %d in [%d, %d]", pt,
                kChunk, kChunk, kMaxPartBlocks * block_size);
  }
  ms->pt = pt;
  ms->parts = num_parts_for(block_size, max_blocks_per_seq, pt);
  ms->qtiles = static_cast<int32_t>(qtiles);
  ms->decode_style = decode_style;
  if (ms->parts > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many context partitions (%d)", ms->parts);
  return PKV_OK;
}

size_t mq_workspace_bytes(int32_t num_query_tokens, int32_t num_heads, int32_t head_dim, int32_t parts) {
  const size_t rows = static_cast<size_t>(num_query_tokens) * num_heads * parts;
  if (rows == 0) return 0;
  const size_t acc = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  const size_t ml = (rows * sizeof(float) + 255) & ~size_t(255);
  return acc + 2 * ml;
}

// Workspace of the cascade on fixed partitions: every (sequence, head) has
// pparts + sparts partial slots, and the reduce always runs.
size_t cascade_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                               const CascadeSizes& cs) {
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * (cs.pparts + cs.sparts);
  if (rows == 0) return 0;
  const size_t acc = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  const size_t ml = (rows * sizeof(float) + 255) & ~size_t(255);
  return acc + 2 * ml;
}

// Shares of the sequences' own tokens in the one-launch cascade, in rounds
// of the GPU's workgroup slots: the shared-prefix workgroups hold slots for
// part of the launch, and smaller shares fill around them.
constexpr int32_t kCascadeShareRounds = 2;
int32_t cascade_shares_for(pkv::KvKind kv) { return kCascadeShareRounds * shares_for(kv); }

// The sequences' own tokens in balanced shares (automatic partitioning,
// the kinds the balanced walk serves): the shared tokens' pparts slots per
// (sequence, head) come first, then the shares' 2 S slots and one slot per
// (sequence, kv-head) unit, per head of a group, then the unit records.
bool cascade_balanced_for(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                          int32_t block_size, int32_t partition_tokens, pkv::KvKind kv) {
  if (partition_tokens != 0 || num_seqs <= 0) return false;
  if (kv != pkv::KvKind::BF16 && kv != pkv::KvKind::I8 && kv != pkv::KvKind::FP8 && kv != pkv::KvKind::E5M2)
    return false;
  const int64_t ctx = static_cast<int64_t>(max_blocks_per_seq) * block_size;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  return units * ((ctx + kChunk - 1) / kChunk) < (int64_t(1) << 40) &&
         units + 2 * int64_t(kCascadeShareRounds) * max_shares() < 0x7fffffff;
}

// The automatic choice for the sequences' own tokens: balanced shares when
// they may span several partitions (as for decode); short ones (a long
// shared prefix, a short tail each) take a workgroup per (sequence,
// kv-head), which measured faster there: 94-100 us against 112-118 us per
// step on the 256 x (2000 shared + 50..500) token workload.
bool cascade_own_balanced(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks_per_seq, int32_t block_size,
                          int32_t partition_tokens, int32_t max_shared_blocks, int32_t own_part_tokens,
                          pkv::KvKind kv) {
  return cascade_balanced_for(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_tokens, kv) &&
         (static_cast<int64_t>(max_blocks_per_seq) - max_shared_blocks) * block_size > own_part_tokens;
}

struct CascadeBalancedLayout {
  size_t rows_pre, acc, ml, unit;
  size_t total() const { return acc + 2 * ml + unit; }
};
CascadeBalancedLayout cascade_balanced_layout(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t pparts, int32_t shares) {
  CascadeBalancedLayout l;
  l.rows_pre = static_cast<size_t>(num_seqs) * num_heads * pparts;
  const size_t rows = l.rows_pre + (static_cast<size_t>(2) * shares + static_cast<size_t>(num_seqs) * num_kv_heads) *
                                       (num_heads / num_kv_heads);
  l.acc = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  l.ml = (rows * sizeof(float) + 255) & ~size_t(255);
  l.unit = (static_cast<size_t>(num_seqs) * num_kv_heads * 2 * sizeof(int32_t) + 255) & ~size_t(255);
  return l;
}

pkv_status validate_write(const void* k, const void* v, const void* k_cache, const void* v_cache,
                          const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int64_t num_blocks) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "num_kv_heads, head_dim, block_size and num_blocks must be positive");
  if (!head_dim_ok(head_dim)) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (!block_size_ok(block_size))
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
  if (num_tokens > 0 && (!k || !v || !k_cache || !v_cache || !slot_mapping))
    return fail(PKV_ERR_INVALID, "null pointer among k, v, k_cache, v_cache, slot_mapping");
  if (num_tokens > (int64_t(1) << 40) / (num_kv_heads * int64_t(head_dim)))
    return fail(PKV_ERR_INVALID, "num_tokens too large");
  return PKV_OK;
}

// PKV_DEBUG=1: the device-data preconditions of a write / of decode-style
// calls, checked on host copies before anything is launched.
pkv_status debug_write(const int64_t* slot_mapping, int64_t num_tokens, int32_t block_size,
                       int64_t num_blocks, void* stream) {
  if (!pkv::debug_checks_enabled() || num_tokens == 0) return PKV_OK;
  return pkv::debug_check_slots(slot_mapping, num_tokens, block_size, num_blocks,
                                static_cast<hipStream_t>(stream));
}

pkv_status debug_tables(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                        int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks, void* stream,
                        std::vector<int32_t>* tables = nullptr, std::vector<int32_t>* lens = nullptr) {
  if (!pkv::debug_checks_enabled() || num_seqs == 0) return PKV_OK;
  std::vector<int32_t> t, l;
  return pkv::debug_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size,
                                 num_blocks, static_cast<hipStream_t>(stream), tables ? tables : &t,
                                 lens ? lens : &l);
}

pkv_status write_codes(const float* k, const float* v, void* k_cache, void* v_cache,
                       float* k_scale, float* v_scale, const int64_t* slot_mapping,
                       int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, pkv::KvKind kind, void* stream,
                       const char* what) {
  pkv_status st = validate_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                 head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_tokens > 0 && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID, "null k_scale or v_scale");
  if (num_tokens == 0) return ok();
  st = debug_write(slot_mapping, num_tokens, block_size, num_blocks, stream);
  if (st != PKV_OK) return st;
  pkv::WriteParams p{k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size};
  hipError_t e = pkv::launch_cache_write_codes(p, kind, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, pkv_dtype dtype, void* stream) {
  pkv_status st = validate_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                 head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (dtype != PKV_F32 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write dtype must be PKV_F32 or PKV_BF16");
  if (num_tokens == 0) return ok();
  st = debug_write(slot_mapping, num_tokens, block_size, num_blocks, stream);
  if (st != PKV_OK) return st;
  pkv::WriteParams p{k, v, k_cache, v_cache, nullptr, nullptr, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size};
  hipError_t e = pkv::launch_cache_write(p, dtype == PKV_F32 ? pkv::KvKind::F32 : pkv::KvKind::BF16,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_cache_write launch failed: %s", hipGetErrorString(e));
  return ok();
}

pkv_status pkv_kv_cache_write_int8(const float* k, const float* v, int8_t* k_cache,
                                   int8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, void* stream) {
  return write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size, num_blocks, pkv::KvKind::I8, stream,
                     "kv_cache_write_int8");
}

pkv_status pkv_kv_cache_write_fp8(const float* k, const float* v, uint8_t* k_cache,
                                  uint8_t* v_cache, float* k_scale, float* v_scale,
                                  const int64_t* slot_mapping, int64_t num_tokens,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int64_t num_blocks, void* stream) {
  return write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size, num_blocks, pkv::KvKind::FP8, stream,
                     "kv_cache_write_fp8");
}

pkv_status pkv_kv_cache_write_fp8_e5m2(const float* k, const float* v, uint8_t* k_cache,
                                       uint8_t* v_cache, float* k_scale, float* v_scale,
                                       const int64_t* slot_mapping, int64_t num_tokens,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int64_t num_blocks, void* stream) {
  return write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size, num_blocks, pkv::KvKind::E5M2, stream,
                     "kv_cache_write_fp8_e5m2");
}

pkv_status pkv_kv_cache_write_int4(const float* k, const float* v, uint8_t* k_cache,
                                   uint8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, int64_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, void* stream) {
  return write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, num_tokens,
                     num_kv_heads, head_dim, block_size, num_blocks, pkv::KvKind::I4, stream,
                     "kv_cache_write_int4");
}

int32_t pkv_paged_attention_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t block_size, int32_t max_blocks_per_seq,
                                             int32_t partition_tokens) {
  if (num_seqs < 0 || num_kv_heads <= 0 || !block_size_ok(block_size) || max_blocks_per_seq <= 0)
    return 0;
  return part_tokens_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, partition_tokens);
}

size_t pkv_paged_attention_workspace_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq,
                                          int32_t partition_tokens) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || !head_dim_ok(head_dim) ||
      !block_size_ok(block_size) || max_blocks_per_seq <= 0)
    return 0;
  const int32_t pt = part_tokens_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq,
                                     partition_tokens);
  if (pt == 0) return 0;
  const size_t fixed = workspace_bytes_for(num_seqs, num_heads, head_dim,
                                           num_parts_for(block_size, max_blocks_per_seq, pt));
  // the cache kind is not an argument: enough for fixed partitions (fp32
  // caches) and for balanced shares (the other kinds)
  if (!balanced_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, partition_tokens,
                    pkv::KvKind::BF16))
    return fixed;
  return std::max(fixed, balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim, max_shares()).total());
}

int32_t pkv_paged_attention_shares(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t partition_tokens, pkv_dtype kv_dtype) {
  if (num_seqs < 0 || num_kv_heads <= 0 || !block_size_ok(block_size) || max_blocks_per_seq <= 0)
    return 0;
  pkv::KvKind kv;
  switch (kv_dtype) {
    case PKV_BF16: kv = pkv::KvKind::BF16; break;
    case PKV_I8: kv = pkv::KvKind::I8; break;
    case PKV_FP8: kv = pkv::KvKind::FP8; break;
    case PKV_FP8_E5M2: kv = pkv::KvKind::E5M2; break;
    case PKV_I4: kv = pkv::KvKind::I4; break;
    default: return 0;
  }
  return balanced_for(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, partition_tokens, kv) ? shares_for(kv)
                                                                                                     : 0;
}

int32_t pkv_paged_attention_streams_cache(int64_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                                          int32_t head_dim, pkv_dtype kv_dtype) {
  if (num_blocks < 0 || num_kv_heads <= 0 || !block_size_ok(block_size) || (head_dim != 64 && head_dim != 128))
    return 0;
  pkv::KvKind kv;
  switch (kv_dtype) {
    case PKV_F32: kv = pkv::KvKind::F32; break;
    case PKV_BF16: kv = pkv::KvKind::BF16; break;
    case PKV_I8: kv = pkv::KvKind::I8; break;
    case PKV_FP8: kv = pkv::KvKind::FP8; break;
    case PKV_FP8_E5M2: kv = pkv::KvKind::E5M2; break;
    case PKV_I4: kv = pkv::KvKind::I4; break;
    default: return 0;
  }
  return stream_loads_for(kv, num_blocks, num_kv_heads, block_size, head_dim) ? 1 : 0;
}

#define PKV_DECODE_ARGS                                                                       \
  out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, num_seqs,    \
      num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, q_dtype, \
      kv_dtype, partition_tokens, workspace, workspace_bytes

#define PKV_DECODE_PARAMS                                                                    \
  void *out, const void *q, const void *k_cache, const void *v_cache, const float *k_scale,  \
      const float *v_scale, const int32_t *block_tables, const int32_t *context_lens,        \
      float scale, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,                \
      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,  \
      pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens, void *workspace,      \
      size_t workspace_bytes, void *stream

pkv_status pkv_paged_attention_decode(PKV_DECODE_PARAMS) {
  DecodeSetup st;
  pkv_status s = validate_decode(PKV_DECODE_ARGS, nullptr, nullptr, false, &st, true, true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_partitions(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  s = launch_reduce(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

pkv_status pkv_paged_attention_decode_partitions(PKV_DECODE_PARAMS) {
  DecodeSetup st;
  pkv_status s = validate_decode(PKV_DECODE_ARGS, nullptr, nullptr, false, &st, true, true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_partitions(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

pkv_status pkv_paged_attention_decode_reduce(PKV_DECODE_PARAMS) {
  DecodeSetup st;
  pkv_status s = validate_decode(PKV_DECODE_ARGS, nullptr, nullptr, false, &st, true, true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_reduce(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

#define PKV_STEP_PARAMS                                                                      \
  void *out, const void *q, const void *k_new, const void *v_new, void *k_cache,             \
      void *v_cache, float *k_scale, float *v_scale, const int32_t *block_tables,            \
      const int32_t *context_lens, float scale, int32_t num_seqs, int32_t num_heads,         \
      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, \
      int64_t num_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,   \
      void *workspace, size_t workspace_bytes, void *stream

pkv_status pkv_paged_attention_decode_step(PKV_STEP_PARAMS) {
  DecodeSetup st;
  pkv_status s = validate_decode(PKV_DECODE_ARGS, k_new, v_new, true, &st, true, true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_partitions(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  s = launch_reduce(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

pkv_status pkv_paged_attention_decode_step_partitions(PKV_STEP_PARAMS) {
  DecodeSetup st;
  pkv_status s = validate_decode(PKV_DECODE_ARGS, k_new, v_new, true, &st, true, true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_partitions(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

size_t pkv_paged_attention_cascade_workspace_size(
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, int32_t partition_tokens, int32_t prefix_partition_tokens) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !head_dim_ok(head_dim) || !block_size_ok(block_size) || max_blocks_per_seq <= 0)
    return 0;
  CascadeSizes cs;
  const std::string saved = g_last_error;
  const pkv_status s = cascade_sizes(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                                     num_groups, max_group_size, max_shared_blocks, partition_tokens,
                                     prefix_partition_tokens, &cs);
  g_last_error = saved;  // a size query leaves the last error alone
  if (s != PKV_OK) return 0;
  const size_t fixed = cascade_workspace_bytes(num_seqs, num_heads, head_dim, cs);
  // as the call chooses; the cache kind (INT4 keeps fixed partitions) is
  // not known here, so enough for either layout
  if (!cascade_own_balanced(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_tokens,
                            max_shared_blocks, cs.spt, pkv::KvKind::BF16))
    return fixed;
  return std::max(fixed, cascade_balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim, cs.pparts,
                                                 kCascadeShareRounds * max_shares())
                             .total());
}

namespace {

// Shared-prefix decode, and (k_new set) the fused step that first writes
// each sequence's new token at position L - 1.
pkv_status cascade_call(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                        const void* v_cache, const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_start,
                        const int32_t* group_shared_blocks, float scale, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t num_groups, int32_t max_group_size, int32_t max_shared_blocks,
                        pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,
                        int32_t prefix_partition_tokens, void* workspace, size_t workspace_bytes, void* stream,
                        bool step) {
  // the plain checks first (sizes, dtypes, pointers); the workspace is
  // checked below against the cascade's own layout
  DecodeSetup st;
  pkv_status s = validate_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                 context_lens, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, num_blocks, q_dtype, kv_dtype,
                                 partition_tokens, nullptr, 0, k_new, v_new, step, &st,
                                 /*check_workspace=*/false);
  if (s != PKV_OK) return s;
  if (st.kv == pkv::KvKind::F32)
    return fail(PKV_ERR_UNSUPPORTED, "cascade decode supports bf16, int8, FP8 and INT4 caches only");
  CascadeSizes cs;
  s = cascade_sizes(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq, num_groups,
                    max_group_size, max_shared_blocks, partition_tokens, prefix_partition_tokens, &cs);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  if (!group_start || !group_shared_blocks)
    return fail(PKV_ERR_INVALID, "cascade decode needs group_start and group_shared_blocks");
  const bool bal = cascade_own_balanced(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_tokens,
                                        max_shared_blocks, cs.spt, st.kv);
  const int32_t shares = bal ? cascade_shares_for(st.kv) : 0;
  const CascadeBalancedLayout bl =
      cascade_balanced_layout(num_seqs, num_heads, num_kv_heads, head_dim, cs.pparts, shares);
  const size_t need = bal ? bl.total() : cascade_workspace_bytes(num_seqs, num_heads, head_dim, cs);
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (pkv::debug_checks_enabled()) {
    std::vector<int32_t> tables, lens;
    s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream,
                     &tables, &lens);
    if (s == PKV_OK)
      s = pkv::debug_check_groups(group_start, group_shared_blocks, tables, lens, num_seqs, max_blocks_per_seq,
                                  block_size, num_groups, max_group_size, max_shared_blocks,
                                  static_cast<hipStream_t>(stream), step);
    if (s != PKV_OK) return s;
  }
  pkv::DecodeParams& p = st.p;
  char* ws = static_cast<char*>(workspace);
  if (bal) {
    // shared tokens' partials in rows [B][H][pparts], then the shares' slots
    p.ws_acc = reinterpret_cast<float*>(ws);
    p.ws_m = reinterpret_cast<float*>(ws + bl.acc);
    p.ws_l = reinterpret_cast<float*>(ws + bl.acc + bl.ml);
    p.ws_unit = reinterpret_cast<int32_t*>(ws + bl.acc + 2 * bl.ml);
    p.bal_shares = shares;
    p.bal_row0 = static_cast<int64_t>(bl.rows_pre);
    p.num_parts = cs.pparts;
  } else {
    const size_t rows = static_cast<size_t>(num_seqs) * num_heads * (cs.pparts + cs.sparts);
    const size_t acc_bytes = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
    const size_t ml_bytes = (rows * sizeof(float) + 255) & ~size_t(255);
    p.ws_acc = reinterpret_cast<float*>(ws);
    p.ws_m = reinterpret_cast<float*>(ws + acc_bytes);
    p.ws_l = reinterpret_cast<float*>(ws + acc_bytes + ml_bytes);
    p.num_parts = cs.pparts + cs.sparts;
  }
  p.group_start = group_start;
  p.group_shared_blocks = group_shared_blocks;
  p.num_groups = num_groups;
  p.max_shared_blocks = max_shared_blocks;
  p.prefix_part_tokens = cs.ppt;
  p.stream_loads = 0;  // the shared blocks are read again from the memory-side cache
  p.prefix_parts = cs.pparts;
  p.part_tokens = cs.spt;
  const hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (st.kv != pkv::KvKind::I4) {
    // one launch: the shared-prefix workgroups and the shares of the
    // sequences' own tokens
    e = pkv::launch_cascade_fused(p, st.kv, max_group_size, strm);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "cascade kernel launch failed: %s", hipGetErrorString(e));
  } else {
    // prefix kernel on the side stream, partition kernel on the caller's,
    // joined before the reduce
    std::unique_lock<std::mutex> lock(g_side_mutex, std::defer_lock);
    SideStream* ss = nullptr;
    if (cs.pparts > 0) {
      lock.lock();
      e = side_stream(&ss);
      if (e == hipSuccess) e = hipEventRecord(ss->fork, strm);
      if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefix stream fork failed: %s", hipGetErrorString(e));
      e = pkv::launch_cascade_prefix(p, st.kv, max_group_size, ss->stream);
      if (e == hipSuccess) e = hipEventRecord(ss->join, ss->stream);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, "prefix kernel launch failed: %s", hipGetErrorString(e));
    }
    e = pkv::launch_decode_mfma(p, st.kv, strm);
    if (ss != nullptr) {  // join even after a failed launch: the prefix kernel writes the workspace
      const hipError_t ej = hipStreamWaitEvent(strm, ss->join, 0);
      if (e == hipSuccess && ej != hipSuccess)
        return fail(PKV_ERR_HIP, "prefix stream join failed: %s", hipGetErrorString(ej));
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "partition kernel launch failed: %s", hipGetErrorString(e));
  }
  e = pkv::launch_decode_reduce(p, st.out_bf16, strm);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "reduce kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

pkv_status pkv_paged_attention_decode_cascade(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_start, const int32_t* group_shared_blocks, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,
    int32_t prefix_partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return cascade_call(out, q, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                      group_start, group_shared_blocks, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, num_groups, max_group_size, max_shared_blocks,
                      q_dtype, kv_dtype, partition_tokens, prefix_partition_tokens, workspace, workspace_bytes,
                      stream, false);
}

pkv_status pkv_paged_attention_decode_cascade_step(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    float* k_scale, float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* group_start, const int32_t* group_shared_blocks, float scale, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_shared_blocks, pkv_dtype q_dtype, pkv_dtype kv_dtype, int32_t partition_tokens,
    int32_t prefix_partition_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return cascade_call(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                      group_start, group_shared_blocks, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                      block_size, max_blocks_per_seq, num_blocks, num_groups, max_group_size, max_shared_blocks,
                      q_dtype, kv_dtype, partition_tokens, prefix_partition_tokens, workspace, workspace_bytes,
                      stream, true);
}

pkv_status pkv_copy_blocks(void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                           const void* src_k, const void* src_v, const float* src_k_scale,
                           const float* src_v_scale, const int32_t* pairs, int32_t n,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, void* stream) {
  if (n < 0) return fail(PKV_ERR_INVALID, "copy_blocks: n must be >= 0");
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID, "copy_blocks: sizes must be positive");
  if (!head_dim_ok(head_dim)) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: head_dim %d not in {64, 128}", head_dim);
  if (!block_size_ok(block_size))
    return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: block_size %d not in {16, 32}", block_size);
  int64_t tile_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim;  // per element byte
  const bool coded = dtype == PKV_I8 || dtype == PKV_FP8 || dtype == PKV_I4 || dtype == PKV_FP8_E5M2;
  if (dtype == PKV_F32) tile_bytes *= 4;
  else if (dtype == PKV_BF16) tile_bytes *= 2;
  else if (dtype == PKV_I4) tile_bytes /= 2;  // two codes per byte
  else if (!coded) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: unknown dtype %d", static_cast<int>(dtype));
  if (n > 65535) return fail(PKV_ERR_UNSUPPORTED, "copy_blocks: at most 65535 pairs per call");
  if (n == 0) return ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs)
    return fail(PKV_ERR_INVALID, "copy_blocks: null pointer among the pools and pairs");
  if (coded && (!dst_k_scale || !dst_v_scale || !src_k_scale || !src_v_scale))
    return fail(PKV_ERR_INVALID, "copy_blocks: int8 / FP8 / INT4 pools need all four scale pointers");
  if (!coded && (dst_k_scale || dst_v_scale || src_k_scale || src_v_scale))
    return fail(PKV_ERR_INVALID, "copy_blocks: scale pointers must be NULL for fp32 / bf16 pools");
  // every pool must be device memory or host memory the device can address
  // (pinned); host memory is passed on as its device-side address
  const void* in[8] = {src_k, src_v, src_k_scale, src_v_scale, dst_k, dst_v, dst_k_scale, dst_v_scale};
  const void* dv[8] = {};
  for (int i = 0; i < 8; ++i) {
    if (!in[i]) continue;
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, in[i]) != hipSuccess) {
      (void)hipGetLastError();  // leave no error behind for later launches
      return fail(PKV_ERR_INVALID, "copy_blocks: pool %d is neither device memory nor pinned host memory", i);
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
      dv[i] = in[i];
    } else if (a.type == hipMemoryTypeHost) {
      void* d = nullptr;
      if (hipHostGetDevicePointer(&d, const_cast<void*>(in[i]), 0) != hipSuccess || !d) {
        (void)hipGetLastError();
        return fail(PKV_ERR_INVALID, "copy_blocks: host pool %d has no device address", i);
      }
      dv[i] = d;
    } else {
      return fail(PKV_ERR_INVALID, "copy_blocks: pool %d is not addressable by the device", i);
    }
  }
  pkv::CopyParams p{};
  for (int i = 0; i < 4; ++i) {
    p.src[i] = dv[i];
    p.dst[i] = const_cast<void*>(dv[4 + i]);
  }
  p.pairs = pairs;
  p.num_pairs = n;
  p.tile_bytes = tile_bytes;
  p.scale_bytes = coded ? static_cast<int64_t>(num_kv_heads) * block_size * 4 : 0;
  const hipError_t e = pkv::launch_copy_blocks(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "copy_blocks launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t pkv_paged_attention_multi_query_workspace_size(
    int32_t num_seqs, int32_t num_query_tokens, int32_t max_queries_per_seq, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t partition_tokens) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !head_dim_ok(head_dim) || !block_size_ok(block_size) || max_blocks_per_seq <= 0)
    return 0;
  MqSizes ms;
  const std::string saved = g_last_error;
  const pkv_status s = mq_sizes(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                                num_query_tokens, max_queries_per_seq, partition_tokens, &ms);
  g_last_error = saved;
  if (s != PKV_OK) return 0;
  return mq_workspace_bytes(num_query_tokens, num_heads, head_dim, ms.parts);
}

pkv_status pkv_paged_attention_multi_query(
    void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* query_start, float scale, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t num_query_tokens, int32_t max_queries_per_seq, pkv_dtype q_dtype,
    pkv_dtype kv_dtype, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
    void* stream) {
  DecodeSetup st;
  pkv_status s = validate_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                 context_lens, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                                 block_size, max_blocks_per_seq, num_blocks, q_dtype, kv_dtype, 0,
                                 nullptr, 0, nullptr, nullptr, false, &st, /*check_workspace=*/false);
  if (s != PKV_OK) return s;
  if (st.kv == pkv::KvKind::F32)
    return fail(PKV_ERR_UNSUPPORTED, "multi-query attention supports bf16, int8, FP8 and INT4 caches only");
  MqSizes ms;
  s = mq_sizes(num_seqs, num_heads, num_kv_heads, block_size, max_blocks_per_seq, num_query_tokens,
               max_queries_per_seq, partition_tokens, &ms);
  if (s != PKV_OK) return s;
  if (num_seqs == 0 || num_query_tokens == 0) return ok();
  if (!query_start) return fail(PKV_ERR_INVALID, "multi-query attention needs query_start");
  const size_t need = mq_workspace_bytes(num_query_tokens, num_heads, head_dim, ms.parts);
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (pkv::debug_checks_enabled()) {
    std::vector<int32_t> tables, lens;
    s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream,
                     &tables, &lens);
    if (s == PKV_OK)
      s = pkv::debug_check_query_start(query_start, lens, num_seqs, num_query_tokens, max_queries_per_seq,
                                       static_cast<hipStream_t>(stream));
    if (s != PKV_OK) return s;
  }
  pkv::DecodeParams& p = st.p;
  const size_t rows = static_cast<size_t>(num_query_tokens) * num_heads * ms.parts;
  const size_t acc_bytes = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  const size_t ml_bytes = (rows * sizeof(float) + 255) & ~size_t(255);
  char* ws = static_cast<char*>(workspace);
  p.ws_acc = reinterpret_cast<float*>(ws);
  p.ws_m = reinterpret_cast<float*>(ws + acc_bytes);
  p.ws_l = reinterpret_cast<float*>(ws + acc_bytes + ml_bytes);
  p.query_start = query_start;
  p.num_query_rows = num_query_tokens;
  p.part_tokens = ms.pt;
  p.num_parts = ms.parts;
  const hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (ms.decode_style) {
    p.mq_tiles = ms.qtiles;
    e = pkv::launch_multi_query_decode(p, st.kv, strm);
  } else {
    e = pkv::launch_multi_query(p, st.kv, max_queries_per_seq, strm);
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "multi-query kernel launch failed: %s", hipGetErrorString(e));
  e = pkv::launch_decode_reduce(p, st.out_bf16, strm);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "reduce kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const float* k_scale, const float* v_scale,
                                              const int32_t* block_tables, const int32_t* context_lens,
                                              float scale, int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t max_blocks_per_seq, int64_t num_blocks, pkv_dtype q_dtype,
                                              pkv_dtype kv_dtype, void* stream) {
  // the plain checks, then the partials' size against the scratch
  DecodeSetup st;
  pkv_status s = validate_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale,
                                 num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                 num_blocks, q_dtype, kv_dtype, 0, nullptr, 0, nullptr, nullptr, false, &st,
                                 /*check_workspace=*/false, /*allow_balanced=*/true);
  if (s != PKV_OK) return s;
  if (num_seqs == 0) return ok();
  if (st.need > PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "decode_noalloc: these sizes need %zu bytes of partials, more than its %zu-byte scratch "
                "(use pkv_paged_attention_decode with a workspace)",
                st.need, static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (st.need > 0) {
    const hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "decode_noalloc: scratch address lookup failed: %s", hipGetErrorString(e));
  }
  s = validate_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, q_dtype,
                      kv_dtype, 0, ws, ws ? PKV_NOALLOC_SCRATCH_BYTES : 0, nullptr, nullptr, false, &st,
                      /*check_workspace=*/true, /*allow_balanced=*/true);
  if (s != PKV_OK) return s;
  s = debug_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size, num_blocks, stream);
  if (s != PKV_OK) return s;
  s = launch_partitions(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  s = launch_reduce(st, static_cast<hipStream_t>(stream));
  if (s != PKV_OK) return s;
  return ok();
}

pkv_status pkv_probe_tile_read(const void* pool, const int32_t* tile_ids, int64_t num_tiles,
                               int32_t grid, int32_t streaming, uint32_t* sink, void* stream) {
  if (!pool || !tile_ids || !sink) return fail(PKV_ERR_INVALID, "probe_tile_read: null pointer");
  if (reinterpret_cast<uintptr_t>(pool) % 4096 != 0)
    return fail(PKV_ERR_INVALID, "probe_tile_read: pool is not 4096-byte aligned");
  if (num_tiles < 0) return fail(PKV_ERR_INVALID, "probe_tile_read: num_tiles < 0");
  if (grid < 1 || grid > 65536) return fail(PKV_ERR_INVALID, "probe_tile_read: grid %d not in [1, 65536]", grid);
  if (streaming != 0 && streaming != 1)
    return fail(PKV_ERR_INVALID, "probe_tile_read: streaming must be 0 or 1, got %d", streaming);
  if (num_tiles == 0) return ok();
  const hipError_t e = pkv::launch_tile_read(pool, tile_ids, num_tiles, grid, streaming != 0, sink,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "probe_tile_read launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

const char* pkv_version(void) { return "0.1.0"; }

}  // extern "C"
