// Shared-prefix ("cascade") decode and LDS-staged multi-query attention:
// the kernel over prefix_body.hpp's workgroups, one per block of the grid
// (group or sequence * Hkv + kv-head, query tile, partition), and its
// launchers.

#include "prefix_body.hpp"

namespace pkv {
namespace {

template <KvKind KV, int D, int BS, int NT, bool kMQ>
__global__ __launch_bounds__(kDecodeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(kPrefixWavesPerSimd<NT>, kPrefixWavesPerSimd<NT>)))
void cascade_prefix_kernel(DecodeParams p) {
  prefix_body<KV, D, BS, NT, kMQ>(p, blockIdx.x, blockIdx.y, blockIdx.z);
}

// max_rows: largest group (cascade) or most new tokens per sequence
// (multi-query); units: groups or sequences; parts: partitions of the span.
template <KvKind KV, int D, int BS, bool kMQ>
hipError_t launch_t(const DecodeParams& p, int units, int max_rows, int parts, hipStream_t s) {
  const int G = p.num_heads / p.num_kv_heads;
  const int64_t cols = static_cast<int64_t>(max_rows) * G;
  const int64_t qtiles = (cols + prefix_queries_for(cols) - 1) / prefix_queries_for(cols);
  const dim3 grid(static_cast<unsigned>(units * p.num_kv_heads), static_cast<unsigned>(qtiles),
                  static_cast<unsigned>(parts));
  static_assert(kPrefixTiles == 2, "one instance per tile count");
  if (prefix_tiles_for(cols) == 1)
    hipLaunchKernelGGL((cascade_prefix_kernel<KV, D, BS, 1, kMQ>), grid, dim3(kDecodeWaves * kWave), 0, s, p);
  else
    hipLaunchKernelGGL((cascade_prefix_kernel<KV, D, BS, 2, kMQ>), grid, dim3(kDecodeWaves * kWave), 0, s, p);
  return hipGetLastError();
}

template <KvKind KV, bool kMQ>
hipError_t launch_kv(const DecodeParams& p, int units, int max_rows, int parts, hipStream_t s) {
  if (p.head_dim == 128)
    return p.block_size == 16 ? launch_t<KV, 128, 16, kMQ>(p, units, max_rows, parts, s)
                              : launch_t<KV, 128, 32, kMQ>(p, units, max_rows, parts, s);
  return p.block_size == 16 ? launch_t<KV, 64, 16, kMQ>(p, units, max_rows, parts, s)
                            : launch_t<KV, 64, 32, kMQ>(p, units, max_rows, parts, s);
}

template <bool kMQ>
hipError_t launch_mode(const DecodeParams& p, KvKind kv, int units, int max_rows, int parts, hipStream_t s) {
  if (kv == KvKind::I8) return launch_kv<KvKind::I8, kMQ>(p, units, max_rows, parts, s);
  if (kv == KvKind::I4) return launch_kv<KvKind::I4, kMQ>(p, units, max_rows, parts, s);
  if (kv == KvKind::FP8) return launch_kv<KvKind::FP8, kMQ>(p, units, max_rows, parts, s);
  if (kv == KvKind::E5M2) return launch_kv<KvKind::E5M2, kMQ>(p, units, max_rows, parts, s);
  return launch_kv<KvKind::BF16, kMQ>(p, units, max_rows, parts, s);
}

}  // namespace

hipError_t launch_cascade_prefix(const DecodeParams& p, KvKind kv, int max_group_size, hipStream_t s) {
  return launch_mode<false>(p, kv, p.num_groups, max_group_size, p.prefix_parts, s);
}

hipError_t launch_multi_query(const DecodeParams& p, KvKind kv, int max_queries, hipStream_t s) {
  return launch_mode<true>(p, kv, p.num_seqs, max_queries, p.num_parts, s);
}

}  // namespace pkv
