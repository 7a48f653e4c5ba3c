// Tile-gather read probe: the decode kernel's HBM access pattern (whole
// 4 KB tiles at positions an index list names) with no arithmetic, to
// measure the read rate the device sustains for that pattern, with the
// default load policy or with the non-temporal hint that decode over a
// large cache pool uses.

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kTileBytes = 4096;
constexpr int kLoadsPerTile = kTileBytes / (16 * kWave);  // 16-byte loads per lane
constexpr int kTilesInFlight = 4;

template <bool kNT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (kNT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool kNT>
__global__ __launch_bounds__(256) void tile_read_kernel(const char* pool, const int32_t* ids,
                                                        int64_t ntiles, uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * blockDim.x / kWave;
  uint32_t acc = 0;
  int64_t t = wave;
  for (; t + (kTilesInFlight - 1) * nwaves < ntiles; t += kTilesInFlight * nwaves) {
    u32x4 v[kTilesInFlight][kLoadsPerTile];
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u) {
      const u32x4* tile = reinterpret_cast<const u32x4*>(
          pool + static_cast<int64_t>(ids[t + u * nwaves]) * kTileBytes);
#pragma unroll
      for (int j = 0; j < kLoadsPerTile; ++j) v[u][j] = load16<kNT>(tile + j * kWave + lane);
    }
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u)
#pragma unroll
      for (int j = 0; j < kLoadsPerTile; ++j) acc ^= v[u][j].x ^ v[u][j].y ^ v[u][j].z ^ v[u][j].w;
  }
  for (; t < ntiles; t += nwaves) {
    const u32x4* tile = reinterpret_cast<const u32x4*>(pool + static_cast<int64_t>(ids[t]) * kTileBytes);
#pragma unroll
    for (int j = 0; j < kLoadsPerTile; ++j) {
      const u32x4 v = load16<kNT>(tile + j * kWave + lane);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_tile_read(const void* pool, const int32_t* ids, int64_t ntiles, int grid, bool streaming,
                            uint32_t* sink, hipStream_t s) {
  if (streaming)
    hipLaunchKernelGGL(tile_read_kernel<true>, dim3(grid), dim3(256), 0, s, static_cast<const char*>(pool), ids,
                       ntiles, sink);
  else
    hipLaunchKernelGGL(tile_read_kernel<false>, dim3(grid), dim3(256), 0, s, static_cast<const char*>(pool), ids,
                       ntiles, sink);
  return hipGetLastError();
}

}  // namespace pkv
