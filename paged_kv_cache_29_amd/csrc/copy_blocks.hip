// Whole-block copies between two KV pools: copy-on-write copies inside the
// device pool, and swapping blocks out to / back from pinned host memory
// ("LLM Engineering (5)", "Block manager: how paging works").
//
// Block b of a pool is four contiguous byte ranges: its K tiles
// k[b][Hkv][bs][D], its V tiles v[b][Hkv][bs/4][D][4] (INT4: half the bytes) and,
// for int8 / FP8 / INT4 caches, its scale rows k_scale[b][Hkv][bs],
// v_scale[b][Hkv][bs].  Workgroup
// (pair, part, piece) copies one 16 KB piece of one part of one pair with
// 16-byte loads and stores; a pool in pinned host memory is read or written
// over the host link directly.

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kPieceBytes = 16384;

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
  const int pair = blockIdx.x;
  const int part = blockIdx.y;
  const int64_t bytes = part < 2 ? p.tile_bytes : p.scale_bytes;
  const int64_t off0 = static_cast<int64_t>(blockIdx.z) * kPieceBytes;
  if (off0 >= bytes) return;  // uniform
  const int64_t src_blk = p.pairs[2 * pair];
  const int64_t dst_blk = p.pairs[2 * pair + 1];
  const char* src = static_cast<const char*>(p.src[part]) + src_blk * bytes;
  char* dst = static_cast<char*>(p.dst[part]) + dst_blk * bytes;
  const int64_t end = min(bytes, off0 + kPieceBytes);
  for (int64_t o = off0 + 16 * static_cast<int64_t>(threadIdx.x); o < end; o += 16 * 256)
    *reinterpret_cast<u32x4*>(dst + o) = *reinterpret_cast<const u32x4*>(src + o);
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t s) {
  const int parts = p.scale_bytes > 0 ? 4 : 2;
  const int64_t pieces = (p.tile_bytes + kPieceBytes - 1) / kPieceBytes;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(p.num_pairs, parts, static_cast<unsigned>(pieces)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
