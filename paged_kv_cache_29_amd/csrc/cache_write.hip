// Slot-scatter writes of new tokens into the paged KV cache.
//
// A new token's K and V go to the slot the block manager assigned it in its
// sequence's tail block ("LLM Engineering (5)", "Block manager: how paging
// works"); a slot is physical_block * block_size + row.  K rows are
// contiguous in the cache; V tiles are dim-major, so a token's V is a column
// of its tile (stride block_size).  Negative slots are skipped.
//
// kv_cache_write copies bits.  kv_cache_write_int8 first quantises each
// (token, kv-head) row on its own: s = absmax / 127 in IEEE fp32,
// code = clamp(rint(x / s), -127, 127); a row whose scale is 0 (all zero,
// or absmax / 127 underflows) gets s = 0 and code 0
// ("LLM Engineering (5)", "KV-cache quantization" and "INT8 weight-only
// quantization"; four-layer inference-optimization article, 2.3).
// kv_cache_write_fp8 does the same with s = absmax / 448 and the nearest
// OCP E4M3 code of x / s (the same section's FP8 KV caches).
// kv_cache_write_fp8_e5m2 does the same with the E5M2 format (s = absmax /
// 57344).  kv_cache_write_int4 uses s = absmax / 7 and codes clamp(rint(x / s), -7, 7),
// stored two per byte (two consecutive head dims of one token, the lower dim
// in the low nibble, 4-bit two's complement); no byte holds two tokens, so
// tokens are written independently.  This
// translation unit is built without fast-math and with correctly rounded
// fp32 division, so the codes and scales are bit-exact.

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(WriteParams p) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  const int D = p.head_dim;
  const int BS = p.block_size;
  const int Hkv = p.num_kv_heads;
  const int vecs = D / EPV;
  const int64_t total = p.num_tokens * Hkv * vecs;
  const T* k = static_cast<const T*>(p.k);
  const T* v = static_cast<const T*>(p.v);
  T* kc = static_cast<T*>(p.k_cache);
  T* vc = static_cast<T*>(p.v_cache);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t th = i / vecs;  // token * Hkv + head
    const int vi = static_cast<int>(i - th * vecs);
    const int64_t t = th / Hkv;
    const int h = static_cast<int>(th - t * Hkv);
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0) continue;
    const int64_t blk = slot / BS;
    const int row = static_cast<int>(slot - blk * BS);
    const int d0 = vi * EPV;
    const int64_t src = th * D + d0;
    const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * D;
    *reinterpret_cast<u32x4*>(kc + tile + static_cast<int64_t>(row) * D + d0) =
        *reinterpret_cast<const u32x4*>(k + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
    const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
    for (int e = 0; e < EPV; ++e) vc[tile + static_cast<int64_t>(d0 + e) * BS + row] = ve[e];
  }
}

// One lane group of D/4 lanes per (token, kv-head, K-or-V) row, 4 values per
// lane; rows alternate K, V.
// KV: I8 (s = absmax / 127, quantize_code), FP8 (s = absmax / 448, fp8_code),
// E5M2 (s = absmax / 57344, e5m2_code) or I4 (s = absmax / 7,
// quantize_sym<7>, tiles of half the bytes).
template <KvKind KV>
__global__ __launch_bounds__(256) void cache_write_codes_kernel(WriteParams p) {
  const int D = p.head_dim;
  const int BS = p.block_size;
  const int Hkv = p.num_kv_heads;
  const int group = D / 4;                    // lanes per row (16 or 32)
  const int rows_per_block = blockDim.x / group;
  const int sub = threadIdx.x % group;
  const int64_t total_rows = p.num_tokens * Hkv * 2;
  const float* k = static_cast<const float*>(p.k);
  const float* v = static_cast<const float*>(p.v);
  uint8_t* kc = static_cast<uint8_t*>(p.k_cache);
  uint8_t* vc = static_cast<uint8_t*>(p.v_cache);
  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block; r0 < total_rows;
       r0 += static_cast<int64_t>(gridDim.x) * rows_per_block) {
    const int64_t r = r0 + threadIdx.x / group;
    // every lane of a row group takes the same branch; the shuffles below
    // stay inside the group (xor offsets < group)
    const bool live = r < total_rows;
    const int64_t th = live ? (r >> 1) : 0;
    const bool is_v = (r & 1) != 0;
    const int64_t t = th / Hkv;
    const int h = static_cast<int>(th - t * Hkv);
    const int64_t slot = live ? p.slot_mapping[t] : -1;
    const float* src = (is_v ? v : k) + th * D + 4 * sub;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (slot >= 0) x = *reinterpret_cast<const f32x4*>(src);
    float a = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    for (int o = group / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
    if (slot < 0) continue;
    const float s = a / (KV == KvKind::FP8    ? 448.0f
                         : KV == KvKind::E5M2 ? 57344.0f
                         : KV == KvKind::I4   ? 7.0f
                                              : 127.0f);
    const int64_t blk = slot / BS;
    const int row = static_cast<int>(slot - blk * BS);
    const int d0 = 4 * sub;
    if constexpr (KV == KvKind::I4) {
      // dims d0 .. d0+3 -> bytes d0/2 and d0/2 + 1 of the token
      const uint32_t b0 = pack_int4_pair(quantize_sym<7>(x[0], s), quantize_sym<7>(x[1], s));
      const uint32_t b1 = pack_int4_pair(quantize_sym<7>(x[2], s), quantize_sym<7>(x[3], s));
      const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * (D / 2);
      const int j = d0 / 2;
      if (!is_v) {
        *reinterpret_cast<uint16_t*>(kc + tile + static_cast<int64_t>(row) * (D / 2) + j) =
            static_cast<uint16_t>(b0 | (b1 << 8));
      } else {
        vc[tile + static_cast<int64_t>(j) * BS + row] = static_cast<uint8_t>(b0);
        vc[tile + static_cast<int64_t>(j + 1) * BS + row] = static_cast<uint8_t>(b1);
      }
      if (sub == 0) (is_v ? p.v_scale : p.k_scale)[(blk * Hkv + h) * BS + row] = (s > 0.f) ? s : 0.f;
      continue;
    }
    uint32_t codes[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      codes[e] = KV == KvKind::FP8    ? fp8_code(x[e], s)
                 : KV == KvKind::E5M2 ? e5m2_code(x[e], s)
                                      : static_cast<uint32_t>(quantize_code(x[e], s));
    const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * D;
    if (!is_v) {
      const uint32_t packed = (codes[0] & 0xffu) | ((codes[1] & 0xffu) << 8) |
                              ((codes[2] & 0xffu) << 16) | ((codes[3] & 0xffu) << 24);
      *reinterpret_cast<uint32_t*>(kc + tile + static_cast<int64_t>(row) * D + d0) = packed;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vc[tile + static_cast<int64_t>(d0 + e) * BS + row] = static_cast<uint8_t>(codes[e] & 0xffu);
    }
    if (sub == 0) {
      const float sc = (s > 0.f) ? s : 0.f;
      (is_v ? p.v_scale : p.k_scale)[(blk * Hkv + h) * BS + row] = sc;
    }
  }
}

unsigned grid_for(int64_t work, int per_block) {
  const int64_t blocks = (work + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;  // enough workgroups to fill 256 CUs many times over
  return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

}  // namespace

hipError_t launch_cache_write(const WriteParams& p, KvKind kind, hipStream_t s) {
  const int epv = kind == KvKind::F32 ? 4 : 8;
  const int64_t work = p.num_tokens * p.num_kv_heads * (p.head_dim / epv);
  const unsigned grid = grid_for(work, 256);
  if (kind == KvKind::F32)
    hipLaunchKernelGGL(cache_write_kernel<float>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(cache_write_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_cache_write_codes(const WriteParams& p, KvKind kind, hipStream_t s) {
  const int rows_per_block = 256 / (p.head_dim / 4);
  const unsigned grid = grid_for(p.num_tokens * p.num_kv_heads * 2, rows_per_block);
  if (kind == KvKind::FP8)
    hipLaunchKernelGGL(cache_write_codes_kernel<KvKind::FP8>, dim3(grid), dim3(256), 0, s, p);
  else if (kind == KvKind::I4)
    hipLaunchKernelGGL(cache_write_codes_kernel<KvKind::I4>, dim3(grid), dim3(256), 0, s, p);
  else if (kind == KvKind::E5M2)
    hipLaunchKernelGGL(cache_write_codes_kernel<KvKind::E5M2>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(cache_write_codes_kernel<KvKind::I8>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
