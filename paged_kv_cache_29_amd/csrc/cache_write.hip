// Slot-scatter writes of new tokens into the paged KV cache.
//
// A new token's K and V go to the slot the block manager assigned it in its
// sequence's tail block ("LLM Engineering (5)", "Block manager: how paging
// works"); a slot is physical_block * block_size + row.  K rows are
// contiguous in the cache; V tiles hold groups of 4 tokens, dim-major
// inside a group (element (r, d) at ((r / 4) D + d) 4 + r % 4), so a
// token's V is every fourth element of its group (D / 16 lines of 128
// bytes at bf16).  Negative slots are skipped.
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

// Lane mapping of both writes: a wave takes 16 consecutive tokens of one
// kv-head (and, for the quantising write, K or V); lane 16 q + i holds token
// t0 + i and every fourth 16-byte piece q, q + 4, ... of its row.
// Consecutive lanes hold consecutive tokens, so when their slots are
// consecutive rows of one block (a prefill or bulk fill), each V store
// instruction writes the 4 contiguous elements of a token group's dim for
// every 4 lanes instead of scattering one element per line; the four lanes
// of a token load and store 64 contiguous bytes of its row at a time.
constexpr int kTokensPerWave = 16;

// The bit-copy write also has a small-batch form: a decode step writes one
// token per sequence, each into a different block, so every V element is a
// store to its own line, and scattered stores go through a CU's address
// path about one line per clock.  There a wave takes 4 tokens (16 lanes per
// token, one 16-byte piece each) and a workgroup is one wave, which spreads
// the stores over up to 4x as many waves and 4x as many CUs as the 16-token
// form (7B step, 32 tokens x 32 kv-heads: 16 CUs -> all 256).
//
// TPW tokens per wave; WPG waves per workgroup.
template <typename T, int D, int TPW, int WPG>
__global__ __launch_bounds__(WPG * kWave) void cache_write_kernel(WriteParams p) {
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  constexpr int LPT = kWave / TPW;     // lanes per token
  constexpr int NV = D / EPV;          // 16-byte vectors per row
  constexpr int VPL = (NV + LPT - 1) / LPT;  // vectors per lane per row
  const int BS = p.block_size;
  const int Hkv = p.num_kv_heads;
  const int lane = threadIdx.x & (kWave - 1);
  const int ti = lane % TPW;
  const int q = lane / TPW;
  const int64_t units = (p.num_tokens + TPW - 1) / TPW * Hkv;
  const T* __restrict__ k = static_cast<const T*>(p.k);
  const T* __restrict__ v = static_cast<const T*>(p.v);
  T* __restrict__ kc = static_cast<T*>(p.k_cache);
  T* __restrict__ vc = static_cast<T*>(p.v_cache);
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * WPG + threadIdx.x / kWave; u < units;
       u += static_cast<int64_t>(gridDim.x) * WPG) {
    const int64_t tg = u / Hkv;
    const int h = static_cast<int>(u - tg * Hkv);
    const int64_t t = tg * TPW + ti;
    if (t >= p.num_tokens) continue;
    const int64_t slot = p.slot_mapping[t];
    if (slot < 0) continue;
    const int64_t blk = slot / BS;
    const int row = static_cast<int>(slot - blk * BS);
    const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * D;
    const int64_t src = (t * Hkv + h) * D;
    // every load of the lane's share of the row first, then the stores: the
    // new rows and the cache are different buffers, and issuing the loads
    // together costs one memory latency instead of one per piece
    // (bf16 at D = 64 in the small-batch form: half the lanes of a token)
    if (NV % LPT != 0 && q >= NV) continue;
    u32x4 kk[VPL], vv[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int d0 = (LPT * j + q) * EPV;
      kk[j] = *reinterpret_cast<const u32x4*>(k + src + d0);
      vv[j] = *reinterpret_cast<const u32x4*>(v + src + d0);
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int d0 = (LPT * j + q) * EPV;
      *reinterpret_cast<u32x4*>(kc + tile + static_cast<int64_t>(row) * D + d0) = kk[j];
      const T* ve = reinterpret_cast<const T*>(&vv[j]);
      T* vg = vc + tile + static_cast<int64_t>(row >> 2) * D * 4 + (row & 3);  // the token's group
#pragma unroll
      for (int e = 0; e < EPV; ++e) vg[static_cast<int64_t>(d0 + e) * 4] = ve[e];
    }
  }
}

// The quantising write: one wave per (16 tokens, kv-head, K or V); the
// four lanes of a token each hold a quarter of its row (4 dims of every 16),
// all loaded before any is used, and the row's absmax is the max over the
// four lane groups.
// KV: I8 (s = absmax / 127, quantize_code), FP8 (s = absmax / 448, fp8_code),
// E5M2 (s = absmax / 57344, e5m2_code) or I4 (s = absmax / 7,
// quantize_sym<7>, tiles of half the bytes).
// Small-batch form as for the bit copy (TPW = 4, one wave per workgroup):
// a token's 16 lanes are contiguous there, and its absmax is a butterfly
// over them.
template <KvKind KV, int D, int TPW, int WPG>
__global__ __launch_bounds__(WPG * kWave) void cache_write_codes_kernel(WriteParams p) {
  constexpr float kMax = KV == KvKind::FP8    ? 448.0f
                         : KV == KvKind::E5M2 ? 57344.0f
                         : KV == KvKind::I4   ? 7.0f
                                              : 127.0f;
  static_assert(TPW == kTokensPerWave || TPW == 4, "token mappings");
  constexpr int LPT = kWave / TPW;     // lanes per token
  constexpr int NJ = D / 4 / LPT;      // 4-dim groups per lane
  const int BS = p.block_size;
  const int Hkv = p.num_kv_heads;
  const int lane = threadIdx.x & (kWave - 1);
  const int ti = TPW == kTokensPerWave ? (lane & 15) : lane / LPT;
  const int q = TPW == kTokensPerWave ? (lane >> 4) : lane % LPT;
  const int64_t units = (p.num_tokens + TPW - 1) / TPW * Hkv * 2;
  const float* __restrict__ k = static_cast<const float*>(p.k);
  const float* __restrict__ v = static_cast<const float*>(p.v);
  uint8_t* __restrict__ kc = static_cast<uint8_t*>(p.k_cache);
  uint8_t* __restrict__ vc = static_cast<uint8_t*>(p.v_cache);
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * WPG + threadIdx.x / kWave; u < units;
       u += static_cast<int64_t>(gridDim.x) * WPG) {
    // u = ((token group) * Hkv + head) * 2 + (K or V): uniform across the wave
    const bool is_v = (u & 1) != 0;
    const int64_t th = u >> 1;
    const int64_t tg = th / Hkv;
    const int h = static_cast<int>(th - tg * Hkv);
    const int64_t t = tg * TPW + ti;
    const int64_t slot = t < p.num_tokens ? p.slot_mapping[t] : -1;
    const float* src = (is_v ? v : k) + (t * Hkv + h) * D;
    f32x4 x[NJ];                       // groups of 4 dims: dims 4 (LPT j + q) + e
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (slot >= 0) x[j] = *reinterpret_cast<const f32x4*>(src + 4 * (LPT * j + q));
    }
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      a = fmaxf(a, fmaxf(fmaxf(fabsf(x[j][0]), fabsf(x[j][1])), fmaxf(fabsf(x[j][2]), fabsf(x[j][3]))));
    // every lane of the wave takes part
    if constexpr (TPW == kTokensPerWave) {
      a = groups_max(a);  // a token's lanes i, i + 16, i + 32, i + 48
    } else {
#pragma unroll
      for (int o = LPT / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
    }
    if (slot < 0) continue;
    const float s = a / kMax;
    const int64_t blk = slot / BS;
    const int row = static_cast<int>(slot - blk * BS);
    if (q == 0) (is_v ? p.v_scale : p.k_scale)[(blk * Hkv + h) * BS + row] = (s > 0.f) ? s : 0.f;
    if constexpr (KV == KvKind::I4) {
      const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * (D / 2);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int d0 = 4 * (LPT * j + q);
        const uint32_t b0 = pack_int4_pair(quantize_sym<7>(x[j][0], s), quantize_sym<7>(x[j][1], s));
        const uint32_t b1 = pack_int4_pair(quantize_sym<7>(x[j][2], s), quantize_sym<7>(x[j][3], s));
        if (!is_v) {
          *reinterpret_cast<uint16_t*>(kc + tile + static_cast<int64_t>(row) * (D / 2) + d0 / 2) =
              static_cast<uint16_t>(b0 | (b1 << 8));
        } else {
          uint8_t* vg = vc + tile + static_cast<int64_t>(row >> 2) * (D / 2) * 4 + (row & 3);
          vg[static_cast<int64_t>(d0 / 2) * 4] = static_cast<uint8_t>(b0);
          vg[static_cast<int64_t>(d0 / 2 + 1) * 4] = static_cast<uint8_t>(b1);
        }
      }
      continue;
    }
    const int64_t tile = (blk * Hkv + h) * static_cast<int64_t>(BS) * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d0 = 4 * (LPT * j + q);
      uint32_t codes[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        codes[e] = KV == KvKind::FP8    ? fp8_code(x[j][e], s)
                   : KV == KvKind::E5M2 ? e5m2_code(x[j][e], s)
                                        : static_cast<uint32_t>(quantize_code(x[j][e], s));
      if (!is_v) {
        const uint32_t packed = (codes[0] & 0xffu) | ((codes[1] & 0xffu) << 8) |
                                ((codes[2] & 0xffu) << 16) | ((codes[3] & 0xffu) << 24);
        *reinterpret_cast<uint32_t*>(kc + tile + static_cast<int64_t>(row) * D + d0) = packed;
      } else {
        uint8_t* vg = vc + tile + static_cast<int64_t>(row >> 2) * D * 4 + (row & 3);
#pragma unroll
        for (int e = 0; e < 4; ++e) vg[static_cast<int64_t>(d0 + e) * 4] = static_cast<uint8_t>(codes[e] & 0xffu);
      }
    }
  }
}

unsigned grid_for(int64_t work, int per_block) {
  const int64_t blocks = (work + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;  // enough workgroups to fill 256 CUs many times over
  return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

template <KvKind KV, int D>
hipError_t launch_codes_t(const WriteParams& p, hipStream_t s) {
  // as launch_write_t: 16-token waves, or 4-token waves for small batches
  const int64_t waves16 = (p.num_tokens + kTokensPerWave - 1) / kTokensPerWave * p.num_kv_heads * 2;
  if (waves16 < 1024) {
    const int64_t waves4 = (p.num_tokens + 3) / 4 * p.num_kv_heads * 2;
    hipLaunchKernelGGL((cache_write_codes_kernel<KV, D, 4, 1>), dim3(grid_for(waves4, 1)), dim3(kWave), 0, s, p);
  } else {
    hipLaunchKernelGGL((cache_write_codes_kernel<KV, D, kTokensPerWave, 4>), dim3(grid_for(waves16, 4)),
                       dim3(4 * kWave), 0, s, p);
  }
  return hipGetLastError();
}

template <KvKind KV>
hipError_t launch_codes(const WriteParams& p, hipStream_t s) {
  return p.head_dim == 128 ? launch_codes_t<KV, 128>(p, s) : launch_codes_t<KV, 64>(p, s);  // else 64
}


}  // namespace

template <typename T, int D>
hipError_t launch_write_t(const WriteParams& p, hipStream_t s) {
  // 16-token waves, four per workgroup; fewer than 1024 such waves (four
  // per CU) is a small batch: 4-token waves, one per workgroup
  const int64_t waves16 = (p.num_tokens + kTokensPerWave - 1) / kTokensPerWave * p.num_kv_heads;
  if (waves16 < 1024) {
    const int64_t waves4 = (p.num_tokens + 3) / 4 * p.num_kv_heads;
    hipLaunchKernelGGL((cache_write_kernel<T, D, 4, 1>), dim3(grid_for(waves4, 1)), dim3(kWave), 0, s, p);
  } else {
    hipLaunchKernelGGL((cache_write_kernel<T, D, kTokensPerWave, 4>), dim3(grid_for(waves16, 4)),
                       dim3(4 * kWave), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_cache_write(const WriteParams& p, KvKind kind, hipStream_t s) {
  const bool d128 = p.head_dim == 128;  // else 64 (validated by the caller)
  if (kind == KvKind::F32) return d128 ? launch_write_t<float, 128>(p, s) : launch_write_t<float, 64>(p, s);
  return d128 ? launch_write_t<uint16_t, 128>(p, s) : launch_write_t<uint16_t, 64>(p, s);
}

hipError_t launch_cache_write_codes(const WriteParams& p, KvKind kind, hipStream_t s) {
  if (kind == KvKind::FP8) return launch_codes<KvKind::FP8>(p, s);
  if (kind == KvKind::I4) return launch_codes<KvKind::I4>(p, s);
  if (kind == KvKind::E5M2) return launch_codes<KvKind::E5M2>(p, s);
  return launch_codes<KvKind::I8>(p, s);
}

}  // namespace pkv
