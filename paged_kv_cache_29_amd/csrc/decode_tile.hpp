// Loading (block, kv-head) K/V tiles as matrix-core operands on gfx950:
// shared by the decode partition kernel and the shared-prefix kernel.
//
// A 32-token chunk is two 16-token sub-tiles h = 0, 1 (two blocks at
// bs = 16, the two halves of one block at bs = 32).  Lane l = 16 g + c loads
//   K: row c of each sub-tile, 8 dims per operand (the A operand of
//      v_mfma_f32_16x16x32_bf16: row l % 16, contraction 8 (l / 16) + e);
//   V: tokens 4g .. 4g+3 of the sub-tile (its token group g) for several
//      dims at once.  V tiles are stored in groups of 4 tokens, dim-major
//      inside a group (element (r, d) at ((r / 4) D + d) 4 + r % 4), so the
//      4 tokens of one dim are contiguous and one 16-byte load holds them
//      for 2 dims (bf16), 4 dims (byte codes) or 4 dim pairs (INT4): the
//      dims 2c, 2c + 1 (4c .. 4c + 3, pairs 4c .. 4c + 3) of a 32-dim
//      (64-dim, 64-pair) block.  Operand n of the PV contraction is one of
//      those dims; which dim a tile row holds does not matter to the
//      contraction, only to where the outputs are written (the kernels'
//      output maps);
//   int8 scales of tokens 4g .. 4g+3.
// Every load is a buffer descriptor over one tile (uniform: scalar
// registers) plus a loop-invariant lane offset.
#pragma once

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 load_u32x2(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ f32x4 load_f32x4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Two int8 codes (bytes 2*half and 2*half+1 of w) -> packed bf16 pair.
// |code| <= 128 has at most 8 significant bits, so the fp32 value is exact
// and its upper half is the exact bf16; one byte permute packs both halves.
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int half) {
  const int32_t lo = static_cast<int32_t>(w << (24 - 16 * half)) >> 24;
  const int32_t hi = static_cast<int32_t>(w << (16 - 16 * half)) >> 24;
  const uint32_t flo = __float_as_uint(static_cast<float>(lo));
  const uint32_t fhi = __float_as_uint(static_cast<float>(hi));
  // result bytes (low to high): flo[2], flo[3], fhi[2], fhi[3]
  return __builtin_amdgcn_perm(fhi, flo, 0x07060302u);
}

// Two FP8 (OCP E4M3) codes (bytes 2*HALF and 2*HALF+1 of w) -> packed bf16
// pair.  Every E4M3 value (subnormals included) is a bf16 value, so the
// hardware conversion with scale 1 is exact.
template <int HALF>
__device__ __forceinline__ uint32_t fp8pair_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HALF != 0));
}

// Two E5M2 codes -> packed bf16 pair (exact: every E5M2 value is a bf16
// value, and no cached code is an infinity or NaN by construction).
template <int HALF>
__device__ __forceinline__ uint32_t e5m2pair_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HALF != 0));
}

// Byte codes of a cache of kind KV (I8, FP8 or E5M2) -> exact bf16 values.
template <KvKind KV, int HALF>
__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t w) {
  if constexpr (KV == KvKind::FP8)
    return fp8pair_to_bf16x2<HALF>(w);
  else if constexpr (KV == KvKind::E5M2)
    return e5m2pair_to_bf16x2<HALF>(w);
  else
    return i8pair_to_bf16x2(w, HALF);
}

// 8 byte codes -> one bf16x8 operand.
template <KvKind KV>
__device__ __forceinline__ bf16x8 codes8_to_bf16(uint32_t w0, uint32_t w1) {
  return as_bf16x8(u32x4{codes_to_bf16x2<KV, 0>(w0), codes_to_bf16x2<KV, 1>(w0),
                         codes_to_bf16x2<KV, 0>(w1), codes_to_bf16x2<KV, 1>(w1)});
}

// INT4 codes (two per byte, 4-bit two's complement) -> bf16 operands.
// Flipping each nibble's top bit turns code c into the unsigned u = c + 8,
// and the bf16 bit pattern 0x4300 | u is the integer 128 + u exactly, so a
// byte permute builds two operands per instruction: every element carries
// the value c + 136, and the kernels subtract the offset's contribution
// (136 times the sum of the other operand) once per contraction.
constexpr float kInt4Offset = 136.0f;

// Nibbles of w, offset: lo = low nibble of each byte, hi = high nibble.
__device__ __forceinline__ void int4_nibbles(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x88888888u;
  lo = u & 0x0f0f0f0fu;
  hi = (u >> 4) & 0x0f0f0f0fu;
}

// Bytes 0, 1 (HALF 0) or 2, 3 (HALF 1) of n (nibble values) -> bf16 pair.
template <int HALF>
__device__ __forceinline__ uint32_t nib_pair_to_bf16x2(uint32_t n) {
  // result bytes: n[2 HALF], 0x43, n[2 HALF + 1], 0x43 (0x43 from the high word)
  return __builtin_amdgcn_perm(0x43434343u, n, HALF ? 0x04030402u : 0x04010400u);
}

// The four bytes of n -> one half (4 elements) of a bf16x8 operand.
__device__ __forceinline__ u32x2 nib4_to_bf16(uint32_t n) {
  return u32x2{nib_pair_to_bf16x2<0>(n), nib_pair_to_bf16x2<1>(n)};
}

// Zero the bf16 elements (pairs packed in w) whose token is >= t_end.
__device__ __forceinline__ uint32_t mask_pair(uint32_t w, int tok, int t_end) {
  const uint32_t lo = (tok < t_end) ? (w & 0xffffu) : 0u;
  const uint32_t hi = (tok + 1 < t_end) ? (w & 0xffff0000u) : 0u;
  return lo | hi;
}

// Raw loads of one 32-token chunk for one lane.  The chunk is two 16-token
// sub-tiles h = 0, 1 (two blocks at bs = 16, the two halves of one block at
// bs = 32).
template <bool kInt8, int D>
struct Chunk {
  static constexpr int NJ = D / 32;
  static constexpr int NN = D / 16;
  // K rows: per sub-tile h, NJ operands of 8 dims (bf16: 16 B each; int8:
  // one 16-byte load feeds two operands, so NJ/2 loads)
  u32x4 k[2][kInt8 ? NJ / 2 : NJ];
  // V^T: per sub-tile h and operand n, tokens 4g .. 4g+3 of one dim (bf16:
  // 8 B, dim 32 (n / 2) + 2c + n % 2; byte codes: 4 B, dim
  // 64 (n / 4) + 4c + n % 4)
  typename std::conditional<kInt8, uint32_t, u32x2>::type v[2][NN];
  f32x4 ks[2], vs[2];  // int8 scales of sub-tile tokens 4g .. 4g+3
};

// Buffer-resource word 3 for raw (untyped, unswizzled) buffers on gfx9-class
// GPUs: 32-bit data format, no stride.
constexpr int kBufferFlags = 0x00020000;

// Cache policy bits of a buffer load: 0 = the default; kNonTemporal = the
// non-temporal hint (nt), for data read once: on MI355X it keeps the loaded
// lines from being kept in the memory-side cache, which raises the read rate
// of a scattered-tile stream (2 GiB of shuffled 4 KB tiles: 5.95 -> 6.65 TB/s)
// but forgoes that cache for data read again (a shared prefix, or a pool
// small enough to stay cached between steps).
constexpr int kNonTemporal = 2;

// POL: the cache policy of the K/V tile loads (0 or kNonTemporal); scale
// rows are always loaded with the default policy (kv-head pairs share them).
template <bool kInt8, int D, int BS, int POL = 0>
struct ChunkLoader {
  using KT = typename std::conditional<kInt8, int8_t, uint16_t>::type;
  static constexpr uint32_t kElem = sizeof(KT);
  static constexpr uint32_t kTileBytes = BS * D * kElem;
  const char* kc;   // cache base addresses (bytes)
  const char* vc;
  const char* ksc;  // int8 scale arrays (bytes)
  const char* vsc;
  int Hkv, kvh;
  // loop-invariant per-lane byte offsets inside a (block, kv-head) tile
  uint32_t koff, voff, soff;

  __device__ __forceinline__ ChunkLoader(const DecodeParams& p, int kvh_, int c, int g)
      : kc(static_cast<const char*>(p.k_cache)), vc(static_cast<const char*>(p.v_cache)),
        ksc(reinterpret_cast<const char*>(p.k_scale)), vsc(reinterpret_cast<const char*>(p.v_scale)),
        Hkv(p.num_kv_heads), kvh(kvh_) {
    // K: row c of the sub-tile; dims 32j + 8g (bf16) or 64jj + 16g (int8)
    koff = (static_cast<uint32_t>(c) * D + (kInt8 ? 16u : 8u) * g) * kElem;
    // V: token group g of the sub-tile, dims 2c, 2c + 1 (bf16) or
    // 4c .. 4c + 3 (byte codes) of each 32- (64-) dim block
    voff = (static_cast<uint32_t>(g) * D + (kInt8 ? 4u : 2u) * c) * 4u * kElem;
    soff = 4u * g * 4u;
  }

  // Buffer resource over one (block, kv-head) tile: the base is uniform, so
  // the descriptor lives in scalar registers and every load is
  // "descriptor + 32-bit lane offset", with no vector address arithmetic.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t tile(const char* base, size_t off, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), static_cast<short>(0),
                                             static_cast<int>(bytes), kBufferFlags);
  }

  // blk[h]: physical block of sub-tile h; row0[h]: its first row in the block.
  __device__ __forceinline__ void load(Chunk<kInt8, D>& ch, const int blk[2], const int row0[2]) const {
    constexpr int NJ = D / 32;
    constexpr int NN = D / 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t t = static_cast<size_t>(blk[h]) * Hkv + kvh;
      const __amdgpu_buffer_rsrc_t rk = tile(kc, t * kTileBytes, kTileBytes);
      const __amdgpu_buffer_rsrc_t rv = tile(vc, t * kTileBytes, kTileBytes);
      // uniform offsets (row of the sub-tile, per-load constants) go in the
      // scalar offset operand, so the lane offset is the only vector input;
      // the sub-tile's first row is a multiple of 4, so its token groups
      // start at row0 * D elements
      const int ks_row = row0[h] * D * kElem;
      const int vs_row = row0[h] * D * kElem;
      if constexpr (kInt8) {
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj)
          ch.k[h][jj] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, ks_row + 64 * jj, POL));
        // V: tokens 4g .. 4g+3 of dims 64k + 4c + j, j = 0..3 (operand
        // n = 4k + j), one 16-byte load per 64 dims
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const u32x4 w = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, vs_row + 256 * k, POL));
#pragma unroll
          for (int j = 0; j < 4; ++j) ch.v[h][4 * k + j] = w[j];
        }
        const __amdgpu_buffer_rsrc_t rks = tile(ksc, t * BS * 4, BS * 4);
        const __amdgpu_buffer_rsrc_t rvs = tile(vsc, t * BS * 4, BS * 4);
        ch.ks[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, soff, row0[h] * 4, 0));
        ch.vs[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, soff, row0[h] * 4, 0));
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          ch.k[h][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, ks_row + 64 * j, POL));
        // V: tokens 4g .. 4g+3 of dims 32k + 2c and 32k + 2c + 1 (operands
        // 2k, 2k + 1), one 16-byte load per 32 dims
#pragma unroll
        for (int k = 0; k < NN / 2; ++k) {
          const u32x4 w = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, vs_row + 256 * k, POL));
          ch.v[h][2 * k] = u32x2{w.x, w.y};
          ch.v[h][2 * k + 1] = u32x2{w.z, w.w};
        }
      }
    }
  }
};

// INT4 chunk.  K: per sub-tile, lane l = 16 g + c holds row c, dims
// (D/4) g .. (D/4) g + D/4 - 1 (D/8 bytes, one load); operand j is the word
// of dims (D/4) g + 8 j .. + 7, its elements in the order of that word's
// low nibbles, then its high nibbles (dims +0, 2, 4, 6, 1, 3, 5, 7).
// V: the tile is [bs/4][D/2][4] bytes (token groups, dim pairs, tokens);
// per sub-tile the lane holds words m = 0 .. D/32 - 1: tokens 4g .. 4g+3 of
// dim pair (D/32) c + m (dims 2 ((D/32) c + m) and that + 1), one load;
// word m's low nibbles feed the rows of output tile 2 m, its high nibbles
// those of tile 2 m + 1.
template <int D>
struct ChunkI4 {
  typename std::conditional<D == 128, u32x4, u32x2>::type k[2];
  uint32_t v[2][D / 32];
  f32x4 ks[2], vs[2];
};

template <int D, int BS, int POL = 0>
struct ChunkLoaderI4 {
  static constexpr uint32_t kTileBytes = BS * D / 2;
  const char* kc;
  const char* vc;
  const char* ksc;
  const char* vsc;
  int Hkv, kvh;
  uint32_t koff, voff, soff;

  __device__ __forceinline__ ChunkLoaderI4(const DecodeParams& p, int kvh_, int c, int g)
      : kc(static_cast<const char*>(p.k_cache)), vc(static_cast<const char*>(p.v_cache)),
        ksc(reinterpret_cast<const char*>(p.k_scale)), vsc(reinterpret_cast<const char*>(p.v_scale)),
        Hkv(p.num_kv_heads), kvh(kvh_) {
    koff = static_cast<uint32_t>(c) * (D / 2) + (D / 8) * g;
    // V: token group g, dim pairs (D/32) c .. (D/32) c + D/32 - 1
    voff = (static_cast<uint32_t>(g) * (D / 2) + (D / 32) * c) * 4u;
    soff = 4u * g * 4u;
  }

  __device__ __forceinline__ void load(ChunkI4<D>& ch, const int blk[2], const int row0[2]) const {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t t = static_cast<size_t>(blk[h]) * Hkv + kvh;
      const __amdgpu_buffer_rsrc_t rk = ChunkLoader<true, D, BS>::tile(kc, t * kTileBytes, kTileBytes);
      const __amdgpu_buffer_rsrc_t rv = ChunkLoader<true, D, BS>::tile(vc, t * kTileBytes, kTileBytes);
      if constexpr (D == 128)
        ch.k[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, row0[h] * (D / 2), POL));
      else
        ch.k[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, koff, row0[h] * (D / 2), POL));
      // the sub-tile's token groups start at row0 * D/2 bytes
      if constexpr (D == 128) {
        const u32x4 w = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, row0[h] * (D / 2), POL));
#pragma unroll
        for (int m = 0; m < 4; ++m) ch.v[h][m] = w[m];
      } else {
        const u32x2 w = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff, row0[h] * (D / 2), POL));
        ch.v[h][0] = w.x;
        ch.v[h][1] = w.y;
      }
      const __amdgpu_buffer_rsrc_t rks = ChunkLoader<true, D, BS>::tile(ksc, t * BS * 4, BS * 4);
      const __amdgpu_buffer_rsrc_t rvs = ChunkLoader<true, D, BS>::tile(vsc, t * BS * 4, BS * 4);
      ch.ks[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, soff, row0[h] * 4, 0));
      ch.vs[h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, soff, row0[h] * 4, 0));
    }
  }
};

// One head's unnormalised output row (fp32, D dims in order) from the PV
// accumulators of a lane (c, g), whose V operands came from the loaders
// above: element i of output tile n is row 4g + i of that tile, whose dim
// follows the lane-to-dim pairing of the V loads (dims
//   bf16:        32k + 8g + 2i + o        for n = 2k + o,
//   byte codes:  64k + 16g + 4i + j       for n = 4k + j,
//   INT4:        8P g + 2P i + n          (P = D/32; n even: the low
//                                          nibble dims, odd: the high ones)
// so each lane writes runs of consecutive dims.
template <KvKind KV, int D>
__device__ __forceinline__ void store_partial_row(float* arow, const f32x4 (&acc)[D / 16], int g) {
  constexpr int NN = D / 16;
  if constexpr (KV == KvKind::I4) {
    constexpr int P = D / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 8 * P * g + 2 * P * i;
#pragma unroll
      for (int n = 0; n < NN; n += 4)
        *reinterpret_cast<f32x4*>(arow + d0 + n) = f32x4{acc[n][i], acc[n + 1][i], acc[n + 2][i], acc[n + 3][i]};
    }
  } else if constexpr (KV != KvKind::BF16) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int d0 = 64 * k + 16 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(arow + d0 + 4 * i) =
            f32x4{acc[4 * k][i], acc[4 * k + 1][i], acc[4 * k + 2][i], acc[4 * k + 3][i]};
    }
  } else {
#pragma unroll
    for (int k = 0; k < NN / 2; ++k) {
      const int d0 = 32 * k + 8 * g;
      const f32x4 e = acc[2 * k], o = acc[2 * k + 1];
      *reinterpret_cast<f32x4*>(arow + d0) = f32x4{e[0], o[0], e[1], o[1]};
      *reinterpret_cast<f32x4*>(arow + d0 + 4) = f32x4{e[2], o[2], e[3], o[3]};
    }
  }
}

}  // namespace pkv
