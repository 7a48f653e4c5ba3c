// Paged decode attention, bf16 query over a bf16 or int8 paged KV cache,
// on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed: for each sequence b and query head h, softmax(scale *
// K_b q) V_b over the L = context_lens[b] cached tokens, gathered through the
// block table ("LLM Engineering (5)" [ENG5], "Paged attention"; every decode
// step reads the whole KV cache: [ENG5] "Two phases with very different
// characteristics").  int8 caches hold codes with one fp32 scale per
// (token, kv-head) ([ENG5] "KV-cache quantization").
//
// Work decomposition.  One workgroup of kDecodeWaves waves owns one
// (sequence, kv-head, context partition of part_tokens tokens).  The G query
// heads of the kv-head share every K/V byte it loads: the tile feeds one
// matrix-core contraction whose N dimension is the head group.  The waves of
// the workgroup take 32-token chunks of the partition round-robin, each
// keeping its own online-softmax state; the states are merged through LDS at
// the end.  A sequence that fits one partition is finished here; longer ones
// leave (max, sum, unnormalised output) partials for the reduce kernel.
//
// Per 32-token chunk (two 16-token sub-tiles, from two blocks at bs=16 or
// one block at bs=32), one wave does:
//   S^T[16 tok x 16 heads] = K_sub[16 x D] . Q^T[D x 16]   D/32 MFMAs per sub-tile
//     A operand: lane l holds row (l % 16) of the K sub-tile, 8 dims; loaded
//     straight from HBM as 16 bytes (bf16) or 16 bytes = two operands (int8).
//     B operand: Q^T, built once per workgroup (heads >= G are zero).
//   online softmax on the 8 scores a lane holds (head l%16, tokens
//     4*(l/16)+i of each sub-tile), max across the 4 lane groups by shuffles.
//   O^T[D x 16 heads] += V^T[D x 32 tok] . P^T[32 tok x 16 heads]   D/16 MFMAs
//     A operand: V tiles are stored dim-major (element (r, d) at d*bs + r),
//     so the 4 tokens a lane needs per sub-tile are 8 contiguous bytes.
//     B operand: the lane's own 8 probabilities, split into a bf16 hi/lo
//     pair (two MFMAs) so the weights keep ~16 bits; no shuffle is needed
//     because the score layout already matches.
// The contraction index of each MFMA is a free pairing of (lane group,
// element) to (dim or token); A and B use the same pairing, so only the row
// / column / accumulator layouts of the instruction matter here.

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 load_u32x2(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ uint32_t load_u32(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ f32x4 load_f32x4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

// Two int8 codes (bytes 0 and 1 of w >> (16*half)) -> packed bf16 pair.
// |code| <= 128 has at most 8 significant bits, so the conversion is exact.
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int half) {
  const int32_t lo = static_cast<int32_t>(w << (24 - 16 * half)) >> 24;
  const int32_t hi = static_cast<int32_t>(w << (16 - 16 * half)) >> 24;
  const uint32_t flo = __float_as_uint(static_cast<float>(lo));
  const uint32_t fhi = __float_as_uint(static_cast<float>(hi));
  return (flo >> 16) | (fhi & 0xffff0000u);
}

// 16 int8 codes -> two bf16x8 operands (codes 0..7 and 8..15).
__device__ __forceinline__ void i8x16_to_bf16(u32x4 w, bf16x8& a, bf16x8& b) {
  u32x4 lo, hi;
  lo.x = i8pair_to_bf16x2(w.x, 0);
  lo.y = i8pair_to_bf16x2(w.x, 1);
  lo.z = i8pair_to_bf16x2(w.y, 0);
  lo.w = i8pair_to_bf16x2(w.y, 1);
  hi.x = i8pair_to_bf16x2(w.z, 0);
  hi.y = i8pair_to_bf16x2(w.z, 1);
  hi.z = i8pair_to_bf16x2(w.w, 0);
  hi.w = i8pair_to_bf16x2(w.w, 1);
  a = as_bf16x8(lo);
  b = as_bf16x8(hi);
}

// Zero the bf16 elements (pairs packed in w) whose token is >= t_end.
__device__ __forceinline__ uint32_t mask_pair(uint32_t w, int tok, int t_end) {
  const uint32_t lo = (tok < t_end) ? (w & 0xffffu) : 0u;
  const uint32_t hi = (tok + 1 < t_end) ? (w & 0xffff0000u) : 0u;
  return lo | hi;
}

template <bool kInt8, int D, int BS, int W>
__global__ __launch_bounds__(W * kWave) void decode_mfma_kernel(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(BS == 16 || BS == 32, "block_size");
  constexpr int NJ = D / 32;  // QK MFMAs per 16-token sub-tile
  constexpr int NN = D / 16;  // PV MFMAs per 32-token chunk

  __shared__ float red_acc[W > 1 ? W - 1 : 1][NN * 4][kWave];
  __shared__ float red_m[W][kWave];
  __shared__ float red_l[W][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c = lane & 15;  // head column
  const int g = lane >> 4;  // lane group

  const int Hkv = p.num_kv_heads;
  const int H = p.num_heads;
  const int G = H / Hkv;
  const int b = blockIdx.x / Hkv;
  const int kvh = blockIdx.x - b * Hkv;
  const int part = blockIdx.y;
  const int PT = p.part_tokens;

  const int L = p.context_lens[b];
  const int t_begin = part * PT;
  if (part != 0 && t_begin >= L) return;  // uniform across the workgroup
  const int h0 = kvh * G;
  uint16_t* out = static_cast<uint16_t*>(p.out);

  if (L <= 0) {  // empty context: zero output
    for (int i = threadIdx.x; i < G * D; i += W * kWave)
      out[(static_cast<size_t>(b) * H + h0) * D + i] = 0;
    return;
  }
  const int t_end = min(L, t_begin + PT);
  const bool single = L <= PT;

  // Q^T operand (B of the score MFMA): lane (c, g), MFMA j, 8 dims.
  bf16x8 qf[NJ];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(b) * H + h0 + c) * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d0 = kInt8 ? (64 * (j >> 1) + 16 * g + 8 * (j & 1)) : (32 * j + 8 * g);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < G) v = load_u32x4(qrow + d0);
      qf[j] = as_bf16x8(v);
    }
  }

  // Physical block ids of the partition: lane i holds entry i.
  const int nblk = (t_end - t_begin + BS - 1) / BS;
  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq + t_begin / BS;
  const int my_blk = (lane < nblk) ? bt[lane] : 0;

  using KT = typename std::conditional<kInt8, int8_t, uint16_t>::type;
  const KT* kc = static_cast<const KT*>(p.k_cache);
  const KT* vc = static_cast<const KT*>(p.v_cache);
  const size_t tile = static_cast<size_t>(BS) * D;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[NN];
#pragma unroll
  for (int n = 0; n < NN; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (t_end - t_begin + 31) / 32;
  for (int ch = wave; ch < nchunks; ch += W) {
    const int t0 = t_begin + ch * 32;
    const bool h1 = (t0 + 16) < t_end;
    int blk0, blk1, row0, row1;
    if (BS == 16) {
      const int lb = (t0 - t_begin) >> 4;
      blk0 = __builtin_amdgcn_readlane(my_blk, lb);
      blk1 = h1 ? __builtin_amdgcn_readlane(my_blk, lb + 1) : blk0;
      row0 = 0;
      row1 = 0;
    } else {
      const int lb = (t0 - t_begin) >> 5;
      blk0 = __builtin_amdgcn_readlane(my_blk, lb);
      blk1 = blk0;
      row0 = 0;
      row1 = 16;
    }
    const size_t tb0 = (static_cast<size_t>(blk0) * Hkv + kvh) * tile;
    const size_t tb1 = (static_cast<size_t>(blk1) * Hkv + kvh) * tile;

    // ---- K sub-tiles -> scores
    bf16x8 ka0[NJ], ka1[NJ];
    {
      const KT* k0 = kc + tb0 + static_cast<size_t>(row0 + c) * D;
      const KT* k1 = kc + tb1 + static_cast<size_t>(row1 + c) * D;
      if constexpr (kInt8) {
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) {
          i8x16_to_bf16(load_u32x4(k0 + 64 * jj + 16 * g), ka0[2 * jj], ka0[2 * jj + 1]);
          u32x4 w1 = {0u, 0u, 0u, 0u};
          if (h1) w1 = load_u32x4(k1 + 64 * jj + 16 * g);
          i8x16_to_bf16(w1, ka1[2 * jj], ka1[2 * jj + 1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          ka0[j] = as_bf16x8(load_u32x4(k0 + 32 * j + 8 * g));
          u32x4 w1 = {0u, 0u, 0u, 0u};
          if (h1) w1 = load_u32x4(k1 + 32 * j + 8 * g);
          ka1[j] = as_bf16x8(w1);
        }
      }
    }
    // ---- V sub-tiles (dim-major): lane needs dims 16n + c, tokens 4g..4g+3
    uint32_t va0[NN][2], va1[NN][2];
    {
      const KT* v0 = vc + tb0 + static_cast<size_t>(c) * BS + row0 + 4 * g;
      const KT* v1 = vc + tb1 + static_cast<size_t>(c) * BS + row1 + 4 * g;
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        if constexpr (kInt8) {
          const uint32_t w0 = load_u32(v0 + 16 * n * BS);
          const uint32_t w1 = h1 ? load_u32(v1 + 16 * n * BS) : 0u;
          va0[n][0] = i8pair_to_bf16x2(w0, 0);
          va0[n][1] = i8pair_to_bf16x2(w0, 1);
          va1[n][0] = i8pair_to_bf16x2(w1, 0);
          va1[n][1] = i8pair_to_bf16x2(w1, 1);
        } else {
          const u32x2 w0 = load_u32x2(v0 + 16 * n * BS);
          u32x2 w1 = {0u, 0u};
          if (h1) w1 = load_u32x2(v1 + 16 * n * BS);
          va0[n][0] = w0.x;
          va0[n][1] = w0.y;
          va1[n][0] = w1.x;
          va1[n][1] = w1.y;
        }
      }
    }
    f32x4 ks0 = {1.f, 1.f, 1.f, 1.f}, ks1 = ks0, vs0 = ks0, vs1 = ks0;
    if constexpr (kInt8) {
      const size_t sb0 = (static_cast<size_t>(blk0) * Hkv + kvh) * BS + row0 + 4 * g;
      const size_t sb1 = (static_cast<size_t>(blk1) * Hkv + kvh) * BS + row1 + 4 * g;
      ks0 = load_f32x4(p.k_scale + sb0);
      vs0 = load_f32x4(p.v_scale + sb0);
      if (h1) {
        ks1 = load_f32x4(p.k_scale + sb1);
        vs1 = load_f32x4(p.v_scale + sb1);
      }
    }

    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[j], qf[j], s0, 0, 0, 0);
    if (h1) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[j], qf[j], s1, 0, 0, 0);
    }

    // ---- online softmax (log2 domain); lane = head c, tokens 4g+i (+16)
    const bool tail = (t0 + 32) > t_end;
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = s0[i] * ks0[i] * p.scale_log2;
      sc[4 + i] = s1[i] * ks1[i] * p.scale_log2;
    }
    if (tail) {  // select, never multiply: masked rows may hold NaN
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (t0 + 4 * g + i >= t_end) {
          sc[i] = -INFINITY;
          vs0[i] = 0.f;
        }
        if (t0 + 16 + 4 * g + i >= t_end) {
          sc[4 + i] = -INFINITY;
          vs1[i] = 0.f;
        }
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[n] *= alpha;
      m_run = m_new;
    }
    // P^T operand as a bf16 pair hi + lo (hi = bf16(p), lo = bf16(p - hi)):
    // two contractions give the weights to ~2^-16 relative instead of 2^-9.
    uint32_t ph[4], pl[4];
    {
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(sc[i] - m_run);
#pragma unroll
      for (int i = 0; i < 8; ++i) l_run += pr[i];
      if constexpr (kInt8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] *= vs0[i];
          pr[4 + i] *= vs1[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
        pl[i] = pack_bf16x2(pr[2 * i] - bf16_lo(ph[i]), pr[2 * i + 1] - bf16_hi(ph[i]));
      }
    }
    const bf16x8 pfh = as_bf16x8(u32x4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 pfl = as_bf16x8(u32x4{pl[0], pl[1], pl[2], pl[3]});

    if (tail) {  // masked tokens must contribute exact zeros, even over NaN
      const int ta = t0 + 4 * g;
      const int tb = t0 + 16 + 4 * g;
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        va0[n][0] = mask_pair(va0[n][0], ta, t_end);
        va0[n][1] = mask_pair(va0[n][1], ta + 2, t_end);
        va1[n][0] = mask_pair(va1[n][0], tb, t_end);
        va1[n][1] = mask_pair(va1[n][1], tb + 2, t_end);
      }
    }
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      const bf16x8 va = as_bf16x8(u32x4{va0[n][0], va0[n][1], va1[n][0], va1[n][1]});
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfh, acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfl, acc[n], 0, 0, 0);
    }
  }

  // per-head sum over the 4 lane groups (each holds different tokens)
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  float M = m_run, Lsum = l_run;
  if constexpr (W > 1) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = l_run;
    if (wave > 0) {
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_acc[wave - 1][4 * n + i][lane] = acc[n][i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, red_m[w][lane]);
    const float f0 = fast_exp2(m_run - M);  // wave 0 always saw a chunk: M finite
    Lsum = l_run * f0;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[n] *= f0;
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const float fw = fast_exp2(red_m[w][lane] - M);  // -inf (idle wave) -> 0
      Lsum += fw * red_l[w][lane];
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[n][i] += fw * red_acc[w - 1][4 * n + i][lane];
    }
  }

  if (c >= G) return;
  const int h = h0 + c;
  const size_t bh = static_cast<size_t>(b) * H + h;
  if (single) {
    uint16_t* orow = out + bh * D;
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      u32x2 w;
      w.x = pack_bf16x2(acc[n][0] / Lsum, acc[n][1] / Lsum);
      w.y = pack_bf16x2(acc[n][2] / Lsum, acc[n][3] / Lsum);
      *reinterpret_cast<u32x2*>(orow + 16 * n + 4 * g) = w;
    }
  } else {
    const size_t slot = bh * p.num_parts + part;
    float* arow = p.ws_acc + slot * D;
#pragma unroll
    for (int n = 0; n < NN; ++n) *reinterpret_cast<f32x4*>(arow + 16 * n + 4 * g) = acc[n];
    if (g == 0) {
      p.ws_m[slot] = M;
      p.ws_l[slot] = Lsum;
    }
  }
}

template <bool kInt8, int D, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.num_seqs * p.num_kv_heads),
                  static_cast<unsigned>(p.num_parts));
  hipLaunchKernelGGL((decode_mfma_kernel<kInt8, D, BS, kDecodeWaves>), grid,
                     dim3(kDecodeWaves * kWave), 0, s, p);
  return hipGetLastError();
}

template <bool kInt8>
hipError_t launch_kv(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128)
    return p.block_size == 16 ? launch_t<kInt8, 128, 16>(p, s) : launch_t<kInt8, 128, 32>(p, s);
  return p.block_size == 16 ? launch_t<kInt8, 64, 16>(p, s) : launch_t<kInt8, 64, 32>(p, s);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, KvKind kv, hipStream_t s) {
  return kv == KvKind::I8 ? launch_kv<true>(p, s) : launch_kv<false>(p, s);
}

}  // namespace pkv
