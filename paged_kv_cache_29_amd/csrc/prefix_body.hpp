// Shared-prefix ("cascade") decode, the workgroup body that attends the
// tokens a group of sequences shares through the same physical blocks once
// for the whole group (also the multi-query kernel's).
//
// Requests with a common prefix (a system prompt, few-shot examples, tool
// definitions) hold the same physical blocks in their block tables ("LLM
// Engineering (5)", "Paged attention": prefix sharing is what prompt caching
// rests on; "SGLang and RadixAttention": the longest shared prefix is
// reused and only the suffix is computed per request).  Plain decode reads
// those blocks once per sequence.  Here each K/V chunk of the shared blocks
// is read once per workgroup and contracted against the queries of many
// sequences at once: the matrix-core N dimension holds (sequence, head)
// pairs of the group instead of one sequence's heads.
//
// Each workgroup owns (group, kv-head, 64 NT queries, partition of
// prefix_part_tokens shared tokens) and leaves, per query, the partial (max,
// sum, unnormalised output) of its partition in workspace slot `partition`;
// the reduce kernel merges them with the partials of each sequence's own
// tokens by the same exact combine as split-context decode.  Query column q
// of the group is sequence group_start[g] + q / G, head kv_head * G + q % G.
// The kv-head index varies fastest in the grid, so with 8 kv-heads each
// XCD's L2 serves one kv-head's shared blocks.
//
// Work split: every wave owns 16 NT queries (NT = 2, or 1 when the unit's
// columns fit 64: prefix_tiles_for) and walks every 32-token chunk of the
// partition.  A chunk is staged once in LDS: its four pieces (K and V of
// the two 16-token sub-tiles, plus the scales of coded caches) are copied
// by the four waves, one piece each, straight from global memory into LDS
// (global_load_lds, 16 bytes per lane, no registers on the way), into a
// ring of three stages: a chunk's copies are issued two chunks before it is
// read, so each wave waits for its own copies of the current chunk only
// (an explicit vmcnt count; the stages are separate LDS arrays, which lets
// the compiler see that reading one does not wait on the copies into the
// others) and one barrier per chunk publishes all four pieces.  Each wave
// then reads its matrix-core operands from LDS in the partition kernel's
// layouts (decode_tile.hpp) and, for each of its query tiles t,
//   S^T[16 tok x 16 q] = K_sub . Q_t^T, online softmax per query, and
//   O_t^T += V^T . P_t^T (P as a bf16 hi/lo pair),
// sharing the chunk's K and V operands (and code widening) between tiles.
// LDS layout per stage: a V sub-tile is the cache's bytes as they are
// (groups of 4 tokens, dim-major inside a group), read at the partition
// kernel's offsets (16 consecutive lanes read 256 consecutive bytes); a K
// sub-tile holds the cache's token rows with the 16-byte units of row r
// permuted (unit u stored at position u ^ f(r)), so that the 16 rows a wave
// reads together fall in distinct banks; the copy lanes pick their source
// units to match, since a copy lane's LDS destination is fixed.

#pragma once

#include "decode_tile.hpp"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {


// LDS stage of one 32-token chunk: pieces K0, K1, V0, V1 (the K and V
// bytes of the two 16-token sub-tiles, SUB bytes each), then the coded
// caches' scales (64 bytes per piece: k for the K pieces, v for the V ones).
template <KvKind KV, int D>
struct PrefixLds {
  static constexpr bool kCoded = KV != KvKind::BF16;
  static constexpr int RB = KV == KvKind::I4 ? D / 2 : D * (kCoded ? 1 : 2);  // bytes of a K token row
  static constexpr int SUB = 16 * RB;        // one sub-tile of K or V
  static constexpr int RU = RB / 16;         // 16-byte units per K row (2 .. 16)
  // K row r's units are permuted by f(r) = (r >> SH) mod RU: over 16 rows the
  // same unit lands on 16 different 16-byte bank groups of a 256-byte span
  static constexpr int SH = RU >= 16 ? 0 : RU == 8 ? 1 : RU == 4 ? 2 : 3;
  static constexpr int SC = kCoded ? 4 * 64 : 0;
  static constexpr int STAGE = 4 * SUB + SC;
  static constexpr int COPIES = (SUB + 16 * kWave - 1) / (16 * kWave);  // 1 KB copies per piece
  static constexpr int PER_CHUNK = COPIES + (kCoded ? 1 : 0);         // copy instructions per wave
  static_assert(RU >= 2 && RU <= 16 && SUB % 16 == 0, "K rows of whole 16-byte units");
};

// s_waitcnt with vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l
// reads src (its own address) and writes lds_dst + 16 l (lds_dst uniform).
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_dst) {
  using global_ptr = __attribute__((address_space(1))) const void*;
  using lds_ptr = __attribute__((address_space(3))) void*;
  __builtin_amdgcn_global_load_lds((global_ptr)src, (lds_ptr)lds_dst, 16, 0, 0);
}

// The ring's barrier: this wave's LDS reads are complete (lgkmcnt(0)), then
// the workgroup barrier, then an acquire fence that keeps later LDS reads
// after it.  (A release fence would also wait for every copy in flight.)
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Waves per SIMD: two tiles' states per wave take two waves' registers;
// one tile's (at most 173 VGPRs) fit three, which hide more of the chunk
// loop's LDS and barrier latency (70B GQA, 8-token verification per call:
// 545 us at two waves, 470 us at three; 667 us with two tiles per wave).
template <int NT>
constexpr int kPrefixWavesPerSimd = NT == 1 ? 3 : 2;

// KV: BF16, or codes with per-token scales (I8, FP8: bytes; I4: nibbles,
// with the partition kernel's INT4 operands and offsets).  kMQ: the
// multi-query form (one sequence's new tokens x heads as the columns, its
// whole context partitioned, each column masked causally at its position).
// (bx, by, bz): (group or sequence * Hkv + kv-head, query tile, partition),
// the block coordinates of the prefix kernel's grid.
template <KvKind KV, int D, int BS, int NT, bool kMQ>
__device__ __forceinline__ void prefix_body(const DecodeParams& p, int bx, int by, int bz) {
  constexpr bool kInt8 = KV != KvKind::BF16;  // codes (int8, FP8 E4M3 / E5M2, INT4) with scales
  constexpr bool kI4 = KV == KvKind::I4;
  using ChunkT = typename std::conditional<kI4, ChunkI4<D>, Chunk<kInt8, D>>::type;
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(BS == 16 || BS == 32, "block_size");
  static_assert(kDecodeWaves == 4, "one chunk piece per wave");
  constexpr int W = kDecodeWaves;
  constexpr int NJ = D / 32;
  constexpr int NN = D / 16;
  constexpr int QW = 16 * NT;  // queries per wave
  using L = PrefixLds<KV, D>;

  // the three stages of the chunk ring (separate arrays: see above)
  __shared__ __attribute__((aligned(16))) char stage0[L::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[L::STAGE];
  __shared__ __attribute__((aligned(16))) char stage2[L::STAGE];
  __shared__ int blk_ids[kMaxPartBlocks];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane & 15;
  const int g = lane >> 4;

  const int Hkv = p.num_kv_heads;
  const int H = p.num_heads;
  const int G = H / Hkv;
  const int kvh = bx % Hkv;
  const int grp = bx / Hkv;
  const int qwg = by * (W * QW);
  const int part = bz;

  // cascade: group grp's members x heads over its shared span; multi-query:
  // sequence grp's new tokens x heads over its whole context
  const int gs = kMQ ? grp : p.group_start[grp];             // whose block table
  const int qrow0 = kMQ ? p.query_start[grp] : 0;             // first query row (multi-query)
  const int nnew = kMQ ? p.query_start[grp + 1] - qrow0 : 0;
  const int nq = kMQ ? nnew * G : (p.group_start[grp + 1] - gs) * G;
  if (qwg >= nq) return;  // uniform across the workgroup
  const int S = kMQ ? p.context_lens[grp] : group_shared_tokens(p, grp);
  const int PTp = kMQ ? p.part_tokens : p.prefix_part_tokens;
  const int t_begin = part * PTp;
  if (t_begin >= S) return;  // uniform across the workgroup
  const int t_end = min(S, t_begin + PTp);  // block-aligned in cascade mode
  const int q0 = qwg + wave * QW;  // this wave's first query
  // multi-query: the last token column r may see (its position), per tile
  int lim[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) lim[t] = S - nnew + (q0 + 16 * t + c) / G;

  // Q^T operands: tile t, lane (c, g), MFMA j: 8 dims from q_dim(j)
  auto q_dim = [&](int j) {
    return kI4 ? ((D / 4) * g + 8 * j) : (kInt8 ? (64 * (j >> 1) + 16 * g + 8 * (j & 1)) : (32 * j + 8 * g));
  };
  bf16x8 qf[NT][NJ];
  float k_off[NT];  // INT4: 136 * sum_d q_d of column c
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = q0 + 16 * t + c;
    const size_t qr = kMQ ? static_cast<size_t>(qrow0 + r / G) : static_cast<size_t>(gs + r / G);
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (qr * H + kvh * G + r % G) * D;
    k_off[t] = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nq) v = load_u32x4(qrow + q_dim(j));
      if constexpr (kI4) {
        // element order of the INT4 K operand: dims +0, 2, 4, 6, 1, 3, 5, 7
        v = u32x4{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                  __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
#pragma unroll
        for (int i = 0; i < 4; ++i) k_off[t] += bf16_lo(v[i]) + bf16_hi(v[i]);
      }
      qf[t][j] = as_bf16x8(v);
    }
    if constexpr (kI4) k_off[t] = kInt4Offset * groups_sum(k_off[t]);
  }

  // block ids of the span (the group's first sequence's table, or the
  // sequence's own), once per workgroup
  const int nblk = (t_end - t_begin + BS - 1) / BS;
  {
    const int32_t* bt = p.block_tables + static_cast<size_t>(gs) * p.max_blocks_per_seq + t_begin / BS;
    for (int i = threadIdx.x; i < nblk; i += W * kWave) blk_ids[i] = bt[i];  // nblk <= kMaxPartBlocks
  }
  __syncthreads();

  // Blocks and first rows of chunk ch's two sub-tiles (uniform).  Past the
  // end of the span the second sub-tile repeats the first: valid memory,
  // masked.
  auto chunk_blocks = [&](int ch, int blk[2], int row0[2]) {
    const int t0 = t_begin + ch * 32;
    if (BS == 16) {
      blk[0] = __builtin_amdgcn_readfirstlane(blk_ids[2 * ch]);
      blk[1] = (t0 + 16 < t_end) ? __builtin_amdgcn_readfirstlane(blk_ids[2 * ch + 1]) : blk[0];
      row0[0] = row0[1] = 0;
    } else {
      blk[0] = blk[1] = __builtin_amdgcn_readfirstlane(blk_ids[ch]);
      row0[0] = 0;
      row0[1] = 16;
    }
  };

  // ---- staging: wave w copies piece w of a chunk (0: K sub-tile 0, 1: K
  // sub-tile 1, 2: V sub-tile 0, 3: V sub-tile 1; coded caches also that
  // piece's 16 scales, k for K pieces and v for V pieces) into a stage
  const int ph = wave & 1;
  const bool pv = wave >= 2;
  auto copy_chunk = [&](char* stage, int ch) {
    int blk[2], row0[2];
    chunk_blocks(ch, blk, row0);
    const size_t tile = static_cast<size_t>(blk[ph]) * Hkv + kvh;
    // K: 16 token rows; V: the sub-tile's 4 token groups (row0 is a multiple
    // of 4): both SUB contiguous bytes from row0 * RB
    const char* src = static_cast<const char*>(pv ? p.v_cache : p.k_cache) + tile * (BS * L::RB) +
                      static_cast<size_t>(row0[ph]) * L::RB;
    char* dst = stage + wave * L::SUB;
#pragma unroll
    for (int i = 0; i < L::COPIES; ++i) {
      const int q = i * kWave + lane;  // 16-byte unit of the piece this lane fills
      if (q * 16 >= L::SUB) break;     // INT4 at D = 64: half the lanes
      int off = q * 16;
      if (!pv) {  // K: position q % RU of row r holds unit (q % RU) ^ f(r)
        const int r = q / L::RU;
        off = r * L::RB + (((q % L::RU) ^ (r >> L::SH)) & (L::RU - 1)) * 16;
      }
      copy16_to_lds(src + off, dst + i * (16 * kWave));
    }
    if constexpr (kInt8) {
      if (lane < 4) {
        const float* sc = (pv ? p.v_scale : p.k_scale) + tile * BS + row0[ph] + 4 * lane;
        copy16_to_lds(sc, stage + 4 * L::SUB + wave * 64);
      }
    }
  };
  // this lane's operands of a staged chunk, in the partition kernel's layouts
  auto lds_chunk = [&](const char* stage, ChunkT& cw) {
    const int kf = (c >> L::SH) & (L::RU - 1);  // the unit permutation of K row c
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const char* kr = stage + h * L::SUB + c * L::RB;
      const char* vt = stage + (2 + h) * L::SUB;
      if constexpr (kI4) {
        // K: this lane's D/4 dims of row c (unit g, or half unit at D = 64);
        // V: tokens 4g .. 4g+3 of dim pairs (D/32) c .. + D/32 - 1
        if constexpr (D == 128) {
          cw.k[h] = *reinterpret_cast<const u32x4*>(kr + ((g ^ kf) & 3) * 16);
          const u32x4 w = *reinterpret_cast<const u32x4*>(vt + g * (D / 2) * 4 + 16 * c);
#pragma unroll
          for (int m = 0; m < 4; ++m) cw.v[h][m] = w[m];
        } else {
          cw.k[h] = *reinterpret_cast<const u32x2*>(kr + (((g >> 1) ^ kf) & 1) * 16 + (g & 1) * 8);
          const u32x2 w = *reinterpret_cast<const u32x2*>(vt + g * (D / 2) * 4 + 8 * c);
          cw.v[h][0] = w.x;
          cw.v[h][1] = w.y;
        }
      } else if constexpr (kInt8) {
        // K: units 4jj + g of row c; V: tokens 4g .. 4g+3 of dims 64k + 4c + j
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj)
          cw.k[h][jj] = *reinterpret_cast<const u32x4*>(kr + (((4 * jj + g) ^ kf) & (L::RU - 1)) * 16);
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(vt + g * D * 4 + 256 * k + 16 * c);
#pragma unroll
          for (int j = 0; j < 4; ++j) cw.v[h][4 * k + j] = w[j];
        }
      } else {
        // K: units 4j + g of row c; V: tokens 4g .. 4g+3 of dims 32k + 2c, + 1
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          cw.k[h][j] = *reinterpret_cast<const u32x4*>(kr + (((4 * j + g) ^ kf) & (L::RU - 1)) * 16);
#pragma unroll
        for (int k = 0; k < NN / 2; ++k) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(vt + g * D * 8 + 256 * k + 16 * c);
          cw.v[h][2 * k] = u32x2{w.x, w.y};
          cw.v[h][2 * k + 1] = u32x2{w.z, w.w};
        }
      }
      if constexpr (kInt8) {
        const char* sc = stage + 4 * L::SUB;
        cw.ks[h] = *reinterpret_cast<const f32x4*>(sc + h * 64 + 16 * g);
        cw.vs[h] = *reinterpret_cast<const f32x4*>(sc + (2 + h) * 64 + 16 * g);
      }
    }
  };

  float m_run[NT], l_run[NT];
  float pv_run[NT];  // INT4: sum_t p_t v_scale_t (this lane's tokens)
  f32x4 acc[NT][NN];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
    pv_run[t] = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto consume = [&](const ChunkT& cw, int ch) {
    const int t0 = t_begin + ch * 32;
    const bool tail = (t0 + 32) > t_end;  // only a lone last block at bs = 16
    // V^T operands of the chunk, shared by the query tiles (INT4: operand
    // 2m holds the even dims of the lane's dim pairs, 2m + 1 the odd ones)
    u32x4 vw[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      if constexpr (kI4) {
        uint32_t lo0, hi0, lo1, hi1;
        int4_nibbles(cw.v[0][n / 2], lo0, hi0);
        int4_nibbles(cw.v[1][n / 2], lo1, hi1);
        const u32x2 a0 = nib4_to_bf16((n & 1) ? hi0 : lo0), a1 = nib4_to_bf16((n & 1) ? hi1 : lo1);
        vw[n] = u32x4{a0.x, a0.y, a1.x, a1.y};
      } else if constexpr (kInt8) {
        vw[n] = u32x4{codes_to_bf16x2<KV, 0>(cw.v[0][n]), codes_to_bf16x2<KV, 1>(cw.v[0][n]),
                      codes_to_bf16x2<KV, 0>(cw.v[1][n]), codes_to_bf16x2<KV, 1>(cw.v[1][n])};
      } else {
        vw[n] = u32x4{cw.v[0][n].x, cw.v[0][n].y, cw.v[1][n].x, cw.v[1][n].y};
      }
      if (tail) {  // masked tokens contribute exact zeros
        const int ta = t0 + 4 * g;
        vw[n].x = mask_pair(vw[n].x, ta, t_end);
        vw[n].y = mask_pair(vw[n].y, ta + 2, t_end);
        vw[n].z = mask_pair(vw[n].z, ta + 16, t_end);
        vw[n].w = mask_pair(vw[n].w, ta + 18, t_end);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // every column of the tile is padding (uniform): skip its arithmetic
      // (not for int8 at D = 128 with two tiles per wave, whose registers
      // are too tight for the branch)
      if (!(KV == KvKind::I8 && D == 128 && NT == 2) && q0 + 16 * t >= nq) continue;
      f32x4 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kI4) {
          s[h] = f32x4{-k_off[t], -k_off[t], -k_off[t], -k_off[t]};
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            uint32_t lo, hi;
            int4_nibbles(cw.k[h][j], lo, hi);
            const u32x2 a = nib4_to_bf16(lo), bq = nib4_to_bf16(hi);
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{a.x, a.y, bq.x, bq.y}), qf[t][j], s[h], 0, 0, 0);
          }
        } else if constexpr (kInt8) {
#pragma unroll
          for (int jj = 0; jj < NJ / 2; ++jj) {
            const u32x4 w = cw.k[h][jj];
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes8_to_bf16<KV>(w.x, w.y), qf[t][2 * jj], s[h], 0, 0, 0);
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes8_to_bf16<KV>(w.z, w.w), qf[t][2 * jj + 1], s[h], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cw.k[h][j]), qf[t][j], s[h], 0, 0, 0);
        }
      }
      // lane (c, g) holds the scores of tokens 16h + 4g + i for query c
      float sc[8];
      f32x4 vs[2] = {f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[h][i];
          if constexpr (kInt8) {
            x *= cw.ks[h][i];
            vs[h][i] = cw.vs[h][i];
          }
          sc[4 * h + i] = x * p.scale_log2;
        }
      }
      if (tail) {  // select, never multiply: masked rows may hold NaN
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) >= t_end) {
            sc[e] = -INFINITY;
            vs[e >> 2][e & 3] = 0.f;
          }
        }
      }
      if constexpr (kMQ) {  // causal: column c sees tokens up to lim[t]
        if (t0 + 31 > lim[t]) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) > lim[t]) sc[e] = -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = groups_max(mx);
      const float m_new = fmaxf(m_run[t], mx);
      if (__any(m_new > m_run[t])) {
        float alpha = fast_exp2(m_run[t] - m_new);
        // multi-query: a column that has seen nothing yet (-inf - -inf)
        if constexpr (kMQ) alpha = (m_new == -INFINITY) ? 1.f : alpha;
        l_run[t] *= alpha;
        if constexpr (kI4) pv_run[t] *= alpha;
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[t][n] *= alpha;
        m_run[t] = m_new;
      }
      uint32_t ph[4], pl[4];
      {
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(sc[e] - m_run[t]);
        if constexpr (kMQ) {  // a column can be masked throughout (m_run = -inf): exact zeros
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] = (sc[e] == -INFINITY) ? 0.f : pr[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run[t] += pr[e];
        if constexpr (kInt8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] *= vs[e >> 2][e & 3];
        }
        if constexpr (kI4) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pv_run[t] += pr[e];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
          pl[i] = pack_bf16x2(pr[2 * i] - bf16_lo(ph[i]), pr[2 * i + 1] - bf16_hi(ph[i]));
        }
      }
      const bf16x8 pfh = as_bf16x8(u32x4{ph[0], ph[1], ph[2], ph[3]});
      const bf16x8 pfl = as_bf16x8(u32x4{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const bf16x8 va = as_bf16x8(vw[n]);
        acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfh, acc[t][n], 0, 0, 0);
        acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfl, acc[t][n], 0, 0, 0);
      }
    }
  };


  // ---- every chunk of the partition through the ring: at chunk ch, wait
  // for this wave's copies of ch (those of ch + 1 may still be in flight),
  // then a barrier (every piece of ch has landed, and every wave is done
  // with the stage of ch - 1), then the copies of ch + 2 into that stage,
  // then the arithmetic on ch.  One body serves every chunk: its masking
  // (past the span's end or, multi-query, past a column's position) sits
  // behind uniform branches; a second, unmasked copy per stage would not fit
  // the registers.  The counts are uniform, so every wave runs the same
  // barriers.
  const int nchunks = (t_end - t_begin + 31) / 32;
  auto step = [&](int ch, const char* cur, char* ahead) {
    if (ch + 1 < nchunks)
      wait_vmcnt<L::PER_CHUNK>();
    else
      wait_vmcnt<0>();
    ring_barrier();
    if (ch + 2 < nchunks) copy_chunk(ahead, ch + 2);
    ChunkT cw;
    lds_chunk(cur, cw);
    consume(cw, ch);
  };
  copy_chunk(stage0, 0);
  if (nchunks > 1) copy_chunk(stage1, 1);
  for (int ch = 0; ch < nchunks; ch += 3) {
    step(ch, stage0, stage2);
    if (ch + 1 < nchunks) step(ch + 1, stage1, stage0);
    if (ch + 2 < nchunks) step(ch + 2, stage2, stage1);
  }

  // ---- this wave's partials
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float Lsum = groups_sum(l_run[t]);
    if constexpr (kI4) {  // remove the V offset of this wave's tokens
      const float v_off = kInt4Offset * groups_sum(pv_run[t]);
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[t][n] -= v_off;
    }
    const int r = q0 + 16 * t + c;
    if (r >= nq) continue;
    const size_t qr = kMQ ? static_cast<size_t>(qrow0 + r / G) : static_cast<size_t>(gs + r / G);
    const size_t bh = qr * H + kvh * G + r % G;
    const size_t slot = bh * p.num_parts + part;
    store_partial_row<KV, D>(p.ws_acc + slot * D, acc[t], g);
    if (g == 0) {
      p.ws_m[slot] = m_run[t];
      p.ws_l[slot] = Lsum;
    }
  }
}

}  // namespace
}  // namespace pkv
