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
// columns fit 64: prefix_tiles_for) and walks every
// 32-token chunk of the partition.  A chunk is staged once in LDS: its four
// pieces (K and V of the two 16-token sub-tiles, plus int8 scales) are
// loaded by the four waves, one piece each, while the previous chunk is
// being consumed (two LDS stages).  Each wave then reads its matrix-core
// operands from LDS in the partition kernel's layouts (decode_tile.hpp) and,
// for each of its query tiles t,
//   S^T[16 tok x 16 q] = K_sub . Q_t^T, online softmax per query, and
//   O_t^T += V^T . P_t^T (P as a bf16 hi/lo pair),
// sharing the chunk's K and V operands (and int8 widening) between tiles.
// LDS layout per stage: K sub-tiles as token rows padded by 16 bytes (the
// 16 rows a wave reads together fall in distinct banks); V sub-tiles
// dim-major, one row of 16 tokens per dim (INT4: per dim pair), gathered
// from the cache's groups of 4 tokens while staging; bf16 rows with their
// 8-byte token quads 2k and 2k + 1 swapped on every other group of 8 dims
// (same purpose).

#pragma once

#include "decode_tile.hpp"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {


// LDS stage of one 32-token chunk.  A token's K row is RB bytes (bf16: 2D,
// byte codes: D, INT4: D/2); V is stored as VR rows (dims, INT4: dim pairs)
// of one sub-tile's 16 tokens.
template <KvKind KV, int D, int BS, int NT>
struct PrefixLds {
  static constexpr int kElem = KV == KvKind::BF16 ? 2 : 1;
  static constexpr int RB = KV == KvKind::I4 ? D / 2 : D * kElem;
  static constexpr int VR = KV == KvKind::I4 ? D / 2 : D;
  static constexpr int KROW = RB + 16;                // padded K token row
  static constexpr int KSUB = 16 * KROW;              // one 16-token K sub-tile
  static constexpr int VROW = 16 * kElem;             // one V row's 16 tokens
  static constexpr int VSUB = VR * VROW;              // one 16-token V sub-tile
  static constexpr int SC = KV != KvKind::BF16 ? 4 * 64 : 0;  // k/v scales of both sub-tiles
  static constexpr int STAGE = 2 * KSUB + 2 * VSUB + SC;
  static constexpr int PIECE = 16 * RB;               // bytes of one K or V sub-tile
  // 16-byte loads per lane per piece (INT4 at D = 64: half the lanes load)
  static constexpr int UNITS = (PIECE + 16 * kWave - 1) / (16 * kWave);
};

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
  using L = PrefixLds<KV, D, BS, NT>;

  __shared__ __attribute__((aligned(16))) char lds[2][L::STAGE];
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

  // ---- staging: wave w moves piece w of a chunk (0: K sub-tile 0, 1: K
  // sub-tile 1, 2: V sub-tile 0, 3: V sub-tile 1; int8 also that piece's
  // 16 scales, k for K pieces and v for V pieces)
  const int ph = wave & 1;
  const bool pv = wave >= 2;
  u32x4 pu[L::UNITS];
  u32x4 psc = {0u, 0u, 0u, 0u};
  auto piece_load = [&](int ch) {
    int blk[2], row0[2];
    chunk_blocks(ch, blk, row0);
    const size_t tile = static_cast<size_t>(blk[ph]) * Hkv + kvh;
    const char* base = static_cast<const char*>(pv ? p.v_cache : p.k_cache) + tile * (BS * L::RB);
#pragma unroll
    for (int i = 0; i < L::UNITS; ++i) {
      const int u = i * kWave + lane;  // 16-byte unit of the piece
      if (u * 16 >= L::PIECE) break;   // INT4 at D = 64: half the lanes
      // K: 16 token rows; V: the sub-tile's 4 token groups (row0 is a
      // multiple of 4): both 16 * RB contiguous bytes from row0 * RB
      const size_t off = static_cast<size_t>(row0[ph]) * L::RB + u * 16;
      pu[i] = load_u32x4(base + off);
    }
    if (kInt8 && lane < 4) {
      const float* sc = pv ? p.v_scale : p.k_scale;
      psc = load_u32x4(sc + tile * BS + row0[ph] + 4 * lane);
    }
  };
  auto piece_store = [&](int st) {
    char* dst = lds[st];
#pragma unroll
    for (int i = 0; i < L::UNITS; ++i) {
      const int u = i * kWave + lane;
      if (u * 16 >= L::PIECE) break;
      if (!pv) {
        const int row = (u * 16) / L::RB;
        const int col = (u * 16) % L::RB;
        *reinterpret_cast<u32x4*>(dst + ph * L::KSUB + row * L::KROW + col) = pu[i];
      } else {
        // unit u of the cache's V sub-tile: token group u / (VR / 4) (4 tokens)
        // of rows 4 (u % (VR / 4)) .. + 3 (byte codes, INT4), or of dims
        // 2 (u % (D / 2)) and + 1 (bf16); each row's 4 tokens go to that
        // row of the dim-major stage
        const u32x4 w = pu[i];
        char* vt = dst + 2 * L::KSUB + ph * L::VSUB;
        if constexpr (kInt8) {
          const int gq = u / (L::VR / 4);
          const int r = 4 * (u % (L::VR / 4));
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(vt + (r + j) * L::VROW + 4 * gq) = w[j];
        } else {
          const int gq = u / (D / 2);
          const int d = 2 * (u % (D / 2));
          const int slot = 8 * (gq ^ ((d >> 3) & 1));  // d and d + 1 share the 8-dim group
          *reinterpret_cast<u32x2*>(vt + d * L::VROW + slot) = u32x2{w.x, w.y};
          *reinterpret_cast<u32x2*>(vt + (d + 1) * L::VROW + slot) = u32x2{w.z, w.w};
        }
      }
    }
    if (kInt8 && lane < 4)
      *reinterpret_cast<u32x4*>(dst + 2 * L::KSUB + 2 * L::VSUB + wave * 64 + lane * 16) = psc;
  };
  // this lane's operands of a staged chunk, in the partition kernel's layouts
  auto lds_chunk = [&](int st, ChunkT& cw) {
    const char* src = lds[st];
    if constexpr (kI4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // K: this lane's D/4 dims of row c; V: word m = tokens 4g .. 4g+3 of
        // dim pair 16m + c
        const char* kr = src + h * L::KSUB + c * L::KROW;
        if constexpr (D == 128)
          cw.k[h] = *reinterpret_cast<const u32x4*>(kr + 16 * g);
        else
          cw.k[h] = *reinterpret_cast<const u32x2*>(kr + 8 * g);
        const char* vr = src + 2 * L::KSUB + h * L::VSUB;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) cw.v[h][m] = *reinterpret_cast<const uint32_t*>(vr + (16 * m + c) * L::VROW + 4 * g);
        const char* sc = src + 2 * L::KSUB + 2 * L::VSUB;
        cw.ks[h] = *reinterpret_cast<const f32x4*>(sc + h * 64 + 16 * g);
        cw.vs[h] = *reinterpret_cast<const f32x4*>(sc + (2 + h) * 64 + 16 * g);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char* kr = src + h * L::KSUB + c * L::KROW;
        if constexpr (kInt8) {
#pragma unroll
          for (int jj = 0; jj < NJ / 2; ++jj) cw.k[h][jj] = *reinterpret_cast<const u32x4*>(kr + 16 * g + 64 * jj);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) cw.k[h][j] = *reinterpret_cast<const u32x4*>(kr + (32 * j + 8 * g) * 2);
        }
        const char* vr = src + 2 * L::KSUB + h * L::VSUB;
#pragma unroll
        for (int n = 0; n < NN; ++n) {
          if constexpr (kInt8) {
            cw.v[h][n] = *reinterpret_cast<const uint32_t*>(vr + (16 * n + c) * L::VROW + 4 * g);
          } else {
            const int gg = g ^ ((c >> 3) & 1);
            cw.v[h][n] = *reinterpret_cast<const u32x2*>(vr + (16 * n + c) * L::VROW + 8 * gg);
          }
        }
        if constexpr (kInt8) {
          const char* sc = src + 2 * L::KSUB + 2 * L::VSUB;
          cw.ks[h] = *reinterpret_cast<const f32x4*>(sc + h * 64 + 16 * g);
          cw.vs[h] = *reinterpret_cast<const f32x4*>(sc + (2 + h) * 64 + 16 * g);
        }
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

  // `masked` (compile time): the chunk may hold tokens past the end of the
  // span or, multi-query, past a column's position; clean chunks take the
  // instantiation without masking code (as a runtime branch the compiler
  // turns the masking into selects that every chunk executes).
  auto consume = [&](const ChunkT& cw, int ch, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int t0 = t_begin + ch * 32;
    const bool tail = kMasked && (t0 + 32) > t_end;  // only a lone last block at bs = 16
    // V^T operands of the chunk, shared by the query tiles (INT4: operand
    // 2m holds the even dims of dim pairs 16m + c, 2m + 1 the odd ones)
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
      if constexpr (kMQ && kMasked) {  // causal: column c sees tokens up to lim[t]
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


  // ---- every chunk of the partition, two LDS stages: the next chunk's
  // pieces are in flight while the current one is consumed
  // Clean chunks (inside the span and, multi-query, at or before the
  // workgroup's first column's position, hence every column's) first, then
  // the rest; the bound is uniform across the workgroup, so every wave runs
  // the same iterations between the barriers.
  const int nchunks = (t_end - t_begin + 31) / 32;
  const int clean_end = kMQ ? min(t_end, S - nnew + qwg / G + 1) : t_end;
  const int nclean = min(nchunks, max(0, (clean_end - t_begin) / 32));
  auto run = [&](int ch0, int ch1, auto masked) {
    for (int ch = ch0; ch < ch1; ++ch) {
      const bool more = ch + 1 < nchunks;
      if (more) piece_load(ch + 1);
      {
        ChunkT cw;
        lds_chunk(ch & 1, cw);
        consume(cw, ch, masked);
      }
      if (more) piece_store((ch + 1) & 1);
      __syncthreads();
    }
  };
  piece_load(0);
  piece_store(0);
  __syncthreads();
  run(0, nclean, std::false_type{});
  run(nclean, nchunks, std::true_type{});

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
    float* arow = p.ws_acc + slot * D;
    if constexpr (kI4) {  // lane holds dims 32m + 8g .. + 7: tiles 2m (even), 2m + 1 (odd)
#pragma unroll
      for (int m = 0; m < NN / 2; ++m) {
        const f32x4 e = acc[t][2 * m], o = acc[t][2 * m + 1];
        *reinterpret_cast<f32x4*>(arow + 32 * m + 8 * g) = f32x4{e[0], o[0], e[1], o[1]};
        *reinterpret_cast<f32x4*>(arow + 32 * m + 8 * g + 4) = f32x4{e[2], o[2], e[3], o[3]};
      }
    } else {
#pragma unroll
      for (int n = 0; n < NN; ++n) *reinterpret_cast<f32x4*>(arow + 16 * n + 4 * g) = acc[t][n];
    }
    if (g == 0) {
      p.ws_m[slot] = m_run[t];
      p.ws_l[slot] = Lsum;
    }
  }
}

}  // namespace
}  // namespace pkv
