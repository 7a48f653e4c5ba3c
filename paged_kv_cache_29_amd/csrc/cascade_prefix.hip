// Shared-prefix ("cascade") decode: the tokens a group of sequences shares
// through the same physical blocks are attended once for the whole group.
//
// Requests with a common prefix (a system prompt, few-shot examples, tool
// definitions) hold the same physical blocks in their block tables ("LLM
// Engineering (5)", "Paged attention": prefix sharing is what prompt caching
// rests on; "SGLang and RadixAttention": the longest shared prefix is
// reused and only the suffix is computed per request).  Plain decode reads
// those blocks once per sequence.  Here each K/V chunk of the shared blocks
// is loaded once per workgroup and contracted against the queries of
// several sequences at a time: the matrix-core N dimension holds
// (sequence, head) pairs of the group instead of one sequence's heads.
//
// Each workgroup owns (group, kv-head, tile of 16 * kPrefixTiles queries,
// partition of prefix_part_tokens shared tokens) and leaves, per query, the
// partial (max, sum, unnormalised output) of its partition in workspace
// slot `partition`; the reduce kernel merges them with the partials of each
// sequence's own tokens by the same exact combine as split-context decode.
// Query column q of the group is sequence group_start[g] + q / G, head
// kv_head * G + q % G.  The kv-head index varies fastest in the grid, so with
// 8 kv-heads each XCD's L2 serves one kv-head's shared blocks.
//
// Operand layouts are those of the partition kernel (decode_tile.hpp);
// per 32-token chunk one wave does, for each query tile t,
//   S^T[16 tok x 16 q] = K_sub . Q_t^T, online softmax per query, and
//   O_t^T += V^T . P_t^T (P as a bf16 hi/lo pair),
// with the chunk's K and V operands (and int8 widening) shared by the tiles.

#include "decode_tile.hpp"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

template <bool kInt8, int D, int BS, int W, int NT>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void cascade_prefix_kernel(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(BS == 16 || BS == 32, "block_size");
  constexpr int NJ = D / 32;
  constexpr int NN = D / 16;
  constexpr int QT = 16 * NT;

  __shared__ float red_acc[W - 1][NT][NN * 4][kWave];
  __shared__ float red_m[W][NT][kWave];
  __shared__ float red_l[W][NT][kWave];
  __shared__ int blk_ids[W][kMaxPartBlocks];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane & 15;
  const int g = lane >> 4;

  const int Hkv = p.num_kv_heads;
  const int H = p.num_heads;
  const int G = H / Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int grp = blockIdx.x / Hkv;
  const int q0 = blockIdx.y * QT;
  const int part = blockIdx.z;

  const int gs = p.group_start[grp];
  const int nq = (p.group_start[grp + 1] - gs) * G;
  if (q0 >= nq) return;  // uniform
  const int S = group_shared_tokens(p, grp);
  const int t_begin = part * p.prefix_part_tokens;
  if (t_begin >= S) return;  // uniform
  const int t_end = min(S, t_begin + p.prefix_part_tokens);  // block-aligned

  // Q^T operands: tile t, lane (c, g), MFMA j: 8 dims from q_dim(j)
  auto q_dim = [&](int j) { return kInt8 ? (64 * (j >> 1) + 16 * g + 8 * (j & 1)) : (32 * j + 8 * g); };
  bf16x8 qf[NT][NJ];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r = q0 + 16 * t + c;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           (static_cast<size_t>(gs + r / G) * H + kvh * G + r % G) * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nq) v = load_u32x4(qrow + q_dim(j));
      qf[t][j] = as_bf16x8(v);
    }
  }

  // the group's shared block ids (from its first sequence's table), staged
  // per wave in LDS as in the partition kernel
  const int nblk = (t_end - t_begin) / BS;
  {
    const int32_t* bt = p.block_tables + static_cast<size_t>(gs) * p.max_blocks_per_seq + t_begin / BS;
    for (int i = lane; i < nblk; i += kWave) blk_ids[wave][i] = bt[i];  // nblk <= kMaxPartBlocks
  }
  __builtin_amdgcn_s_waitcnt(0);  // wave-private slice: own stores only
  const int* my_ids = blk_ids[wave];

  const ChunkLoader<kInt8, D, BS> ld(p, kvh, c, g);
  auto chunk_blocks = [&](int ch, int blk[2], int row0[2]) {
    const int t0 = t_begin + ch * 32;
    if (BS == 16) {
      const int lb = ch * 2;
      blk[0] = __builtin_amdgcn_readfirstlane(my_ids[lb]);
      blk[1] = (t0 + 16 < t_end) ? __builtin_amdgcn_readfirstlane(my_ids[lb + 1]) : blk[0];
      row0[0] = 0;
      row0[1] = 0;
    } else {
      blk[0] = blk[1] = __builtin_amdgcn_readfirstlane(my_ids[ch]);
      row0[0] = 0;
      row0[1] = 16;
    }
  };

  float m_run[NT], l_run[NT];
  f32x4 acc[NT][NN];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto consume = [&](const Chunk<kInt8, D>& cw, int ch) {
    const int t0 = t_begin + ch * 32;
    const bool tail = (t0 + 32) > t_end;  // only a lone last block at bs = 16
    // V^T operands of the chunk, shared by the query tiles
    u32x4 vw[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n) {
      if constexpr (kInt8) {
        vw[n] = u32x4{i8pair_to_bf16x2(cw.v[0][n], 0), i8pair_to_bf16x2(cw.v[0][n], 1),
                      i8pair_to_bf16x2(cw.v[1][n], 0), i8pair_to_bf16x2(cw.v[1][n], 1)};
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
      f32x4 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kInt8) {
#pragma unroll
          for (int jj = 0; jj < NJ / 2; ++jj) {
            const u32x4 w = cw.k[h][jj];
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(i8x8_to_bf16(w.x, w.y), qf[t][2 * jj], s[h], 0, 0, 0);
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(i8x8_to_bf16(w.z, w.w), qf[t][2 * jj + 1], s[h], 0, 0, 0);
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
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = groups_max(mx);
      const float m_new = fmaxf(m_run[t], mx);
      if (__any(m_new > m_run[t])) {
        const float alpha = fast_exp2(m_run[t] - m_new);
        l_run[t] *= alpha;
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[t][n] *= alpha;
        m_run[t] = m_new;
      }
      uint32_t ph[4], pl[4];
      {
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(sc[e] - m_run[t]);
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run[t] += pr[e];
        if constexpr (kInt8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] *= vs[e >> 2][e & 3];
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

  const int nchunks = (t_end - t_begin + 31) / 32;
  {
    Chunk<kInt8, D> cb;
    int blk[2], row0[2];
    for (int ch = wave; ch < nchunks; ch += W) {
      chunk_blocks(ch, blk, row0);
      ld.load(cb, blk, row0);
      consume(cb, ch);
    }
  }

  // merge the waves' states per query (wave 0 keeps the result)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    l_run[t] = groups_sum(l_run[t]);
    red_m[wave][t][lane] = m_run[t];
    red_l[wave][t][lane] = l_run[t];
    if (wave > 0) {
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_acc[wave - 1][t][4 * n + i][lane] = acc[t][n][i];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float M = m_run[t];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, red_m[w][t][lane]);
    // M is finite: wave 0 always has chunk 0 (the partition is non-empty)
    const float f0 = fast_exp2(m_run[t] - M);
    float Lsum = l_run[t] * f0;
#pragma unroll
    for (int n = 0; n < NN; ++n) acc[t][n] *= f0;
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const float fw = fast_exp2(red_m[w][t][lane] - M);  // -inf (idle wave) -> 0
      Lsum += fw * red_l[w][t][lane];
#pragma unroll
      for (int n = 0; n < NN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][n][i] += fw * red_acc[w - 1][t][4 * n + i][lane];
    }
    const int r = q0 + 16 * t + c;
    if (r >= nq) continue;
    const size_t bh = static_cast<size_t>(gs + r / G) * H + kvh * G + r % G;
    const size_t slot = bh * p.num_parts + part;
    float* arow = p.ws_acc + slot * D;
#pragma unroll
    for (int n = 0; n < NN; ++n) *reinterpret_cast<f32x4*>(arow + 16 * n + 4 * g) = acc[t][n];
    if (g == 0) {
      p.ws_m[slot] = M;
      p.ws_l[slot] = Lsum;
    }
  }
}

template <bool kInt8, int D, int BS>
hipError_t launch_t(const DecodeParams& p, int max_group_size, hipStream_t s) {
  const int G = p.num_heads / p.num_kv_heads;
  const int qtiles = (max_group_size * G + 16 * kPrefixTiles - 1) / (16 * kPrefixTiles);
  const dim3 grid(static_cast<unsigned>(p.num_groups * p.num_kv_heads), static_cast<unsigned>(qtiles),
                  static_cast<unsigned>(p.prefix_parts));
  hipLaunchKernelGGL((cascade_prefix_kernel<kInt8, D, BS, kDecodeWaves, kPrefixTiles>), grid,
                     dim3(kDecodeWaves * kWave), 0, s, p);
  return hipGetLastError();
}

template <bool kInt8>
hipError_t launch_kv(const DecodeParams& p, int max_group_size, hipStream_t s) {
  if (p.head_dim == 128)
    return p.block_size == 16 ? launch_t<kInt8, 128, 16>(p, max_group_size, s)
                              : launch_t<kInt8, 128, 32>(p, max_group_size, s);
  return p.block_size == 16 ? launch_t<kInt8, 64, 16>(p, max_group_size, s)
                            : launch_t<kInt8, 64, 32>(p, max_group_size, s);
}

}  // namespace

hipError_t launch_cascade_prefix(const DecodeParams& p, KvKind kv, int max_group_size, hipStream_t s) {
  return kv == KvKind::I8 ? launch_kv<true>(p, max_group_size, s) : launch_kv<false>(p, max_group_size, s);
}

}  // namespace pkv
