// Paged decode attention, bf16 query over a bf16, int8, FP8 or INT4 paged KV
// cache, on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed: for each sequence b and query head h, softmax(scale *
// K_b q) V_b over the L = context_lens[b] cached tokens, gathered through the
// block table ("LLM Engineering (5)" [ENG5], "Paged attention"; every decode
// step reads the whole KV cache: [ENG5] "Two phases with very different
// characteristics").  int8, FP8 and INT4 caches hold codes with one fp32
// scale per (token, kv-head) ([ENG5] "KV-cache quantization").
//
// Work decomposition.  A workgroup of kDecodeWaves waves attends token
// ranges of (sequence, kv-head) units: one (unit, context partition of
// part_tokens tokens) on fixed partitions, or the units its equal share of
// all units' chunks covers (kBal, below).  The G query heads of the kv-head
// share every K/V byte it loads: the tile feeds one matrix-core contraction
// whose N dimension is the head group (one head per kv-head: the vector
// ALUs instead, kVec).  The waves take 32-token chunks of a range
// round-robin, each keeping its own online-softmax state; the states are
// merged through LDS at the end.  A unit attended whole is finished here;
// split ones leave (max, sum, unnormalised output) partials for the reduce
// kernel.  Each wave issues the loads of a batch of two chunks before
// consuming either.
//
// Per 32-token chunk (two 16-token sub-tiles: two blocks at bs=16, the two
// halves of one block at bs=32), one wave does:
//   S^T[16 tok x 16 heads] = K_sub[16 x D] . Q^T[D x 16]   D/32 MFMAs per sub-tile
//     A operand: lane l holds row l % 16 of the K sub-tile, 8 dims, loaded
//     straight from HBM (16 bytes); B operand Q^T is built once (heads >= G
//     are zero).  The accumulator gives lane group g = l / 16 the scores of
//     sub-tile tokens 4g .. 4g+3 for head l % 16.
//   online softmax on the 8 scores a lane holds, max across the 4 lane
//     groups by lane swaps (v_permlane16/32_swap).
//   O^T[D x 16 heads] += V^T[D x 32 tok] . P^T[32 tok x 16 heads]   2 * D/16 MFMAs
//     A operand: V tiles are stored in groups of 4 tokens, dim-major inside
//     a group (element (r, d) at ((r / 4) D + d) 4 + r % 4), so the 4 tokens
//     a lane needs from each sub-tile are contiguous for every dim, and one
//     16-byte load gives them for several dims (decode_tile.hpp).
//     B operand: the lane's own 8 probabilities, split into a bf16 hi/lo
//     pair (two MFMAs) so the weights keep ~16 bits; no shuffle is needed
//     because the score layout already matches.
// Every load address is a uniform block base (scalar registers) plus a
// loop-invariant lane offset, so prefetching a chunk needs no vector
// address arithmetic.
// The contraction index of each MFMA is a free pairing of (lane group,
// element) to (dim or token); A and B use the same pairing, so only the row
// / column / accumulator layouts of the instruction matter here.
//
// INT4 caches: codes enter the contractions as c + 136 (see decode_tile.hpp).
// The score accumulator starts at -136 * sum_d q_d, which cancels the offset
// in K; the offset in V adds 136 * sum_t p_t v_scale_t to every output dim
// of a head, which each wave subtracts from its accumulator before the
// waves are merged.  Output tile 2m takes the even dims of the dim pairs a
// lane loaded, tile 2m + 1 the odd ones.

#include <type_traits>

#include "decode_append.hpp"
#include "decode_tile.hpp"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"
#include "prefix_body.hpp"

namespace pkv {
namespace {



// Chunks whose loads one wave issues together (32 KB of bf16 K/V, 16.5 KB of
// int8 codes and scales), at two waves per SIMD.  Larger int8 batches were
// measured slower.
template <KvKind KV>
constexpr int kBatch = 2;

// Waves per SIMD.  Two chunks in flight per wave at two waves saturate
// the bf16, int8 and FP8 streams; an INT4 chunk carries half the bytes for
// the same arithmetic, and a third wave (162 VGPRs fit) hides more of the
// load latency (measured 8% faster; int8 and FP8 gain nothing).  Several
// column tiles (multi-query) need the registers of two waves per SIMD.
template <KvKind KV, int NT>
constexpr int kWavesPerSimd = KV == KvKind::I4 && NT == 1 ? 3 : 2;

// Chunks of the smallest share of the balanced mode (below, 256 tokens):
// fewer chunks would cost more in per-segment set-up than they gain in
// spread.
constexpr int kMinShareChunks = 8;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// KV: BF16, or codes with per-token scales (I8, FP8: bytes; I4: nibbles).
// kMQ: multi-query attention (speculative verification of a few new tokens
// per sequence).  The columns are (new token, head) pairs of one sequence's
// kv-head group instead of its heads: its n new tokens x G heads make
// p.mq_tiles tiles of 16, and a workgroup takes NT consecutive ones (all of
// them, or one per workgroup); column i sits at position L - n + i / G and
// sees tokens 0 .. L - n + i / G (causal); every partition leaves partials
// (empty ones with max -inf, sum 0) and the reduce always runs.  With
// NT > 1 tiles every wave carries the tiles' states over one chunk in
// flight: each K and V operand is loaded and widened once for all of them.
// kBal: balanced shares instead of fixed partitions.  The chunks of every
// (sequence, kv-head) unit, laid end to end in unit order (u = b * Hkv +
// kvh), are cut into equal contiguous shares, one per workgroup of a grid
// sized to the GPU's workgroup slots; a workgroup attends the pieces of
// the units its share covers one after the other (segments).  A unit that
// lies inside one share is finished there; a split unit is the first or
// the last segment of each share it touches, so its partials go to that
// share's two slots (2s, 2s + 1), and the workgroup holding its first chunk
// records where they are ({first slot, count} in ws_unit) for the reduce.
// kVec: one query head per kv-head (MHA), bf16.  A single column would use
// 1 of the 16 of every matrix-core tile, so the contractions run on the
// vector ALUs instead, over the same loaded chunk: lane (c, g) takes the
// dot product of its 32 dims of token c of each sub-tile (v_dot2c_f32_bf16,
// summed over the 4 lane groups), and for PV fetches the probabilities of
// its V tokens 4g .. 4g+3 from the lanes that scored them (ds_bpermute).
// kPrefixNT > 0: shared-prefix decode in one launch.  Workgroups [0,
// p.fused_prefix_wgs) attend the groups' shared tokens (prefix_body.hpp
// with kPrefixNT query tiles per wave; block coordinates from the linear
// index, the (group, kv-head) index fastest so that one kv-head's shared
// blocks stay on one XCD), the rest take balanced shares of the sequences'
// own tokens.  One launch rather than two streams: a cross-stream fork and
// join idle the GPU for longer than running the two side by side gains,
// and the shared-prefix workgroups, dispatched first, leave the shares to
// fill the GPU around them.  fused_prefix_wgs is a multiple of 8, so a
// share's XCD follows its index as in the plain balanced launch.
// kNT: the K/V tiles are loaded with the non-temporal hint (one-query
// decode over a pool too large for the memory-side cache to keep between
// steps; the host decides from the pool's size).
template <KvKind KV, int D, int BS, int W, bool kMQ, int NT, bool kBal, bool kVec = false, int kPrefixNT = 0,
          bool kNT = false>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<KV, NT>, kWavesPerSimd<KV, NT>)))
void decode_mfma_kernel(DecodeParams p) {
  static_assert(kPrefixNT == 0 || (!kMQ && W == kDecodeWaves), "one-launch cascade: one query per sequence");

  // the workgroup's share and the number of shares (balanced mode), or its
  // (sequence, kv-head) and partition
  int vbid = blockIdx.x, vgrid = gridDim.x, vpart = blockIdx.y;
  if constexpr (kPrefixNT > 0) {
    const int np = p.fused_prefix_wgs;
    if (vbid < np) {
      const int px = p.num_groups * p.num_kv_heads, py = p.fused_prefix_qtiles;
      if (vbid < px * py * p.prefix_parts)  // else padding
        prefix_body<KV, D, BS, kPrefixNT, false>(p, vbid % px, (vbid / px) % py, vbid / (px * py));
      return;
    }
    vbid -= np;
    vgrid -= np;
    // (fixed partitions: a workgroup per unit, in whole slabs of 16 units;
    // it attends the unit's partitions in turn, so vpart stays 0)
  }
  constexpr bool kInt8 = KV != KvKind::BF16;  // codes (int8, FP8, INT4) with scales
  constexpr bool kI4 = KV == KvKind::I4;
  using ChunkT = typename std::conditional<kI4, ChunkI4<D>, Chunk<kInt8, D>>::type;
  // kNT: K/V tiles loaded with the non-temporal hint (one-query decode over
  // a pool too large to stay in the memory-side cache)
  static_assert(!kNT || (!kMQ && kPrefixNT == 0), "non-temporal loads: plain decode and step");
  constexpr int kPol = kNT ? kNonTemporal : 0;
  using LoaderT = typename std::conditional<kI4, ChunkLoaderI4<D, BS, kPol>, ChunkLoader<kInt8, D, BS, kPol>>::type;
  static_assert(NT >= 1 && NT <= kMqDecodeMaxTiles && (kMQ || NT == 1), "column tiles");
  static_assert(!(kBal && kMQ), "balanced shares are a one-query mode");
  static_assert(!kVec || (KV == KvKind::BF16 && NT == 1 && !kMQ), "vector-ALU path: bf16, one head");
  // the registers of the extra tiles' states replace the second chunk
  constexpr int NB = NT > 1 ? 1 : kBatch<KV>;
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(BS == 16 || BS == 32, "block_size");
  constexpr int NJ = D / 32;  // QK MFMAs per score tile
  constexpr int NN = D / 16;  // PV MFMA pairs per chunk
  constexpr int kPiece = kMaxPartBlocks * BS;  // tokens whose block ids one staging holds

  __shared__ float red_acc[W > 1 ? W - 1 : 1][NN * 4][kWave];
  __shared__ float red_m[W][kWave];
  __shared__ float red_l[W][kWave];
  __shared__ int blk_ids[W][kMaxPartBlocks];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane & 15;  // head column / row in the MFMA tiles
  const int g = lane >> 4;  // lane group

  const int Hkv = p.num_kv_heads;
  const int H = p.num_heads;
  const int G = H / Hkv;
  uint16_t* out = static_cast<uint16_t*>(p.out);

  // Attends tokens [t_begin, t_end) of sequence b (context L >= 1) for
  // kv-head kvh: the column tiles tile0 .. tile0 + NT - 1 (multi-query:
  // query rows from qrow0, nnew new tokens, ncol columns; else the G heads).
  // final_out: the range is the whole context, so the normalised output is
  // written; otherwise the partial goes to slot pslot (fixed partitions:
  // slot pslot of the (row, head)'s num_parts; balanced: share slot pslot,
  // one row per head of the group).
  // The piece whose block ids this wave's LDS slice holds (sequence, first
  // and end token): the next segment of a share is mostly the next kv-head
  // of the same sequence over the same tokens, whose block ids are the same.
  int staged_b = -1, staged_pb = -1, staged_pe = -1;
  auto run = [&](int b, int kvh, int L, int t_begin, int t_end, int tile0, int qrow0, int nnew,
                 int ncol, bool final_out, int64_t pslot) {
    const int h0 = kvh * G;
    // multi-query: column 16 t + c of tile t sees tokens 0 .. lim[t]; the
    // workgroup reads nothing past its last column's position
    int lim[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) lim[t] = kMQ ? L - nnew + (16 * (tile0 + t) + c) / G : 0;
    const int lim_lo = kMQ ? L - nnew + (16 * tile0) / G : 0;  // the first column's

    // Fused step: the range holding the newest token writes it, and the
    // wave that will attend it (chunk append_ch of the piece starting at
    // append_pb; a piece's chunks go to the waves round-robin) is the one
    // that writes.  Its loads are issued here, beside the query's; its
    // stores go out once the wave's first chunk loads are in flight (or,
    // when that first load batch holds the chunk itself, just before it),
    // and the wave waits for them only before it loads that chunk.  No other
    // wave waits.
    int append_pb = -1, append_ch = -1;
    bool append_pending = false;
    AppendRegs<KV, D> app;
    if (!kMQ && p.k_new != nullptr && L - 1 >= t_begin && L - 1 < t_end) {
      append_pb = t_begin + (L - 1 - t_begin) / kPiece * kPiece;
      append_ch = (L - 1 - append_pb) / 32;
      if (wave == append_ch % W) {
        append_load<KV, D, BS>(p, b, kvh, L - 1, lane, app);
        append_pending = true;
      }
    }
    auto append_flush = [&]() {
      if (append_pending) {
        append_store<KV, D, BS>(p, kvh, L - 1, lane, app);
        append_pending = false;
      }
    };
    // INT4 (three waves per SIMD) has no registers to carry the row: it
    // stores at once
    if constexpr (kI4) append_flush();

    // Q^T operand (B of the score MFMA): lane (c, g), tile t, MFMA j, 8 dims.
    bf16x8 qf[NT][NJ];
    float k_off[NT];  // INT4: 136 * sum_d q_d of column c
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * (tile0 + t) + c;
      // (vector-ALU path: every lane holds the one head's dims)
      const size_t qr = kMQ ? (static_cast<size_t>(qrow0 + col / G) * H + h0 + col % G)
                            : (static_cast<size_t>(b) * H + h0 + (kVec ? 0 : c));
      const bool qvalid = kMQ ? (col < ncol) : (kVec || c < G);
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + qr * D;
      k_off[t] = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int d0 = kI4 ? ((D / 4) * g + 8 * j)
                           : (kInt8 ? (64 * (j >> 1) + 16 * g + 8 * (j & 1)) : (32 * j + 8 * g));
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qvalid) v = load_u32x4(qrow + d0);
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

    const int32_t* bt_row = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
    const int* my_ids = blk_ids[wave];
    const LoaderT ld(p, kvh, c, g);

    float m_run[NT], l_run[NT];
    float pv_run[NT];  // INT4: sum_t p_t v_scale_t (this lane's tokens)
    f32x4 acc[NT][NN];
    // vector-ALU path: dims 32k + 2c + o (n = 2k + o) over the lane
    // group's tokens
    float vacc[kVec ? NN : 1];
#pragma unroll
    for (int n = 0; n < (kVec ? NN : 1); ++n) vacc[n] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m_run[t] = -INFINITY;
      l_run[t] = 0.f;
      pv_run[t] = 0.f;
#pragma unroll
      for (int n = 0; n < NN; ++n) acc[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The range in pieces of at most kPiece tokens (one staging of block ids
    // each; fixed partitions are one piece).  Pieces start on chunk
    // boundaries, so only the last chunk of the last piece can be partial.
    for (int pb = t_begin; pb < t_end; pb += kPiece) {
      const int pe = min(t_end, pb + kPiece);
      // Physical block ids of the piece, staged in this wave's LDS slice so
      // that reading them later waits on LDS traffic only, never on the K/V
      // loads in flight (unless the slice holds them already).
      if (b != staged_b || pb != staged_pb || pe != staged_pe) {
        const int nblk = (pe - pb + BS - 1) / BS;  // <= kMaxPartBlocks
        const int32_t* bt = bt_row + pb / BS;
        for (int i = lane; i < nblk; i += kWave) blk_ids[wave][i] = bt[i];
        __builtin_amdgcn_s_waitcnt(0);  // wave-private slice: own stores only
        staged_b = b;
        staged_pb = pb;
        staged_pe = pe;
      }

      // Block ids of chunk `ch` of the piece (uniform).  Past the end of the
      // range the second half reuses the first block: valid memory whose rows
      // are masked.
      auto chunk_blocks = [&](int ch, int blk[2], int row0[2]) {
        const int t0 = pb + ch * 32;
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

      // `masked` (a compile-time bool): the chunk may hold tokens past the
      // end of the range or past a column's position.  Clean chunks (all but
      // the last of a range) take the instantiation without any masking
      // code: left to a runtime branch, the compiler turns the masking into
      // selects that every chunk executes.
      auto consume = [&](const ChunkT& cw, int ch, auto masked) {
        constexpr bool kMasked = decltype(masked)::value;
        const int t0 = pb + ch * 32;
        if constexpr (kVec) {
          // ---- scores of chunk tokens 16h + c (every lane group holds all)
          float sc[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const u32x4 qw = __builtin_bit_cast(u32x4, qf[0][j]);
#pragma unroll
              for (int w = 0; w < 4; ++w) a = dot2_bf16(cw.k[h][j][w], qw[w], a);
            }
            sc[h] = groups_sum(a) * p.scale_log2;
          }
          const bool past_end = kMasked && (t0 + 32) > t_end;
          if (past_end) {  // select, never multiply: masked rows may hold NaN
#pragma unroll
            for (int h = 0; h < 2; ++h)
              if (t0 + 16 * h + c >= t_end) sc[h] = -INFINITY;
          }
          // ---- online softmax: every row of 16 lanes holds the chunk's 32
          // scores, so the maximum and the state are uniform
          const float m_new = fmaxf(m_run[0], row16_max(fmaxf(sc[0], sc[1])));
          if (m_new > m_run[0]) {
            const float alpha = fast_exp2(m_run[0] - m_new);
            l_run[0] *= alpha;
#pragma unroll
            for (int n = 0; n < NN; ++n) vacc[n] *= alpha;
            m_run[0] = m_new;
          }
          float pr[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) pr[h] = fast_exp2(sc[h] - m_run[0]);
          l_run[0] += pr[0] + pr[1];  // summed over the row at the end
          // ---- PV: probabilities of sub-tile tokens 4g + i (lane 20g + i
          // scored them), as bf16 hi + lo pairs as in the matrix-core path
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float pt[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pt[i] = lane_get(pr[h], 20 * g + i);
            const uint32_t h01 = pack_bf16x2(pt[0], pt[1]), h23 = pack_bf16x2(pt[2], pt[3]);
            const uint32_t l01 = pack_bf16x2(pt[0] - bf16_lo(h01), pt[1] - bf16_hi(h01));
            const uint32_t l23 = pack_bf16x2(pt[2] - bf16_lo(h23), pt[3] - bf16_hi(h23));
#pragma unroll
            for (int n = 0; n < NN; ++n) {
              u32x2 v = cw.v[h][n];
              if (past_end) {  // masked tokens contribute exact zeros, even over NaN
                v.x = mask_pair(v.x, t0 + 16 * h + 4 * g, t_end);
                v.y = mask_pair(v.y, t0 + 16 * h + 4 * g + 2, t_end);
              }
              float a = vacc[n];
              a = dot2_bf16(v.x, h01, a);
              a = dot2_bf16(v.x, l01, a);
              a = dot2_bf16(v.y, h23, a);
              vacc[n] = dot2_bf16(v.y, l23, a);
            }
          }
          return;
        }
        // ---- scores: S^T of sub-tiles h = 0, 1 for every column tile; each K
        // operand is widened once and feeds the tiles' contractions
        f32x4 s[NT][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            s[t][h] = kI4 ? f32x4{-k_off[t], -k_off[t], -k_off[t], -k_off[t]} : f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (kI4) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              uint32_t lo, hi;
              int4_nibbles(cw.k[h][j], lo, hi);
              const u32x2 a = nib4_to_bf16(lo), bq = nib4_to_bf16(hi);
              const bf16x8 ka = as_bf16x8(u32x4{a.x, a.y, bq.x, bq.y});
#pragma unroll
              for (int t = 0; t < NT; ++t) s[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[t][j], s[t][h], 0, 0, 0);
            }
          } else if constexpr (kInt8) {
#pragma unroll
            for (int jj = 0; jj < NJ / 2; ++jj) {
              const u32x4 w = cw.k[h][jj];
              const bf16x8 k0 = codes8_to_bf16<KV>(w.x, w.y), k1 = codes8_to_bf16<KV>(w.z, w.w);
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                s[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[t][2 * jj], s[t][h], 0, 0, 0);
                s[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[t][2 * jj + 1], s[t][h], 0, 0, 0);
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
              for (int t = 0; t < NT; ++t)
                s[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cw.k[h][j]), qf[t][j], s[t][h], 0, 0, 0);
          }
        }
        // ---- online softmax (log2 domain); lane = column c, tokens 4g + i of
        // sub-tile h (chunk token 16h + 4g + i), element e = 4h + i
        // multi-query: also mask tokens past a column's position
        const bool past_end = kMasked && (t0 + 32) > t_end;
        const bool tail = kMasked && (past_end || (kMQ && t0 + 31 > lim_lo));
        // V scales of the lane's tokens; zero past the end of the range,
        // where rows may hold NaN (select, never multiply)
        f32x4 vs[2] = {f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};
        if constexpr (kInt8) {
          vs[0] = cw.vs[0];
          vs[1] = cw.vs[1];
        }
        if (past_end) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t0 + 16 * (e >> 2) + 4 * g + (e & 3) >= t_end) vs[e >> 2][e & 3] = 0.f;
        }
        // P^T operands as bf16 pairs hi + lo (hi = bf16(p), lo = bf16(p - hi)):
        // two contractions give the weights to ~2^-16 relative instead of 2^-9.
        uint32_t ph[NT][4], pl[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float sc[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = s[t][h][i];
              if constexpr (kInt8) x *= cw.ks[h][i];
              sc[4 * h + i] = x * p.scale_log2;
            }
          }
          if (tail) {  // select, never multiply: masked rows may hold NaN
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int tok = t0 + 16 * (e >> 2) + 4 * g + (e & 3);
              if (tok >= t_end || (kMQ && tok > lim[t])) sc[e] = -INFINITY;
            }
          }
          float mx = sc[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
          mx = groups_max(mx);
          const float m_new = fmaxf(m_run[t], mx);
          if (__any(m_new > m_run[t])) {
            float alpha = fast_exp2(m_run[t] - m_new);
            if constexpr (kMQ) alpha = (m_new == -INFINITY) ? 1.f : alpha;  // a column that saw nothing yet
            l_run[t] *= alpha;
            if constexpr (kI4) pv_run[t] *= alpha;
#pragma unroll
            for (int n = 0; n < NN; ++n) acc[t][n] *= alpha;
            m_run[t] = m_new;
          }
          float pr[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(sc[e] - m_run[t]);
          if constexpr (kMQ) {  // -inf - -inf: a column that saw nothing yet
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
            ph[t][i] = pack_bf16x2(pr[2 * i], pr[2 * i + 1]);
            pl[t][i] = pack_bf16x2(pr[2 * i] - bf16_lo(ph[t][i]), pr[2 * i + 1] - bf16_hi(ph[t][i]));
          }
        }
        // ---- O^T += V^T . P^T; each V operand is widened once for the tiles
        if constexpr (kI4) {
#pragma unroll
          for (int m = 0; m < NN / 2; ++m) {
            uint32_t lo0, hi0, lo1, hi1;
            int4_nibbles(cw.v[0][m], lo0, hi0);
            int4_nibbles(cw.v[1][m], lo1, hi1);
            const u32x2 a0 = nib4_to_bf16(lo0), a1 = nib4_to_bf16(lo1);
            const u32x2 b0 = nib4_to_bf16(hi0), b1 = nib4_to_bf16(hi1);
            u32x4 ve = {a0.x, a0.y, a1.x, a1.y};  // dim 32m + 2c, tokens e = 4h + i
            u32x4 vo = {b0.x, b0.y, b1.x, b1.y};  // dim 32m + 2c + 1
            if (past_end) {  // masked tokens contribute exact zeros
              const int ta = t0 + 4 * g;
              ve.x = mask_pair(ve.x, ta, t_end);
              ve.y = mask_pair(ve.y, ta + 2, t_end);
              ve.z = mask_pair(ve.z, ta + 16, t_end);
              ve.w = mask_pair(ve.w, ta + 18, t_end);
              vo.x = mask_pair(vo.x, ta, t_end);
              vo.y = mask_pair(vo.y, ta + 2, t_end);
              vo.z = mask_pair(vo.z, ta + 16, t_end);
              vo.w = mask_pair(vo.w, ta + 18, t_end);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const bf16x8 pfh = as_bf16x8(u32x4{ph[t][0], ph[t][1], ph[t][2], ph[t][3]});
              const bf16x8 pfl = as_bf16x8(u32x4{pl[t][0], pl[t][1], pl[t][2], pl[t][3]});
              acc[t][2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ve), pfh, acc[t][2 * m], 0, 0, 0);
              acc[t][2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ve), pfl, acc[t][2 * m], 0, 0, 0);
              acc[t][2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vo), pfh, acc[t][2 * m + 1], 0, 0, 0);
              acc[t][2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vo), pfl, acc[t][2 * m + 1], 0, 0, 0);
            }
          }
          return;
        }
#pragma unroll
        for (int n = 0; n < NN; ++n) {
          u32x4 vw;
          if constexpr (kInt8) {
            vw = u32x4{codes_to_bf16x2<KV, 0>(cw.v[0][n]), codes_to_bf16x2<KV, 1>(cw.v[0][n]),
                       codes_to_bf16x2<KV, 0>(cw.v[1][n]), codes_to_bf16x2<KV, 1>(cw.v[1][n])};
          } else {
            vw = u32x4{cw.v[0][n].x, cw.v[0][n].y, cw.v[1][n].x, cw.v[1][n].y};
          }
          if (past_end) {  // masked tokens contribute exact zeros, even over NaN
            const int ta = t0 + 4 * g;
            vw.x = mask_pair(vw.x, ta, t_end);
            vw.y = mask_pair(vw.y, ta + 2, t_end);
            vw.z = mask_pair(vw.z, ta + 16, t_end);
            vw.w = mask_pair(vw.w, ta + 18, t_end);
          }
          const bf16x8 va = as_bf16x8(vw);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16x8 pfh = as_bf16x8(u32x4{ph[t][0], ph[t][1], ph[t][2], ph[t][3]});
            const bf16x8 pfl = as_bf16x8(u32x4{pl[t][0], pl[t][1], pl[t][2], pl[t][3]});
            acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfh, acc[t][n], 0, 0, 0);
            acc[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfl, acc[t][n], 0, 0, 0);
          }
        }
      };

      // ---- this wave's chunks ch = wave, wave + W, ... of the piece in
      // batches of NB: the loads of the whole batch are issued before any
      // chunk is consumed, and no load stays pending across iterations, so
      // every wait counts exactly the loads behind it.  A batch is loaded and
      // consumed last chunk first, so the full-batch and tail branches share
      // no leading code the compiler could hoist, together with its waits,
      // above the batch's other loads.
      // Full batches take only clean chunks (every token inside the range
      // and, multi-query, at or before every column's position); from the
      // first batch that would reach an unclean chunk on, chunks go one at a
      // time through the masked instantiation.
      // (Batches of one chunk, several column tiles, keep the one masked body
      // for every chunk, and so does INT4 at bs = 32: a second copy of their
      // body spills.)
      constexpr bool kCleanBatches = NB > 1 && !(kI4 && BS == 32);
      using kBatchMasked = std::integral_constant<bool, !kCleanBatches>;
      const int nchunks = (pe - pb + 31) / 32;
      const int nclean = kCleanBatches ? max(0, ((kMQ ? min(pe, lim_lo + 1) : pe) - pb) / 32) : nchunks;
      {
        ChunkT cb[NB];
        int blk[2], row0[2];
        // this wave holds the chunk written by the append in this piece,
        // among chunks ch .. last: store now if not done yet, and wait for
        // the append's stores before loading it
        auto append_wait = [&](int ch, int last) {
          if (pb == append_pb && wave == append_ch % W && append_ch >= ch && append_ch <= last) {
            append_flush();
            __builtin_amdgcn_s_waitcnt(0);
          }
        };
        for (int ch = wave; ch < nchunks; ch += NB * W) {
          if (ch + (NB - 1) * W < nclean) {
            append_wait(ch, ch + (NB - 1) * W);
#pragma unroll
            for (int k = NB - 1; k >= 0; --k) {
              chunk_blocks(ch + k * W, blk, row0);
              ld.load(cb[k], blk, row0);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of the math
            append_flush();  // the append's stores behind the batch's loads
#pragma unroll
            for (int k = NB - 1; k >= 0; --k) consume(cb[k], ch + k * W, kBatchMasked{});
          } else {
            for (int c2 = ch; c2 < nchunks; c2 += W) {
              append_wait(c2, c2);
              chunk_blocks(c2, blk, row0);
              ld.load(cb[0], blk, row0);
              append_flush();
              consume(cb[0], c2, std::true_type{});
            }
          }
        }
      }
    }

    if constexpr (kVec) {
      // to the matrix-core path's state: the sum over a row of lanes; the
      // output dims summed over the lane groups and moved to the
      // accumulator layout (element i of tile n = 2k + o in lane (c, g): dim
      // 32k + 8g + 2i + o, i.e. column 4g + i here)
      l_run[0] = row16_sum(l_run[0]);
#pragma unroll
      for (int n = 0; n < NN; ++n) {
        const float v = groups_sum(vacc[n]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[0][n][i] = lane_get(v, 4 * g + i);
      }
    }
    // per-column sums over the 4 lane groups (each holds different tokens)
    float M[NT], Lsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (!kVec) l_run[t] = groups_sum(l_run[t]);
      if constexpr (kI4) {  // remove the V offset of this wave's tokens
        const float v_off = kInt4Offset * groups_sum(pv_run[t]);
#pragma unroll
        for (int n = 0; n < NN; ++n) acc[t][n] -= v_off;
      }
      M[t] = m_run[t];
      Lsum[t] = l_run[t];
    }

    if constexpr (W > 1) {
      // the waves' states merge into wave 0 through LDS, one column tile at a
      // time (the buffers hold one tile)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t > 0) __syncthreads();  // wave 0 has read the previous tile
        red_m[wave][lane] = m_run[t];
        red_l[wave][lane] = l_run[t];
        if (wave > 0) {
#pragma unroll
          for (int n = 0; n < NN; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) red_acc[wave - 1][4 * n + i][lane] = acc[t][n][i];
        }
        __syncthreads();
        if (wave == 0) {
          float Mt = m_run[t];
#pragma unroll
          for (int w = 1; w < W; ++w) Mt = fmaxf(Mt, red_m[w][lane]);
          // Mt finite: wave 0 saw a chunk (multi-query: unless the column saw nothing)
          const float f0 = (kMQ && Mt == -INFINITY) ? 0.f : fast_exp2(m_run[t] - Mt);
          float Ls = l_run[t] * f0;
#pragma unroll
          for (int n = 0; n < NN; ++n) acc[t][n] *= f0;
#pragma unroll
          for (int w = 1; w < W; ++w) {
            const float fw = (kMQ && Mt == -INFINITY) ? 0.f : fast_exp2(red_m[w][lane] - Mt);  // idle wave -> 0
            Ls += fw * red_l[w][lane];
#pragma unroll
            for (int n = 0; n < NN; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[t][n][i] += fw * red_acc[w - 1][4 * n + i][lane];
          }
          M[t] = Mt;
          Lsum[t] = Ls;
        }
      }
      if (wave != 0) return;
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * (tile0 + t) + c;
      if (kMQ ? col >= ncol : c >= G) continue;
      // output row: (sequence, head), or (query row, head) in multi-query mode
      const size_t bh = kMQ ? static_cast<size_t>(qrow0 + col / G) * H + h0 + col % G
                            : static_cast<size_t>(b) * H + h0 + c;
      const size_t slot = kBal ? static_cast<size_t>(p.bal_row0 + pslot * G + c) : bh * p.num_parts + pslot;
      // Output maps: accumulator element i of tile n in lane (c, g) is row
      // 4g + i of that tile, and the row's dim follows the V operand loads
      // (decode_tile.hpp); each lane ends up with runs of consecutive dims.
      uint16_t* orow = out + bh * D;
      float* arow = p.ws_acc + slot * D;
      const float ls = Lsum[t];  // final outputs are acc / ls
      if (!final_out) {
        store_partial_row<KV, D>(arow, acc[t], g);
      } else if constexpr (kI4) {
        // the normalised output in bf16 over the same dims as the partial
        // row (store_partial_row): 8P g + 2P i + n, P = D/32
        constexpr int P = D / 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = 8 * P * g + 2 * P * i;
          uint32_t wv[P];
#pragma unroll
          for (int m = 0; m < P; ++m) wv[m] = pack_bf16x2(acc[t][2 * m][i] / ls, acc[t][2 * m + 1][i] / ls);
          if constexpr (P == 4)
            *reinterpret_cast<u32x4*>(orow + d0) = u32x4{wv[0], wv[1], wv[2], wv[3]};
          else
            *reinterpret_cast<u32x2*>(orow + d0) = u32x2{wv[0], wv[1]};
        }
      } else if constexpr (kInt8) {
        // byte codes: dims 64k + 16g + 4i + j
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const int d0 = 64 * k + 16 * g;
          uint32_t wv[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            wv[2 * i] = pack_bf16x2(acc[t][4 * k][i] / ls, acc[t][4 * k + 1][i] / ls);
            wv[2 * i + 1] = pack_bf16x2(acc[t][4 * k + 2][i] / ls, acc[t][4 * k + 3][i] / ls);
          }
          *reinterpret_cast<u32x4*>(orow + d0) = u32x4{wv[0], wv[1], wv[2], wv[3]};
          *reinterpret_cast<u32x4*>(orow + d0 + 8) = u32x4{wv[4], wv[5], wv[6], wv[7]};
        }
      } else {
        // bf16: dims 32k + 8g + 2i + o
#pragma unroll
        for (int k = 0; k < NN / 2; ++k) {
          const int d0 = 32 * k + 8 * g;
          const f32x4 e = acc[t][2 * k], o = acc[t][2 * k + 1];
          *reinterpret_cast<u32x4*>(orow + d0) =
              u32x4{pack_bf16x2(e[0] / ls, o[0] / ls), pack_bf16x2(e[1] / ls, o[1] / ls),
                    pack_bf16x2(e[2] / ls, o[2] / ls), pack_bf16x2(e[3] / ls, o[3] / ls)};
        }
      }
      if (!final_out && g == 0) {
        p.ws_m[slot] = M[t];
        p.ws_l[slot] = Lsum[t];
      }
    }
  };

  if constexpr (kBal) {
    // ---- the workgroup's share.  Unit u = b * Hkv + kvh covers tokens
    // [S_b, L_b) of sequence b (S_b: its group's shared tokens in cascade
    // mode, else 0) in n_b = ceil((L_b - S_b) / 32) chunks; sequence b's
    // units start at chunk Hkv * P_b, P_b = sum of n over the sequences
    // before b.  The waves read the sequences in rounds of W * 64, one per
    // lane, and combine their sums through LDS; the values stay uniform.
    const int B = p.num_seqs;
    const bool cascade = p.group_start != nullptr;
    auto own_begin = [&](int bb) { return cascade ? group_shared_tokens(p, group_of(p, bb)) : 0; };
    constexpr int R = W * kWave;  // sequences per round
    __shared__ int64_t bal_wsum[W];
    __shared__ int64_t bal_found[4];  // b, L, S, first chunk of b's units
    // one round from sequence `base`: this lane's sequence (length, own
    // start, chunks, chunks of the round's sequences before it) and the
    // round's total; every wave takes part
    struct Round {
      int L, S, n;
      int64_t x, tot;
    };
    auto round_at = [&](int base) {
      Round r;
      const int bb = base + wave * kWave + lane;
      r.L = bb < B ? max(p.context_lens[bb], 0) : 0;
      r.S = bb < B ? own_begin(bb) : 0;
      r.n = r.L > r.S ? (r.L - r.S + 31) >> 5 : 0;
      const int64_t incl = wave_incl_scan(r.n);
      if (lane == kWave - 1) bal_wsum[wave] = incl;
      __syncthreads();
      int64_t woff = 0;
      r.tot = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const int64_t t = bal_wsum[w];
        woff += w < wave ? t : 0;
        r.tot += t;
      }
      __syncthreads();  // bal_wsum is rewritten by the next round
      r.x = woff + incl - r.n;
      return r;
    };
    Round r0{};  // the first round's (all of them when B <= R)
    int64_t C = 0;  // chunks of all units
    for (int base = 0; base < B; base += R) {
      const Round r = round_at(base);
      if (base == 0) r0 = r;
      // a sequence without tokens of its own is in no share: its unit
      // records say so ({0, 0}: zero output, or the shared tokens' partials
      // alone), written by one workgroup of the grid
      const int bb = base + wave * kWave + lane;
      if (bb < B && r.n == 0 && bb % vgrid == vbid) {
        for (int kv = 0; kv < Hkv; ++kv)
          *reinterpret_cast<int2*>(p.ws_unit + 2 * (static_cast<size_t>(bb) * Hkv + kv)) = int2{0, 0};
      }
      C += r.tot;
    }
    C *= Hkv;
    // shares: at least kMinShareChunks chunks each, at most one per
    // workgroup, a multiple of 8 (the XCD count) once there are 8
    int64_t se = min(static_cast<int64_t>(vgrid), C / kMinShareChunks);
    se = max(se, int64_t(1));
    if (se >= 8) se &= ~int64_t(7);
    const int Se = static_cast<int>(se);
    const int bid = vbid;
    if (bid >= Se) return;
    // workgroups go to the XCDs round-robin; share s = XCD-major, so each
    // XCD takes a contiguous run of shares and the kv-heads whose scale rows
    // share cache lines run on one XCD's L2
    const int s = Se >= 8 ? (bid & 7) * (Se >> 3) + (bid >> 3) : bid;
    const int64_t cq = C / Se, cr = C % Se;
    const int64_t a = cq * s + (cr * s) / Se;            // floor(s C / Se)
    const int64_t e = cq * (s + 1) + (cr * (s + 1)) / Se;
    if (a >= e) return;  // no chunks at all
    // share holding chunk x: the largest s' with floor(s' C / Se) <= x
    auto share_of = [&](int64_t x) { return ((x + 1) * Se - 1) / C; };

    // the sequence holding chunk a (exactly one lane's), and where its
    // units start; from the kept first round, or (B > R) rounds read again
    int64_t pos0 = 0;  // chunks of the units before the round
    Round r = r0;
    for (int base = 0;; base += R) {
      if (base > 0) r = round_at(base);
      if (pos0 + r.tot * Hkv > a || base + R >= B) {
        const int bb = base + wave * kWave + lane;
        const int64_t first = pos0 + r.x * Hkv;
        if (bb < B && r.n > 0 && first <= a && a < first + static_cast<int64_t>(r.n) * Hkv) {
          bal_found[0] = bb;
          bal_found[1] = r.L;
          bal_found[2] = r.S;
          bal_found[3] = first;
        }
        break;
      }
      pos0 += r.tot * Hkv;
    }
    __syncthreads();
    int b = __builtin_amdgcn_readfirstlane(static_cast<int>(bal_found[0]));
    int L = __builtin_amdgcn_readfirstlane(static_cast<int>(bal_found[1]));
    int S = __builtin_amdgcn_readfirstlane(static_cast<int>(bal_found[2]));
    const int64_t pos = readlane64(bal_found[3], 0);
    int nb = (L - S + 31) >> 5;
    int kvh = static_cast<int>((a - pos) / nb);
    int64_t cu = pos + static_cast<int64_t>(kvh) * nb;  // first chunk of unit (b, kvh)
    int64_t lo = a;
    for (;;) {
      const int64_t uend = cu + nb;
      const int64_t hi = min(uend, e);
      const bool whole = lo == cu && hi == uend;
      // split segments: the share's first or last slot; a whole unit of a
      // cascade (which leaves a partial too) has a slot of its own after
      // the shares' (several can lie inside one share)
      const int64_t pslot = (whole && cascade) ? 2 * int64_t(p.bal_shares) + static_cast<int64_t>(b) * Hkv + kvh
                            : lo == a           ? 2 * int64_t(s)
                                                : 2 * int64_t(s) + 1;
      if (lo == cu && threadIdx.x == 0) {  // this share holds the unit's first chunk
        const int nsplit = whole ? 1 : static_cast<int>(share_of(uend - 1) - s + 1);
        *reinterpret_cast<int2*>(p.ws_unit + 2 * (static_cast<size_t>(b) * Hkv + kvh)) =
            int2{static_cast<int>(pslot), nsplit};
      }
      // (cascade: never the final output, the shared tokens' partials remain)
      run(b, kvh, L, S + static_cast<int>(lo - cu) * 32, min(L, S + static_cast<int>(hi - cu) * 32), 0, 0, 0,
          G, whole && !cascade, pslot);
      if (uend >= e) break;
      __syncthreads();  // the merge buffers are reused by the next segment
      lo = cu = uend;
      if (++kvh == Hkv) {
        // the next sequence with tokens of its own (one exists: chunks
        // remain before e)
        kvh = 0;
        do {
          ++b;
          L = p.context_lens[b];
          S = own_begin(b);
        } while (L <= S);
        nb = (L - S + 31) >> 5;
      }
    }
  } else {
    int b, kvh, tile0 = 0;
    if constexpr (kMQ) {
      // blockIdx.x = ((u / 8) * groups + tg) * 8 + u % 8 for u = b * Hkv + kvh
      // and tile group tg (tiles tg * NT ..): the tile groups of one (sequence,
      // kv-head) run on the same XCD (workgroups go to XCDs round-robin) and
      // share its L2
      const int groups = (p.mq_tiles + NT - 1) / NT;
      const int rest = blockIdx.x >> 3;
      tile0 = (rest % groups) * NT;
      const int u = (rest / groups) * 8 + (blockIdx.x & 7);
      if (u >= p.num_seqs * Hkv) return;  // uniform across the workgroup
      b = u / Hkv;
      kvh = u - b * Hkv;
    } else {
      // slabs of 16 (sequence, kv-head) units: unit 16s + 2q + j runs as
      // workgroup 16s + 8j + q, so units 2q and 2q + 1 (kv-heads whose scale
      // rows share a 128-byte line) run on one XCD (workgroups go to the 8
      // XCDs round-robin) and the line is fetched into one L2
      const int u = (vbid & ~15) | ((vbid & 7) << 1) | ((vbid >> 3) & 1);
      if (u >= p.num_seqs * Hkv) return;  // padding, uniform across the workgroup
      b = u / Hkv;
      kvh = u - b * Hkv;
    }
    const int part = vpart;
    const int PT = p.part_tokens;

    const int L = p.context_lens[b];
    // multi-query: this sequence's n new tokens x G heads are its columns
    int qrow0 = 0, nnew = 0, ncol = G;
    if constexpr (kMQ) {
      qrow0 = p.query_start[b];
      nnew = p.query_start[b + 1] - qrow0;
      ncol = nnew * G;
      if (16 * tile0 >= ncol) return;  // uniform; also every sequence with L == 0
    }
    // cascade: the group's shared tokens are attended by the prefix kernel
    const bool cascade = !kMQ && p.group_start != nullptr;
    const int S = cascade ? group_shared_tokens(p, group_of(p, b)) : 0;
    if constexpr (kPrefixNT > 0) {
      // one-launch cascade: the workgroup attends every partition of the
      // sequence's own tokens in turn (the grid holds one workgroup per
      // unit, so no workgroup is launched for a partition past a short tail)
      for (int pt = 0; S + pt * PT < L; ++pt) {
        if (pt > 0) __syncthreads();  // the merge buffers are reused
        run(b, kvh, L, S + pt * PT, min(L, S + (pt + 1) * PT), 0, 0, 0, G, false, p.prefix_parts + pt);
      }
      return;
    }
    const int t_begin = S + part * PT;
    if ((kMQ || cascade || part != 0) && t_begin >= L) return;  // uniform across the workgroup

    if (L <= 0) {  // empty context: zero output
      for (int i = threadIdx.x; i < G * D; i += W * kWave)
        out[(static_cast<size_t>(b) * H + kvh * G) * D + i] = 0;
      return;
    }
    const int t_end = kMQ ? max(t_begin, min(min(L, t_begin + PT),
                                             L - nnew + min(16 * (tile0 + NT) - 1, ncol - 1) / G + 1))
                          : min(L, t_begin + PT);
    const bool single = !kMQ && !cascade && L <= PT;
    run(b, kvh, L, t_begin, t_end, tile0, qrow0, nnew, ncol, single, (cascade ? p.prefix_parts : 0) + part);
  }
}

// One-query decode (and the fused step): balanced shares or fixed
// partitions, the vector-ALU form for one bf16 head per kv-head, and the
// K/V load policy.
template <KvKind KV, int D, int BS, bool kBal, bool kNT>
void launch_plain(dim3 grid, bool vec, const DecodeParams& p, hipStream_t s) {
  const dim3 block(kDecodeWaves * kWave);
  if constexpr (KV == KvKind::BF16) {
    if (vec) {
      hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, true, 0, kNT>), grid, block, 0,
                         s, p);
      return;
    }
  }
  hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, false, 0, kNT>), grid, block, 0, s,
                     p);
}

template <KvKind KV, int D, int BS, bool kMQ>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  // cascade: slots [0, prefix_parts) belong to the shared-prefix kernel
  const int parts = p.group_start != nullptr ? p.num_parts - p.prefix_parts : p.num_parts;
  const unsigned units = static_cast<unsigned>(p.num_seqs * p.num_kv_heads);
  const dim3 block(kDecodeWaves * kWave);
  // one head per kv-head, bf16: the vector-ALU contractions
  const bool vec = KV == KvKind::BF16 && p.num_heads == p.num_kv_heads;
  if constexpr (kMQ) {
    if (p.mq_tiles < 1 || p.mq_tiles > kMqDecodeMaxTiles) return hipErrorInvalidValue;
    // (sequence, kv-head) units padded to whole groups of 8, x tile groups
    const unsigned padded = (units + 7u) / 8u * 8u;
    if (KV == KvKind::I4 || p.mq_tiles == 1) {
      // INT4: one tile per workgroup (more tiles' states do not fit beside
      // its conversion registers at two waves per SIMD)
      const dim3 grid(padded * static_cast<unsigned>(p.mq_tiles), static_cast<unsigned>(parts));
      hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, true, 1, false>), grid, block, 0, s, p);
    } else {
      // every column tile of a (sequence, kv-head) in one workgroup
      static_assert(kMqDecodeMaxTiles == 3, "one instance per tile count");
      const dim3 grid(padded, static_cast<unsigned>(parts));
      if constexpr (KV != KvKind::I4) {
        if (p.mq_tiles == 2)
          hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, true, 2, false>), grid, block, 0, s, p);
        else
          hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, true, 3, false>), grid, block, 0, s, p);
      }
    }
  } else if (p.bal_shares > 0) {
    // balanced shares: one workgroup per share, a 1-D grid (not INT4)
    if constexpr (KV == KvKind::I4) {
      return hipErrorInvalidValue;
    } else {
      const dim3 grid(static_cast<unsigned>(p.bal_shares));
      if (p.stream_loads)
        launch_plain<KV, D, BS, true, true>(grid, vec, p, s);
      else
        launch_plain<KV, D, BS, true, false>(grid, vec, p, s);
    }
  } else {
    const dim3 grid((units + 15u) & ~15u, static_cast<unsigned>(parts));  // whole slabs of 16 units
    if (p.stream_loads)
      launch_plain<KV, D, BS, false, true>(grid, vec, p, s);
    else
      launch_plain<KV, D, BS, false, false>(grid, vec, p, s);
  }
  return hipGetLastError();
}

template <KvKind KV, bool kMQ = false>
hipError_t launch_kv(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128)
    return p.block_size == 16 ? launch_t<KV, 128, 16, kMQ>(p, s) : launch_t<KV, 128, 32, kMQ>(p, s);
  return p.block_size == 16 ? launch_t<KV, 64, 16, kMQ>(p, s) : launch_t<KV, 64, 32, kMQ>(p, s);
}

}  // namespace

int balanced_slots_per_cu(KvKind kv) {
  return kv == KvKind::I4 ? kWavesPerSimd<KvKind::I4, 1> : kWavesPerSimd<KvKind::BF16, 1>;
}

hipError_t launch_decode_mfma(const DecodeParams& p, KvKind kv, hipStream_t s) {
  if (kv == KvKind::I8) return launch_kv<KvKind::I8>(p, s);
  if (kv == KvKind::I4) return launch_kv<KvKind::I4>(p, s);
  if (kv == KvKind::E5M2) return launch_kv<KvKind::E5M2>(p, s);
  if (kv == KvKind::FP8) return launch_kv<KvKind::FP8>(p, s);
  return launch_kv<KvKind::BF16>(p, s);
}

template <KvKind KV, int D, int BS, bool kBal>
void launch_fused_inst(const DecodeParams& p, dim3 grid, hipStream_t s) {
  const dim3 block(kDecodeWaves * kWave);
  const int G = p.num_heads / p.num_kv_heads;
  const bool two = p.fused_prefix_tiles != 1;
  if constexpr (KV == KvKind::BF16) {
    if (G == 1) {  // one head per kv-head: the vector-ALU path
      if (two)
        hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, true, 2>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, true, 1>), grid, block, 0, s, p);
      return;
    }
  }
  if (two)
    hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, false, 2>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<KV, D, BS, kDecodeWaves, false, 1, kBal, false, 1>), grid, block, 0, s, p);
}

template <KvKind KV, int D, int BS>
hipError_t launch_fused_t(const DecodeParams& p, hipStream_t s) {
  // balanced shares, or a workgroup per (sequence, kv-head) that attends
  // the partitions of its own tokens in turn
  const int64_t own = p.bal_shares > 0
                          ? p.bal_shares
                          : ((static_cast<int64_t>(p.num_seqs) * p.num_kv_heads + 15) & ~int64_t(15));
  const int64_t total = static_cast<int64_t>(p.fused_prefix_wgs) + own;
  if (own <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(total));
  if (p.bal_shares > 0)
    launch_fused_inst<KV, D, BS, true>(p, grid, s);
  else
    launch_fused_inst<KV, D, BS, false>(p, grid, s);
  return hipGetLastError();
}

template <KvKind KV>
hipError_t launch_fused_kv(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128)
    return p.block_size == 16 ? launch_fused_t<KV, 128, 16>(p, s) : launch_fused_t<KV, 128, 32>(p, s);
  return p.block_size == 16 ? launch_fused_t<KV, 64, 16>(p, s) : launch_fused_t<KV, 64, 32>(p, s);
}

hipError_t launch_cascade_fused(DecodeParams p, KvKind kv, int max_group_size, hipStream_t s) {
  // shared-prefix workgroups: (group, kv-head) x query tiles x partitions,
  // padded to a multiple of 8
  const int G = p.num_heads / p.num_kv_heads;
  const int64_t cols = static_cast<int64_t>(max_group_size) * G;
  const int64_t qtiles = (cols + prefix_queries_for(cols) - 1) / prefix_queries_for(cols);
  const int64_t cells = static_cast<int64_t>(p.num_groups) * p.num_kv_heads * qtiles * p.prefix_parts;
  if (qtiles > 0x7fffffff || cells > 0x7fffffff - 8) return hipErrorInvalidValue;
  p.fused_prefix_wgs = static_cast<int32_t>((cells + 7) / 8 * 8);
  p.fused_prefix_qtiles = static_cast<int32_t>(qtiles);
  p.fused_prefix_tiles = prefix_tiles_for(cols);
  if (kv == KvKind::I8) return launch_fused_kv<KvKind::I8>(p, s);
  if (kv == KvKind::FP8) return launch_fused_kv<KvKind::FP8>(p, s);
  if (kv == KvKind::E5M2) return launch_fused_kv<KvKind::E5M2>(p, s);
  if (kv == KvKind::BF16) return launch_fused_kv<KvKind::BF16>(p, s);
  return hipErrorInvalidValue;  // INT4 and fp32: two launches
}

hipError_t launch_multi_query_decode(const DecodeParams& p, KvKind kv, hipStream_t s) {
  if (kv == KvKind::I8) return launch_kv<KvKind::I8, true>(p, s);
  if (kv == KvKind::I4) return launch_kv<KvKind::I4, true>(p, s);
  if (kv == KvKind::FP8) return launch_kv<KvKind::FP8, true>(p, s);
  if (kv == KvKind::E5M2) return launch_kv<KvKind::E5M2, true>(p, s);
  return launch_kv<KvKind::BF16, true>(p, s);
}

}  // namespace pkv
