// Paged decode attention with an fp32 query over an fp32 paged KV cache, on
// the vector ALUs.  Same definition, grid and partial format as the
// matrix-core kernel (decode_mfma.hip); fp32 operands keep the result within
// fp32 rounding of the exact attention, which the bf16 matrix cores cannot.
//
// One workgroup per (sequence, kv-head, context partition).  The
// partition's block ids are staged in LDS once; its waves then take
// 8-token chunks round-robin (a chunk lies inside one block), a lane owning
// dims lane and lane + 64.  A wave issues the loads of a batch of chunks
// (per chunk 8 K rows, and the V columns as two 4-token groups) before
// using any, then scores each chunk's 8 tokens for every head of the group
// (dot products summed across the wave by lane moves on the vector ALUs:
// DPP inside each row of 16 lanes, then lane swaps across the rows) and
// updates each head's online softmax once per chunk, so a batch costs one
// memory latency rather than one per token.  The waves' states are merged
// through LDS.

#include "decode_append.hpp"
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kMaxGroup = 16;

template <int D, int BS, int W>
__global__ __launch_bounds__(W * kWave) void decode_f32_kernel(DecodeParams p) {
  constexpr int ND = D / kWave;  // dims per lane
  __shared__ float red_acc[W][kMaxGroup][D];
  __shared__ float red_m[W][kMaxGroup];
  __shared__ float red_l[W][kMaxGroup];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int Hkv = p.num_kv_heads;
  const int H = p.num_heads;
  const int G = H / Hkv;
  const int b = blockIdx.x / Hkv;
  const int kvh = blockIdx.x - b * Hkv;
  const int part = blockIdx.y;
  const int PT = p.part_tokens;
  const int L = p.context_lens[b];
  const int t_begin = part * PT;
  if (part != 0 && t_begin >= L) return;
  const int h0 = kvh * G;
  float* out = static_cast<float*>(p.out);
  if (L <= 0) {
    for (int i = threadIdx.x; i < G * D; i += W * kWave)
      out[(static_cast<size_t>(b) * H + h0) * D + i] = 0.f;
    return;
  }
  const int t_end = min(L, t_begin + PT);
  const bool single = L <= PT;

  // The query rows first, so their loads overlap the staging below.
  float qv[kMaxGroup][ND];
  float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][ND];
  const float* q = static_cast<const float*>(p.q);
#pragma unroll
  for (int cc = 0; cc < kMaxGroup; ++cc) {
    m[cc] = -INFINITY;
    l[cc] = 0.f;
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      acc[cc][k] = 0.f;
      qv[cc][k] = (cc < G) ? q[(static_cast<size_t>(b) * H + h0 + cc) * D + lane + kWave * k] : 0.f;
    }
  }

  // Block ids of the partition (at most kMaxPartBlocks: partitions are at
  // most that many blocks), staged once for all waves.
  __shared__ int ids[kMaxPartBlocks];
  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq + t_begin / BS;
  const int nblk = (t_end - t_begin + BS - 1) / BS;
  for (int i = threadIdx.x; i < nblk; i += W * kWave) ids[i] = bt[i];

  // Fused step: the partition holding the newest token writes it, by the
  // wave that reads token L - 1 (in chunk app_ch, 8 tokens a chunk).  Its
  // loads go out here; its stores once the wave's first batch of loads is
  // in flight, or just before that batch if it holds chunk app_ch; the
  // wave waits for them only before loading that chunk.  Nothing else
  // reads the token.
  const int app_ch = (p.k_new != nullptr && L - 1 >= t_begin && L - 1 < t_end) ? (L - 1 - t_begin) >> 3 : -1;
  bool app_pending = false;
  AppendRegs<KvKind::F32, D> app;
  if (app_ch >= 0 && wave == app_ch % W) {
    append_load<KvKind::F32, D, BS>(p, b, kvh, L - 1, lane, app);
    app_pending = true;
  }
  auto app_flush = [&]() {
    if (app_pending) {
      append_store<KvKind::F32, D, BS>(p, kvh, L - 1, lane, app);
      app_pending = false;
    }
  };
  __syncthreads();

  const float* kc = static_cast<const float*>(p.k_cache);
  const float* vc = static_cast<const float*>(p.v_cache);
  const int nch = (t_end - t_begin + 7) >> 3;
  // the loads of NB chunks go out before any is used (one at D = 128, where
  // a second chunk beside 16 heads' states leaves the registers)
  constexpr int NB = D == 64 ? 4 : 1;
  for (int j0 = wave; j0 < nch; j0 += NB * W) {
    // this batch holds the appended chunk: its stores first, then wait
    if (app_ch >= j0 && app_ch <= j0 + (NB - 1) * W && wave == app_ch % W) {
      app_flush();
      __builtin_amdgcn_s_waitcnt(0);
    }
    float kk[NB][8][ND], vv[NB][8][ND];
    int nvalid[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      // chunks past the range re-read the last one and count no token
      const int j = min(j0 + c * W, nch - 1);
      nvalid[c] = j0 + c * W < nch ? min(8, t_end - t_begin - 8 * j) : 0;
      const int t0 = t_begin + 8 * j;  // 8-aligned, so the chunk lies in one block
      const int blk = __builtin_amdgcn_readfirstlane(ids[(t0 - t_begin) / BS]);
      const int r0 = t0 % BS;
      const size_t tile = (static_cast<size_t>(blk) * Hkv + kvh) * (BS * D);
      // K rows past the range re-read the range's last row (valid data);
      // those tokens get score -inf, probability 0 and V 0
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = min(t0 + i, t_end - 1) % BS;
#pragma unroll
        for (int k = 0; k < ND; ++k) kk[c][i][k] = kc[tile + static_cast<size_t>(r) * D + lane + kWave * k];
      }
      // V tile: token r, dim d at ((r / 4) D + d) 4 + r % 4; the chunk's two
      // groups of 4 tokens are one 16-byte load per dim each
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
#pragma unroll
        for (int k = 0; k < ND; ++k) {
          const size_t off = tile + (static_cast<size_t>((r0 >> 2) + gq) * D + lane + kWave * k) * 4;
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(vc + off);
#pragma unroll
          for (int i = 0; i < 4; ++i) vv[c][4 * gq + i][k] = v4[i];
        }
      }
    }
    app_flush();  // the append's stores behind the batch's loads
#pragma unroll
    for (int c = 0; c < NB; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < ND; ++k) vv[c][i][k] = (i < nvalid[c]) ? vv[c][i][k] : 0.f;  // select: may be NaN
#pragma unroll
      for (int cc = 0; cc < kMaxGroup; ++cc) {
        if (cc >= G) continue;
        float sc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float part_dot = 0.f;
#pragma unroll
          for (int k = 0; k < ND; ++k) part_dot = fmaf(qv[cc][k], kk[c][i][k], part_dot);
          sc[i] = part_dot;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = (i < nvalid[c]) ? groups_sum(row16_sum(sc[i])) * p.scale_log2 : -INFINITY;
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
        // finite: the batch's first chunk holds a token of the range
        const float m_new = fmaxf(m[cc], mx);
        const float alpha = exp2f(m[cc] - m_new);
        float lsum = 0.f, o[ND];
#pragma unroll
        for (int k = 0; k < ND; ++k) o[k] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pr = exp2f(sc[i] - m_new);  // 0 for tokens past the range
          lsum += pr;
#pragma unroll
          for (int k = 0; k < ND; ++k) o[k] = fmaf(pr, vv[c][i][k], o[k]);
        }
        l[cc] = fmaf(l[cc], alpha, lsum);
#pragma unroll
        for (int k = 0; k < ND; ++k) acc[cc][k] = fmaf(acc[cc][k], alpha, o[k]);
        m[cc] = m_new;
      }
    }
  }

  // merge the waves' states through LDS
#pragma unroll
  for (int cc = 0; cc < kMaxGroup; ++cc) {
    if (cc >= G) continue;
#pragma unroll
    for (int k = 0; k < ND; ++k) red_acc[wave][cc][lane + kWave * k] = acc[cc][k];
    if (lane == 0) {
      red_m[wave][cc] = m[cc];
      red_l[wave][cc] = l[cc];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += W * kWave) {
    const int cc = i / D;
    const int d = i - cc * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, red_m[w][cc]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = (red_m[w][cc] == -INFINITY) ? 0.f : exp2f(red_m[w][cc] - M);
      num = fmaf(f, red_acc[w][cc][d], num);
      den = fmaf(f, red_l[w][cc], den);
    }
    const size_t bh = static_cast<size_t>(b) * H + h0 + cc;
    if (single) {
      out[bh * D + d] = num / den;
    } else {
      const size_t slot = bh * p.num_parts + part;
      p.ws_acc[slot * D + d] = num;
      if (d == 0) {
        p.ws_m[slot] = M;
        p.ws_l[slot] = den;
      }
    }
  }
}

template <int D, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.num_seqs * p.num_kv_heads),
                  static_cast<unsigned>(p.num_parts));
  // D = 64: eight waves (measured on the tiny 4-sequence fp32 workload:
  // 10.4 us against 13.8 us with four; four waves with batches of 8 chunks
  // instead of 4 measured 20.1 us); D = 128 keeps four, whose LDS merge
  // buffers then take the same 32 KB
  constexpr int W = D == 64 ? 8 : kDecodeWaves;
  hipLaunchKernelGGL((decode_f32_kernel<D, BS, W>), grid, dim3(W * kWave), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128) return p.block_size == 16 ? launch_t<128, 16>(p, s) : launch_t<128, 32>(p, s);
  return p.block_size == 16 ? launch_t<64, 16>(p, s) : launch_t<64, 32>(p, s);
}

}  // namespace pkv
