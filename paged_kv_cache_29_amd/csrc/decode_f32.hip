// Paged decode attention with an fp32 query over an fp32 paged KV cache, on
// the vector ALUs.  Same definition, grid and partial format as the
// matrix-core kernel (decode_mfma.hip); fp32 operands keep the result within
// fp32 rounding of the exact attention, which the bf16 matrix cores cannot.
//
// One workgroup per (sequence, kv-head, context partition).  Its waves take
// the partition's tokens round-robin; a lane owns dims lane and lane + 64.
// For each token the wave reads the K row and the V column once and updates
// the online softmax of all G heads of the group (scores reduced across the
// wave by shuffles).  The waves' states are merged through LDS.

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

  // Fused step: the partition holding the newest token writes it, by the
  // wave that reads token L - 1 (waves take tokens round-robin), which
  // waits for its own stores; nothing else reads the token.
  if (p.k_new != nullptr && L - 1 >= t_begin && L - 1 < t_end && wave == (L - 1 - t_begin) % W) {
    append_new_token<KvKind::F32, D, BS>(p, b, kvh, L - 1, lane);
    __builtin_amdgcn_s_waitcnt(0);
  }

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

  const float* kc = static_cast<const float*>(p.k_cache);
  const float* vc = static_cast<const float*>(p.v_cache);
  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  for (int t = t_begin + wave; t < t_end; t += W) {
    const int blk = bt[t / BS];
    const int r = t % BS;
    const size_t tile = (static_cast<size_t>(blk) * Hkv + kvh) * (BS * D);
    float kk[ND], vv[ND];
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const int d = lane + kWave * k;
      kk[k] = kc[tile + static_cast<size_t>(r) * D + d];
      vv[k] = vc[tile + (static_cast<size_t>(r >> 2) * D + d) * 4 + (r & 3)];
    }
#pragma unroll
    for (int cc = 0; cc < kMaxGroup; ++cc) {
      if (cc >= G) continue;
      float part_dot = 0.f;
#pragma unroll
      for (int k = 0; k < ND; ++k) part_dot = fmaf(qv[cc][k], kk[k], part_dot);
      const float s = wave_sum(part_dot) * p.scale_log2;
      const float m_new = fmaxf(m[cc], s);
      const float alpha = exp2f(m[cc] - m_new);
      const float pr = exp2f(s - m_new);
      l[cc] = l[cc] * alpha + pr;
#pragma unroll
      for (int k = 0; k < ND; ++k) acc[cc][k] = fmaf(acc[cc][k], alpha, pr * vv[k]);
      m[cc] = m_new;
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
  hipLaunchKernelGGL((decode_f32_kernel<D, BS, kDecodeWaves>), grid, dim3(kDecodeWaves * kWave),
                     0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t s) {
  if (p.head_dim == 128) return p.block_size == 16 ? launch_t<128, 16>(p, s) : launch_t<128, 32>(p, s);
  return p.block_size == 16 ? launch_t<64, 16>(p, s) : launch_t<64, 32>(p, s);
}

}  // namespace pkv
