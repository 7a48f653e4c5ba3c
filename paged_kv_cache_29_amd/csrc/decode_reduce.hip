// Split-context combine: merges the per-partition partials of sequences
// longer than one partition into the final output.
//
// Partition p of a (sequence, head) left M_p (max scaled score, log2
// domain), S_p = sum_t exp2(s_t - M_p) and A_p = sum_t exp2(s_t - M_p) v_t.
// With M = max_p M_p and w_p = exp2(M_p - M):
//   out = (sum_p w_p A_p) / (sum_p w_p S_p),
// which equals softmax over the whole context exactly (up to rounding), so
// the split never changes the definition.
//
// One wave per (sequence, query head), four per workgroup; a lane owns dims
// lane and lane + 64.  The weights of up to 64 partitions are computed
// lane-parallel and read back one by one with readlane, so the partial rows
// are independent loads the unrolled loop keeps in flight together; the
// first 8 rows are loaded with the partitions' maxima and sums, before the
// wave knows the overall maximum (the kernel is bound by its chain of
// dependent loads, not by its bytes).

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kReduceWaves = 4;

template <int D, bool kOutBf16>
__global__ __launch_bounds__(kReduceWaves * kWave) void decode_reduce_kernel(DecodeParams p) {
  constexpr int ND = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const bool mq = p.query_start != nullptr;
  // (sequence, head), or (query row, head) in multi-query mode
  const int bh = __builtin_amdgcn_readfirstlane(blockIdx.x * kReduceWaves + (threadIdx.x >> 6));
  if (bh >= (mq ? p.num_query_rows : p.num_seqs) * p.num_heads) return;  // the whole wave
  const int b = mq ? range_of(p.query_start, p.num_seqs, bh / p.num_heads) : bh / p.num_heads;
  const int L = p.context_lens[b];
  // Partials i = 0 .. nparts-1 live in workspace rows idx(i): partitions of
  // the context, or (cascade) npre shared-prefix partitions in slots
  // 0 .. npre-1 followed by the partitions of the rest of the context from
  // slot prefix_parts on, or (balanced shares) the share slots the unit's
  // first workgroup recorded.
  int npre = 0, nparts, skip = 0;
  int slot0 = 0, gh = 0;  // balanced: first slot of the unit; head within its group
  if (p.bal_shares > 0) {
    if (L <= 0) {  // empty context: no share attended it
      for (int k = lane; k < D; k += kWave) {
        const size_t idx = static_cast<size_t>(bh) * D + k;
        if constexpr (kOutBf16)
          static_cast<uint16_t*>(p.out)[idx] = 0;
        else
          static_cast<float*>(p.out)[idx] = 0.f;
      }
      return;
    }
    const int G = p.num_heads / p.num_kv_heads;
    const int h = bh - b * p.num_heads;
    gh = h % G;
    const int2 u = *reinterpret_cast<const int2*>(p.ws_unit + 2 * (static_cast<size_t>(b) * p.num_kv_heads + h / G));
    slot0 = __builtin_amdgcn_readfirstlane(u.x);
    nparts = __builtin_amdgcn_readfirstlane(u.y);
    if (nparts <= 1) return;  // written whole by the partition kernel
  } else if (p.group_start != nullptr) {
    const int S = group_shared_tokens(p, group_of(p, b));
    npre = (S + p.prefix_part_tokens - 1) / p.prefix_part_tokens;
    nparts = npre + (L > S ? (L - S + p.part_tokens - 1) / p.part_tokens : 0);
    skip = p.prefix_parts - npre;
    if (nparts == 0) {  // empty context: zero output
      for (int k = lane; k < D; k += kWave) {
        const size_t idx = static_cast<size_t>(bh) * D + k;
        if constexpr (kOutBf16)
          static_cast<uint16_t*>(p.out)[idx] = 0;
        else
          static_cast<float*>(p.out)[idx] = 0.f;
      }
      return;
    }
  } else if (mq) {
    // every partition of the context left a partial (empty ones: max -inf,
    // sum 0); the first always holds token 0, which every query sees
    nparts = (L + p.part_tokens - 1) / p.part_tokens;
  } else {
    nparts = (L + p.part_tokens - 1) / p.part_tokens;
    if (nparts <= 1) return;  // written by the partition kernel
  }
  const bool bal = p.bal_shares > 0;
  const int G = p.num_heads / p.num_kv_heads;
  const size_t base = static_cast<size_t>(bh) * p.num_parts;
  // workspace row (of ws_m / ws_l, and of D floats in ws_acc) of partial i
  auto slot = [&](int i) -> size_t {
    if (bal) return static_cast<size_t>(i == 0 ? slot0 : 2 * ((slot0 >> 1) + i)) * G + gh;
    return base + (i < npre ? i : i + skip);
  };
  const float* m = p.ws_m;
  const float* l = p.ws_l;
  const float* row = p.ws_acc + lane;
  // groups of 8 rows: 8 independent loads per lane in flight; rows past
  // cnt re-read the last valid row and get weight 0 (wv is 0 there)
  auto load8 = [&](float (&x)[8][ND], int first, int j0, int cnt) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t j = slot(first + min(j0 + u, max(cnt - 1, 0)));
#pragma unroll
      for (int k = 0; k < ND; ++k) x[u][k] = row[j * D + kWave * k];
    }
  };
  float num[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) num[k] = 0.f;
  auto add8 = [&](const float (&x)[8][ND], int j0, int cnt, float wv) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), (j0 + u) & (kWave - 1)));
      const float wu = (j0 + u < cnt) ? w : 0.f;
#pragma unroll
      for (int k = 0; k < ND; ++k) num[k] = fmaf(wu, x[u][k], num[k]);
    }
  };

  // the first 8 rows go out with the maxima and sums
  float x0[8][ND];
  load8(x0, 0, 0, min(kWave, nparts));
  const float m0 = lane < nparts ? m[slot(lane)] : -INFINITY;
  const float l0 = lane < nparts ? l[slot(lane)] : 0.f;
  float M = m0;
  for (int i = lane + kWave; i < nparts; i += kWave) M = fmaxf(M, m[slot(i)]);
  M = wave_max(M);

  float den = 0.f;
  for (int first = 0; first < nparts; first += kWave) {
    const int i = first + lane;
    const float mi = first == 0 ? m0 : (i < nparts ? m[slot(i)] : -INFINITY);
    const float li = first == 0 ? l0 : (i < nparts ? l[slot(i)] : 0.f);
    const float wv = (i < nparts) ? exp2f(mi - M) : 0.f;
    if (i < nparts) den = fmaf(wv, li, den);
    const int cnt = min(kWave, nparts - first);
    int j0 = 0;
    if (first == 0) {
      add8(x0, 0, cnt, wv);
      j0 = 8;
    }
    for (; j0 < cnt; j0 += 8) {
      float x[8][ND];
      load8(x, first, j0, cnt);
      add8(x, j0, cnt, wv);
    }
  }
  den = wave_sum(den);
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const float o = num[k] / den;
    const size_t idx = static_cast<size_t>(bh) * D + lane + kWave * k;
    if constexpr (kOutBf16)
      static_cast<uint16_t*>(p.out)[idx] = f32_to_bf16(o);
    else
      static_cast<float*>(p.out)[idx] = o;
  }
}

template <int D>
hipError_t launch_t(const DecodeParams& p, bool out_bf16, hipStream_t s) {
  const int rows = p.query_start != nullptr ? p.num_query_rows : p.num_seqs;
  const int64_t waves = static_cast<int64_t>(rows) * p.num_heads;
  const dim3 grid(static_cast<unsigned>((waves + kReduceWaves - 1) / kReduceWaves));
  const dim3 block(kReduceWaves * kWave);
  if (out_bf16)
    hipLaunchKernelGGL((decode_reduce_kernel<D, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<D, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, bool out_bf16, hipStream_t s) {
  return p.head_dim == 128 ? launch_t<128>(p, out_bf16, s) : launch_t<64>(p, out_bf16, s);
}

}  // namespace pkv
