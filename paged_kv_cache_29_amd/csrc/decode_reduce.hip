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
  // Partials i = 0 .. nparts-1 live in workspace rows slot(i): partitions
  // of the context, or (cascade) npre shared-prefix partitions in slots
  // 0 .. npre-1 followed by the partitions of the rest of the context from
  // slot prefix_parts on.
  int npre = 0, nparts, skip = 0;
  if (p.group_start != nullptr) {
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
  const size_t base = static_cast<size_t>(bh) * p.num_parts;
  // workspace row (of ws_m / ws_l, and of D floats in ws_acc) of partial i
  auto slot = [&](int i) -> size_t { return base + (i < npre ? i : i + skip); };
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
  M = groups_max(row16_max(M));  // lane moves on the vector ALUs, no LDS

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
  den = groups_sum(row16_sum(den));
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

// Balanced shares: one wave per (sequence, kv-head) unit.  The unit's
// record {first slot, splits} says where its partials are (split j >= 1 in
// slot 2 (first / 2 + j)); 1 split: written whole by the partition kernel;
// 0: an empty context, zero output.  Shared-prefix decode: the partials of
// the group's shared tokens (per head, in rows [0, bal_row0)) come first
// and every unit is merged, whatever its count.  The wave serves all G heads of the
// unit: 64 / G lanes per head, each owning DPL = D G / 64 consecutive dims,
// so a unit that needs nothing costs one load.  The first batch of
// partials (maxima, sums and rows) is loaded with the maxima of the rest,
// and each later batch's loads are all issued before any is used, so a
// merge of up to NBATCH partials waits on two dependent loads: the record,
// then everything else.  (Balanced shares serve bf16 queries only, so
// the output is bf16.)
template <int D, int G>
__global__ __launch_bounds__(kReduceWaves * kWave) void decode_reduce_units_kernel(DecodeParams p) {
  constexpr int LPH = kWave / G;  // lanes per head
  constexpr int DPL = D / LPH;    // dims per lane
  constexpr int NV = (DPL + 3) / 4;  // f32x4 (or shorter) pieces per row
  // partials per batch: a 70B-shaped unit splits over up to ~6 shares (G = 8),
  // merged in one batch
  constexpr int NBATCH = DPL >= 64 ? 2 : (DPL >= 32 ? 4 : 8);
  const int lane = threadIdx.x & (kWave - 1);
  const int u = __builtin_amdgcn_readfirstlane(blockIdx.x * kReduceWaves + (threadIdx.x >> 6));
  if (u >= p.num_seqs * p.num_kv_heads) return;  // the whole wave
  const int2 rec = *reinterpret_cast<const int2*>(p.ws_unit + 2 * static_cast<size_t>(u));
  const int first = __builtin_amdgcn_readfirstlane(rec.x);
  const int nsplit = max(__builtin_amdgcn_readfirstlane(rec.y), 0);
  const bool cascade = p.group_start != nullptr;
  if (!cascade && nsplit == 1) return;
  // shared-prefix partials of the unit's sequence
  const int npre = cascade ? (group_shared_tokens(p, group_of(p, u / p.num_kv_heads)) + p.prefix_part_tokens - 1) /
                                 p.prefix_part_tokens
                           : 0;
  const int n = npre + nsplit;
  const int gh = lane / LPH;  // head within the group
  const int d0 = (lane % LPH) * DPL;
  const size_t hrow = static_cast<size_t>(u) * G + gh;  // output row b * H + h
  uint16_t* orow = static_cast<uint16_t*>(p.out) + hrow * D + d0;
  if (n == 0) {  // empty context
#pragma unroll
    for (int k = 0; k < DPL; ++k) orow[k] = 0;
    return;
  }
  // workspace row of partial j: the shared tokens' partitions, then the splits
  auto slot = [&](int j) -> size_t {
    if (j < npre) return hrow * p.num_parts + j;
    j -= npre;
    return static_cast<size_t>(p.bal_row0) + static_cast<size_t>(j == 0 ? first : 2 * ((first >> 1) + j)) * G + gh;
  };
  auto load_row = [&](size_t r, float (&x)[NV * 4]) {
    const float* a = p.ws_acc + r * D + d0;
    if constexpr (DPL % 4 == 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(a + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * v + e] = w[e];
      }
    } else {
#pragma unroll
      for (int k = 0; k < DPL; ++k) x[k] = a[k];
    }
  };
  // the first batch's maxima, sums and rows are loaded together with the
  // maxima of any later partials, before the overall maximum is known
  float num[NV * 4];
#pragma unroll
  for (int k = 0; k < NV * 4; ++k) num[k] = 0.f;
  float den = 0.f;
  float x0[NBATCH][NV * 4], m0[NBATCH], l0[NBATCH];
#pragma unroll
  for (int q = 0; q < NBATCH; ++q) {
    const size_t r = slot(min(q, n - 1));  // past the last partial: weight 0 below
    m0[q] = p.ws_m[r];
    l0[q] = p.ws_l[r];
    load_row(r, x0[q]);
  }
  float M = -INFINITY;
  for (int j = NBATCH; j < n; ++j) M = fmaxf(M, p.ws_m[slot(j)]);
#pragma unroll
  for (int q = 0; q < NBATCH; ++q) M = fmaxf(M, m0[q]);
#pragma unroll
  for (int q = 0; q < NBATCH; ++q) {
    const float w = (q < n) ? exp2f(m0[q] - M) : 0.f;
    den = fmaf(w, l0[q], den);
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] = fmaf(w, x0[q][k], num[k]);
  }
  for (int j0 = NBATCH; j0 < n; j0 += NBATCH) {
    float x[NBATCH][NV * 4];
    float mj[NBATCH], lj[NBATCH];
#pragma unroll
    for (int q = 0; q < NBATCH; ++q) {
      const size_t r = slot(min(j0 + q, n - 1));
      mj[q] = p.ws_m[r];
      lj[q] = p.ws_l[r];
      load_row(r, x[q]);
    }
#pragma unroll
    for (int q = 0; q < NBATCH; ++q) {
      const float w = (j0 + q < n) ? exp2f(mj[q] - M) : 0.f;
      den = fmaf(w, lj[q], den);
#pragma unroll
      for (int k = 0; k < DPL; ++k) num[k] = fmaf(w, x[q][k], num[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) orow[k] = f32_to_bf16(num[k] / den);
}

template <int D, int G>
void launch_units(const DecodeParams& p, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads;
  const dim3 grid(static_cast<unsigned>((waves + kReduceWaves - 1) / kReduceWaves));
  hipLaunchKernelGGL((decode_reduce_units_kernel<D, G>), grid, dim3(kReduceWaves * kWave), 0, s, p);
}

template <int D>
hipError_t launch_t(const DecodeParams& p, bool out_bf16, hipStream_t s) {
  if (p.bal_shares > 0) {
    if (!out_bf16) return hipErrorInvalidValue;  // balanced shares take bf16 queries only
    switch (p.num_heads / p.num_kv_heads) {
      case 1: launch_units<D, 1>(p, s); break;
      case 2: launch_units<D, 2>(p, s); break;
      case 4: launch_units<D, 4>(p, s); break;
      case 8: launch_units<D, 8>(p, s); break;
      case 16: launch_units<D, 16>(p, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
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
