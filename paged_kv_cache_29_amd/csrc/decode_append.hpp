// Appending a sequence's new token inside a decode launch.
//
// The fused decode step writes each sequence's newest token (position
// L - 1, through the block table) into the cache and then attends over the
// whole context, in one launch.  Only the workgroups of the partition that
// holds position L - 1 write, each only its own kv-head's row, and within a
// workgroup the wave that will attend that position writes it, so no other
// wave or workgroup reads what is written and no barrier is needed.  The write is the same operation
// as the slot-scatter cache write ("LLM Engineering (5)", "Block manager:
// how paging works"); for an int8 cache it is the same quantisation as the
// int8 cache write, through the same quantize_code().
#pragma once

#include <type_traits>

#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {

// Called by one whole wave (lane = its lane index); pos = L - 1 >= 0.  KV:
// F32 or BF16 (bit copy), I8, FP8, E5M2 or I4 (quantised from fp32 rows,
// K then V).  The stores are not waited for here: the caller waits for them
// (s_waitcnt vmcnt(0)) before it loads what they write.
template <KvKind KV, int D, int BS>
__device__ __forceinline__ void append_new_token(const DecodeParams& p, int b, int kvh, int pos, int lane) {
  using KT = typename std::conditional<
      KV == KvKind::F32, float,
      typename std::conditional<KV == KvKind::BF16, uint16_t, uint8_t>::type>::type;
  const int Hkv = p.num_kv_heads;
  const int blk = p.block_tables[static_cast<size_t>(b) * p.max_blocks_per_seq + pos / BS];
  const int row = pos % BS;
  const size_t unit = static_cast<size_t>(blk) * Hkv + kvh;
  const size_t tile = unit * (static_cast<size_t>(BS) * D);
  const size_t src = (static_cast<size_t>(b) * Hkv + kvh) * D;
  KT* kc = static_cast<KT*>(const_cast<void*>(p.k_cache));
  KT* vc = static_cast<KT*>(const_cast<void*>(p.v_cache));
  if constexpr (KV == KvKind::I4) {
    // lane < D/2 owns dims 2 lane and 2 lane + 1, which share one byte
    const size_t tile4 = unit * (static_cast<size_t>(BS) * D / 2);
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // K, then V
      const float* x = static_cast<const float*>(which == 0 ? p.k_new : p.v_new) + src;
      float2 v = {0.f, 0.f};
      if (lane < D / 2) v = *reinterpret_cast<const float2*>(x + 2 * lane);
      const float a = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
      const float s = a / 7.0f;
      if (lane < D / 2) {
        const uint8_t byte = static_cast<uint8_t>(pack_int4_pair(quantize_sym<7>(v.x, s), quantize_sym<7>(v.y, s)));
        if (which == 0)
          kc[tile4 + static_cast<size_t>(row) * (D / 2) + lane] = byte;
        else  // token group row / 4, dim pair lane, token row % 4
          vc[tile4 + (static_cast<size_t>(row >> 2) * (D / 2) + lane) * 4 + (row & 3)] = byte;
      }
      if (lane == 0) {
        float* sc = const_cast<float*>(which == 0 ? p.k_scale : p.v_scale);
        sc[unit * BS + row] = (s > 0.f) ? s : 0.f;
      }
    }
  } else if constexpr (KV == KvKind::I8 || KV == KvKind::FP8 || KV == KvKind::E5M2) {
    // lane owns dims lane + 64i
    constexpr int ND = D / kWave;
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // K, then V
      const float* x = static_cast<const float*>(which == 0 ? p.k_new : p.v_new) + src;
      float v[ND];
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        v[i] = x[lane + kWave * i];
        a = fmaxf(a, fabsf(v[i]));
      }
      a = wave_max(a);
      const float s = a / (KV == KvKind::FP8 ? 448.0f : (KV == KvKind::E5M2 ? 57344.0f : 127.0f));
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const int d = lane + kWave * i;
        const KT code = KV == KvKind::FP8    ? static_cast<KT>(fp8_code(v[i], s))
                        : KV == KvKind::E5M2 ? static_cast<KT>(e5m2_code(v[i], s))
                                             : static_cast<KT>(quantize_code(v[i], s));
        if (which == 0)
          kc[tile + static_cast<size_t>(row) * D + d] = code;
        else
          vc[tile + (static_cast<size_t>(row >> 2) * D + d) * 4 + (row & 3)] = code;
      }
      if (lane == 0) {
        float* sc = const_cast<float*>(which == 0 ? p.k_scale : p.v_scale);
        sc[unit * BS + row] = (s > 0.f) ? s : 0.f;
      }
    }
  } else {
    const KT* kn = static_cast<const KT*>(p.k_new) + src;
    const KT* vn = static_cast<const KT*>(p.v_new) + src;
#pragma unroll
    for (int i = lane; i < D; i += kWave) {
      kc[tile + static_cast<size_t>(row) * D + i] = kn[i];
      // token group row / 4, dim i, token row % 4
      vc[tile + (static_cast<size_t>(row >> 2) * D + i) * 4 + (row & 3)] = vn[i];
    }
  }
}

}  // namespace pkv
