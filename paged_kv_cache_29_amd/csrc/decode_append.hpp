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

// The append in two halves, so that its loads can be issued early and its
// stores late: append_load() reads the new rows and the block id into
// registers without waiting for them; append_store() quantises (coded
// caches) and stores.  Both are called by one whole wave (lane = its lane
// index); pos = L - 1 >= 0.  KV: F32 or BF16 (bit copy), I8, FP8, E5M2 or I4
// (quantised from fp32 rows, K then V).  The stores are not waited for:
// the caller waits for them (s_waitcnt vmcnt(0)) before it loads what they
// write.
template <KvKind KV, int D>
struct AppendRegs {
  static constexpr bool kCoded = KV == KvKind::I8 || KV == KvKind::FP8 || KV == KvKind::E5M2;
  // values per lane of each row: bit copies (lane owns dims lane + 64i),
  // coded (the same dims, fp32), INT4 (lane < D/2 owns dims 2 lane, 2 lane + 1)
  static constexpr int N = KV == KvKind::I4 ? 2 : (D + kWave - 1) / kWave;
  using T = typename std::conditional<KV == KvKind::BF16, uint16_t, float>::type;
  T k[N], v[N];
  int blk;
};

template <KvKind KV, int D, int BS>
__device__ __forceinline__ void append_load(const DecodeParams& p, int b, int kvh, int pos, int lane,
                                            AppendRegs<KV, D>& r) {
  using R = AppendRegs<KV, D>;
  r.blk = p.block_tables[static_cast<size_t>(b) * p.max_blocks_per_seq + pos / BS];
  const size_t src = (static_cast<size_t>(b) * p.num_kv_heads + kvh) * D;
  const typename R::T* kn = static_cast<const typename R::T*>(p.k_new) + src;
  const typename R::T* vn = static_cast<const typename R::T*>(p.v_new) + src;
  if constexpr (KV == KvKind::I4) {
    float2 a = {0.f, 0.f}, c = {0.f, 0.f};
    if (lane < D / 2) {
      a = *reinterpret_cast<const float2*>(kn + 2 * lane);
      c = *reinterpret_cast<const float2*>(vn + 2 * lane);
    }
    r.k[0] = a.x;
    r.k[1] = a.y;
    r.v[0] = c.x;
    r.v[1] = c.y;
  } else {
#pragma unroll
    for (int i = 0; i < R::N; ++i) {
      const int d = lane + kWave * i;
      r.k[i] = d < D ? kn[d] : typename R::T(0);
      r.v[i] = d < D ? vn[d] : typename R::T(0);
    }
  }
}

template <KvKind KV, int D, int BS>
__device__ __forceinline__ void append_store(const DecodeParams& p, int kvh, int pos, int lane,
                                             const AppendRegs<KV, D>& r) {
  using KT = typename std::conditional<
      KV == KvKind::F32, float,
      typename std::conditional<KV == KvKind::BF16, uint16_t, uint8_t>::type>::type;
  using R = AppendRegs<KV, D>;
  const int row = pos % BS;
  const size_t unit = static_cast<size_t>(r.blk) * p.num_kv_heads + kvh;
  const size_t tile = unit * (static_cast<size_t>(BS) * D);
  KT* kc = static_cast<KT*>(const_cast<void*>(p.k_cache));
  KT* vc = static_cast<KT*>(const_cast<void*>(p.v_cache));
  if constexpr (KV == KvKind::I4) {
    const size_t tile4 = unit * (static_cast<size_t>(BS) * D / 2);
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // K, then V
      const float x0 = which == 0 ? r.k[0] : r.v[0], x1 = which == 0 ? r.k[1] : r.v[1];
      const float a = groups_max(row16_max(fmaxf(fabsf(x0), fabsf(x1))));
      const float s = a / 7.0f;
      if (lane < D / 2) {
        const uint8_t byte = static_cast<uint8_t>(pack_int4_pair(quantize_sym<7>(x0, s), quantize_sym<7>(x1, s)));
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
  } else if constexpr (R::kCoded) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // K, then V
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < R::N; ++i) a = fmaxf(a, fabsf(which == 0 ? r.k[i] : r.v[i]));
      a = groups_max(row16_max(a));  // the row's absmax (exact in any order)
      const float s = a / (KV == KvKind::FP8 ? 448.0f : (KV == KvKind::E5M2 ? 57344.0f : 127.0f));
#pragma unroll
      for (int i = 0; i < R::N; ++i) {
        const int d = lane + kWave * i;
        const float x = which == 0 ? r.k[i] : r.v[i];
        const KT code = KV == KvKind::FP8    ? static_cast<KT>(fp8_code(x, s))
                        : KV == KvKind::E5M2 ? static_cast<KT>(e5m2_code(x, s))
                                             : static_cast<KT>(quantize_code(x, s));
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
#pragma unroll
    for (int i = 0; i < R::N; ++i) {
      const int d = lane + kWave * i;
      if (d < D) {
        kc[tile + static_cast<size_t>(row) * D + d] = r.k[i];
        // token group row / 4, dim d, token row % 4
        vc[tile + (static_cast<size_t>(row >> 2) * D + d) * 4 + (row & 3)] = r.v[i];
      }
    }
  }
}

// Both halves at once.
template <KvKind KV, int D, int BS>
__device__ __forceinline__ void append_new_token(const DecodeParams& p, int b, int kvh, int pos, int lane) {
  AppendRegs<KV, D> r;
  append_load<KV, D, BS>(p, b, kvh, pos, lane, r);
  append_store<KV, D, BS>(p, kvh, pos, lane, r);
}

}  // namespace pkv
