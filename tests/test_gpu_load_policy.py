"""GPU: the K/V load policy changes no result.

Decode loads K/V with the non-temporal hint when the cache pool is larger
than 512 MiB (pkv.streams_cache).  A small ragged workload is placed at the
start of pools just large enough to stream (the blocks past it are never
named by a table); the fused step, then plain decode and the no-allocation
call, on those pools equal the same calls on the workload's own small pools
(default policy) bit for bit, outputs and caches."""

import numpy as np
import pytest
import torch

import paged_kv_cache_29_amd as pkv
from paged_kv_cache_29_amd import workloads

from gpu_helpers import DEV, DeviceWorkload, assert_parity, oracle_out, out_f64

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 64, 100, 255, 256, 257, 700, 2049, 3000]
KV_BYTES = {"bf16": 4, "i8": 2, "fp8": 2, "e5m2": 2, "i4": 1}  # K + V bytes per dim
TORCH_KV = {"bf16": torch.bfloat16, "i8": torch.int8, "fp8": torch.float8_e4m3fn,
            "e5m2": torch.float8_e5m2, "i4": torch.uint8}


def _streaming_blocks(w):
    """The fewest blocks whose pool streams."""
    per_block = w.num_kv_heads * w.block_size * (
        KV_BYTES[w.kv_dtype] * w.head_dim + (0 if w.kv_dtype == "bf16" else 8))
    nb = (512 << 20) // per_block + 1
    assert pkv.streams_cache(nb, w.num_kv_heads, w.block_size, w.head_dim, TORCH_KV[w.kv_dtype])
    assert not pkv.streams_cache(nb - 1, w.num_kv_heads, w.block_size, w.head_dim, TORCH_KV[w.kv_dtype])
    return nb


def _grow(dw, nb):
    def big(t):
        b = torch.empty((nb,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)
        b[: t.shape[0]].copy_(t)
        return b
    dw.k_cache, dw.v_cache = big(dw.k_cache), big(dw.v_cache)
    if dw.k_scale is not None:
        dw.k_scale, dw.v_scale = big(dw.k_scale), big(dw.v_scale)


def _bytes(t, n):
    return t[:n].contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("pt", [0, 64])
@pytest.mark.parametrize("kv,G,D,bs", [("bf16", 1, 128, 16), ("bf16", 8, 128, 32), ("bf16", 4, 64, 16),
                                       ("i8", 8, 128, 16), ("fp8", 4, 128, 32), ("e5m2", 1, 128, 16),
                                       ("i4", 8, 128, 16), ("i4", 2, 64, 32)])
def test_streamed_loads_equal_default_loads(kv, G, D, bs, pt):
    Hkv = 2
    w = workloads.make_custom(300 + G + bs + D, RAGGED, G * Hkv, Hkv, D, bs, kv_dtype=kv)
    assert not pkv.streams_cache(w.num_blocks, Hkv, bs, D, TORCH_KV[kv])
    nb = _streaming_blocks(w)
    print(f"\n[load policy] {kv} G={G} D={D} bs={bs} pt={pt}: {w.num_blocks} -> {nb} blocks", flush=True)
    small, large = DeviceWorkload(w), DeviceWorkload(w)
    _grow(large, nb)

    ref = small.step_fused(partition_tokens=pt)
    got = large.step_fused(partition_tokens=pt)
    assert np.array_equal(got, ref), "fused step: streamed loads differ from default loads"
    n = w.num_blocks
    caches = [(small.k_cache, large.k_cache), (small.v_cache, large.v_cache)]
    if small.k_scale is not None:
        caches += [(small.k_scale, large.k_scale), (small.v_scale, large.v_scale)]
    for a, b in caches:
        assert np.array_equal(_bytes(a, n), _bytes(b, n)), "caches differ after the step"
    assert_parity(got, oracle_out(w), kv, f"streamed fused step {kv} G={G} D={D} bs={bs}")

    # plain decode (and, with automatic partitions, the no-allocation call)
    # over the caches the step left
    ref2 = out_f64(small.decode(partition_tokens=pt, out=torch.empty_like(small.q)))
    got2 = out_f64(large.decode(partition_tokens=pt, out=torch.empty_like(large.q)))
    assert np.array_equal(got2, ref2), "decode: streamed loads differ from default loads"
    assert np.array_equal(got2, got), "decode after the step differs from the step"
    if pt == 0:
        out = torch.empty_like(large.q)
        pkv.paged_attention_decode_noalloc(out, large.q, large.k_cache, large.v_cache, large.block_tables,
                                           large.context_lens, w.scale, w.num_heads, Hkv, D, bs,
                                           k_scale=large.k_scale, v_scale=large.v_scale)
        assert np.array_equal(out_f64(out), ref2), "no-allocation decode: streamed loads differ"
    torch.cuda.synchronize()

