"""GPU: decode without a workspace (pkv_paged_attention_decode_noalloc)
against decode with one, through the C ABI.

The no-allocation entry point runs decode's kernels with the split-context
partials in the library's own per-GPU scratch array.  On the same inputs
its output must equal decode's bit for bit (same kernels, same split), and
match the oracle.  Two calls in a row, the second with a smaller input, so
the second reads none of what the first left in the scratch; sizes whose
partials exceed the scratch are refused before anything launches.
"""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_29_amd as pkv
from paged_kv_cache_29_amd import _lib, workloads

from gpu_helpers import DEV, DeviceWorkload, assert_parity, oracle_out, out_f64

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def _both(dw):
    """decode with a workspace, then the no-allocation call into a fresh output."""
    w = dw.w
    dw.step()  # writes the new tokens, then decode into dw.out
    ref = out_f64(dw.out)
    out = torch.full_like(dw.q, float("nan"))
    pkv.paged_attention_decode_noalloc(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables,
                                       dw.context_lens, w.scale, w.num_heads, w.num_kv_heads,
                                       w.head_dim, w.block_size, k_scale=dw.k_scale, v_scale=dw.v_scale)
    torch.cuda.synchronize()
    return out_f64(out), ref


def _need(w):
    return pkv.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                              w.max_blocks_per_seq)


def test_noalloc_two_calls_second_smaller():
    # 1: a 70B-shaped GQA batch (balanced shares, split contexts, reduce)
    lens = [int(x) for x in np.random.default_rng(3).integers(1000, 20000, 24)]
    w1 = workloads.build("noalloc_1", 3, lens, 64, 8, 128, 16, "bf16", "bf16", spare=0.1)
    assert pkv.balanced_shares(w1.num_seqs, w1.num_kv_heads, w1.block_size, w1.max_blocks_per_seq,
                               torch.bfloat16) > 0
    got1, ref1 = _both(DeviceWorkload(w1))
    assert np.array_equal(got1, ref1), "noalloc differs from decode (call 1)"
    assert_parity(got1, oracle_out(w1), "bf16", "noalloc call 1")
    # 2: a smaller int8 batch (fewer units, fewer shares, different split)
    w2 = workloads.build("noalloc_2", 4, [5000, 37, 0, 2100, 900], 16, 2, 128, 16, "i8", "bf16", spare=0.1)
    got2, ref2 = _both(DeviceWorkload(w2))
    assert np.array_equal(got2, ref2), "noalloc differs from decode (call 2)"
    assert_parity(got2, oracle_out(w2), "i8", "noalloc call 2")
    assert np.all(got2[2] == 0.0)


@pytest.mark.parametrize("kind,lens,G,Hkv,D,bs", [
    ("i4", [8192] * 8, 8, 8, 128, 16),       # fixed partitions + reduce
    ("fp8", [3000, 20, 4100], 4, 2, 64, 32),  # balanced, bs 32
    ("bf16", [64] * 128, 1, 8, 128, 16),      # one partition per sequence: no scratch used
    ("f32", [47, 200, 16, 1, 700], 1, 4, 64, 16),
])
def test_noalloc_matches_decode(kind, lens, G, Hkv, D, bs):
    w = workloads.build(f"noalloc_{kind}", 5, lens, G * Hkv, Hkv, D, bs, kind,
                        "f32" if kind == "f32" else "bf16", spare=0.1)
    assert _need(w) <= SCRATCH_BYTES
    got, ref = _both(DeviceWorkload(w))
    assert np.array_equal(got, ref), f"noalloc differs from decode ({kind})"
    assert_parity(got, oracle_out(w), kind, f"noalloc {kind}")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """INT4 (fixed 2048-token partitions) at 64 x 64 heads over 32K-token
    tables needs 34 MB of partials: refused, nothing launched, out untouched.
    (The tables are valid and every context empty, so the inputs are safe
    even though nothing reads them.)"""
    B, H, Hkv, D, bs, MB = 64, 64, 8, 128, 16, 2048
    q = torch.zeros((B, H, D), dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(q, 7.0)
    kc = torch.zeros((1, Hkv, bs, D // 2), dtype=torch.uint8, device=DEV)
    vc = torch.zeros((1, Hkv, bs // 4, D // 2, 4), dtype=torch.uint8, device=DEV)
    ks = torch.zeros((1, Hkv, bs), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    bt = torch.zeros((B, MB), dtype=torch.int32, device=DEV)
    cl = torch.zeros((B,), dtype=torch.int32, device=DEV)
    assert pkv.workspace_size(B, H, Hkv, D, bs, MB) > SCRATCH_BYTES
    with pytest.raises(ValueError, match="scratch"):
        pkv.paged_attention_decode_noalloc(out, q, kc, vc, bt, cl, 0.1, H, Hkv, D, bs, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
    # the same refusal straight through the C ABI, with its status code
    lib = _lib.load()
    st = lib.pkv_paged_attention_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
        ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(ks.data_ptr()), ctypes.c_void_p(vs.data_ptr()),
        ctypes.c_void_p(bt.data_ptr()), ctypes.c_void_p(cl.data_ptr()), 0.1, B, H, Hkv, D, bs, MB, 1,
        _lib.PKV_BF16, _lib.PKV_I4, None)
    assert st == _lib.PKV_ERR_WORKSPACE
