"""GPU: shared-prefix (cascade) decode against the oracle.

The cascade computes the same attention as plain decode, with each group's
shared blocks attended once for all its members and the partials merged by
the split-context combine; the oracle is plain decode's definition on the
members' full block tables."""

import numpy as np
import pytest
import torch

from paged_kv_cache_29_amd import workloads

from gpu_helpers import DeviceWorkload, assert_parity, oracle_out, sample_pairs

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 100, 255, 700]


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "e5m2", "i4"])
@pytest.mark.parametrize("G,D,bs", [(4, 128, 16), (8, 128, 32), (1, 64, 16), (2, 64, 32), (16, 128, 16)])
@pytest.mark.parametrize("prefix,group", [(33, 3), (200, None), (64, 4)])
def test_cascade_matches_oracle(kv, G, D, bs, prefix, group):
    lens = [prefix + x for x in RAGGED]
    w = workloads.make_custom(300 + G + bs + prefix, lens, G * 2, 2, D, bs, kv_dtype=kv,
                              prefix=prefix, prefix_group_size=group)
    dw = DeviceWorkload(w)
    got = dw.step_cascade()
    gs, gsb, mg, ms = dw.groups
    assert ms >= prefix // bs - 1 and mg >= 3  # the sharing is really used
    ref = oracle_out(w)
    assert_parity(got, ref, kv, f"cascade {kv} G={G} D={D} bs={bs} prefix={prefix} group={group}")


@pytest.mark.parametrize("ppt,spt", [(32, 32), (64, 0), (0, 64), (32, 0)])
def test_cascade_partition_sizes(ppt, spt):
    w = workloads.make_custom(41, [200 + x for x in RAGGED], 8, 2, 128, 16, prefix=200)
    dw = DeviceWorkload(w)
    got = dw.step_cascade(partition_tokens=spt, prefix_partition_tokens=ppt)
    assert_parity(got, oracle_out(w), "bf16", f"cascade ppt={ppt} spt={spt}")


def _cache_bytes(dw):
    out = [t.view(torch.uint8).cpu().numpy() for t in (dw.k_cache, dw.v_cache)]
    if dw.k_scale is not None:
        out += [t.view(torch.uint8).cpu().numpy() for t in (dw.k_scale, dw.v_scale)]
    return out


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "e5m2", "i4"])
@pytest.mark.parametrize("G,D,bs,own", [(4, 128, 16, RAGGED), (1, 64, 32, RAGGED),
                                        (8, 128, 16, [1, 900, 3000, 40, 2200])])
@pytest.mark.parametrize("spt", [0, 64])
def test_cascade_fused_step_equals_write_then_cascade(kv, G, D, bs, own, spt):
    """The fused step (new tokens written inside the call) gives the output
    and the caches of kv_cache_write followed by cascade decode, bit for bit:
    automatic and fixed partitions of the own tokens (short tails: one
    workgroup per sequence and kv-head; long ones: balanced shares)."""
    prefix = 96
    lens = [prefix + x for x in own]
    w = workloads.make_custom(500 + G + bs + len(own), lens, G * 2, 2, D, bs, kv_dtype=kv, prefix=prefix,
                              prefix_group_size=3)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    ref = a.step_cascade(partition_tokens=spt)
    got = b.step_cascade(fused=True, partition_tokens=spt)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), "outputs differ"
    for x, y in zip(_cache_bytes(a), _cache_bytes(b)):
        assert np.array_equal(x, y), "caches differ"
    assert_parity(got, oracle_out(w), kv, f"fused cascade step {kv} G={G} bs={bs} spt={spt}")


@pytest.mark.parametrize("kv", ["bf16", "i8", "fp8", "e5m2"])
@pytest.mark.parametrize("G,D,bs,group", [(4, 128, 16, 3), (1, 64, 32, None), (8, 128, 16, 5)])
def test_cascade_many_short_tails(kv, G, D, bs, group):
    """Many sequences with short own tails past a shared prefix (1024
    (sequence, kv-head) units, tails of 1 .. 400 tokens): against the
    oracle, and the fused step equals kv_cache_write followed by the
    cascade, bit for bit."""
    prefix, Hkv, B = 96, 8, 128
    tails = [1, 2, 15, 16, 17, 33, 100, 255, 400, 7, 64]
    lens = [prefix + tails[i % len(tails)] for i in range(B)]
    w = workloads.make_custom(900 + G + bs, lens, G * Hkv, Hkv, D, bs, kv_dtype=kv, prefix=prefix,
                              prefix_group_size=group)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    ref = a.step_cascade()
    got = b.step_cascade(fused=True)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), "outputs differ"
    for x, y in zip(_cache_bytes(a), _cache_bytes(b)):
        assert np.array_equal(x, y), "caches differ"
    samples = sample_pairs(w, n=32, seed=G + bs)
    ref_o = oracle_out(w, samples=samples)
    for bb, h in samples:
        assert_parity(got[bb, h], ref_o[bb, h], kv, f"short tails {kv} G={G} bs={bs} (b={bb}, h={h})")


def test_cascade_equals_plain_decode_within_rounding():
    w = workloads.make_custom(42, [500 + x for x in RAGGED], 32, 8, 128, 16, prefix=500)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    got = a.step_cascade()
    ref = b.step()
    # both are fp32-accumulated sums of the same terms in different orders,
    # rounded to bf16: at most one bf16 unit apart (plus fp32 noise)
    bound = 2.0 ** -7 * np.maximum(np.abs(got), np.abs(ref)) + 1e-5
    assert np.all(np.abs(got - ref) <= bound)


def test_cascade_without_sharing_and_empty_contexts():
    # no prefix: every sequence is its own group with nothing shared (the
    # prefix kernel is not launched); L = 0 gives zeros
    w = workloads.make_custom(7, [0, 5, 17, 40, 1, 300], 8, 2, 64, 16)
    dw = DeviceWorkload(w)
    got = dw.step_cascade()
    gs, gsb, mg, ms = dw.groups
    assert ms == 0 and mg == 1
    assert np.all(got[0] == 0)
    assert_parity(got, oracle_out(w), "bf16", "cascade without sharing")


def test_cascade_min_shared_blocks_leaves_short_prefixes_to_plain_path():
    w = workloads.make_custom(8, [40 + x for x in RAGGED], 8, 2, 64, 16, prefix=40)
    dw = DeviceWorkload(w)
    got = dw.step_cascade()  # 2 shared blocks
    got_plain_groups = DeviceWorkload(w).step_cascade(min_shared_blocks=3)  # no group qualifies
    ref = oracle_out(w)
    assert_parity(got, ref, "bf16", "cascade, 2 shared blocks")
    assert_parity(got_plain_groups, ref, "bf16", "cascade, no groups")


@pytest.mark.parametrize("bs", [16, 32])
def test_cascade_shared_prefix_workload_full_size(bs):
    w = workloads.make_config(4, 0, bs)
    dw = DeviceWorkload(w)
    got = dw.step_cascade()
    gs, gsb, mg, ms = dw.groups
    assert len(gsb) == 1 and mg == 256 and ms == (125 if bs == 16 else 62)
    samples = sample_pairs(w, n=8, seed=bs)
    ref = oracle_out(w, samples=samples)
    for b, h in samples:
        assert_parity(got[b, h], ref[b, h], "bf16", f"prefix bs={bs} (b={b}, h={h})")


def test_cascade_graph_replays_match_eager():
    """The cascade call forks its prefix kernel onto the library's second
    stream and joins it back by events; captured in a graph, every replay
    (new queries copied in eagerly, synchronised between replays) equals an
    eager call on the same inputs bit for bit."""
    import torch
    from gpu_helpers import DEV, out_f64
    import paged_kv_cache_29_amd as pkv
    from paged_kv_cache_29_amd import blocks

    w = workloads.make_custom(77, [300 + x for x in RAGGED], 16, 2, 128, 16, prefix=300)
    dw = DeviceWorkload(w)
    dw.step_cascade()                                   # cache written; side stream created
    gs, gsb, mg, ms = blocks.cascade_groups(w.block_tables, w.context_lens, w.block_size)
    gs_d, gsb_d = torch.from_numpy(gs).to(DEV), torch.from_numpy(gsb).to(DEV)
    need = pkv.cascade_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                      w.block_size, w.block_tables.shape[1], len(gsb), mg, ms)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    q = dw.q.clone()
    out = torch.empty_like(q)

    def call(o):
        pkv.paged_attention_decode_cascade(o, q, dw.k_cache, dw.v_cache, dw.block_tables,
                                           dw.context_lens, gs_d, gsb_d, w.scale, w.num_heads,
                                           w.num_kv_heads, w.head_dim, w.block_size, mg, ms,
                                           workspace=ws)

    call(out)                                           # warm, outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    gen = torch.Generator(device="cpu").manual_seed(5)
    for i in range(3):
        q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_f64(out)
        ref = torch.empty_like(q)
        call(ref)
        torch.cuda.synchronize()
        assert np.array_equal(got, out_f64(ref)), f"replay {i} differs from the eager call"
