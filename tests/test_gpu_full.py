"""GPU: the workloads at full size, in the launch configuration the
benchmark times (automatic partition length), checked on sampled outputs the
oracle computes one by one, plus properties that hold at any size."""

import numpy as np
import pytest
import torch

from paged_kv_cache_29_amd import workloads

from gpu_helpers import DeviceWorkload, assert_parity, bf16_bits_of, oracle_caches, oracle_out

pytestmark = pytest.mark.gpu


def sample_seqs(w, n, seed):
    """Sequences to check whole (every head): the longest and the shortest,
    the first and the last, and random others."""
    rng = np.random.default_rng(1000 + seed)
    lens = w.context_lens
    seqs = {int(np.argmax(lens)), int(np.argmin(lens)), 0, w.num_seqs - 1}
    while len(seqs) < min(n, w.num_seqs):
        seqs.add(int(rng.integers(w.num_seqs)))
    return sorted(seqs)


CONFIGS = [(1, None), (2, None), (3, None), (4, 16), (4, 32), (5, None), (6, None), (7, None), (8, None)]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cfg,bs", CONFIGS)
def test_full_size_sampled(cfg, bs, seed):
    _full_size(cfg, bs, seed, fused=False)


@pytest.mark.parametrize("cfg,bs", CONFIGS)
def test_full_size_fused_step_sampled(cfg, bs):
    """The fused step (the call the benchmark times: the partition kernel
    appends each new token, then attends) at full size, seed 0."""
    _full_size(cfg, bs, 0, fused=True)


def _full_size(cfg, bs, seed, fused):
    w = workloads.make_config(cfg, seed, block_size=bs)
    print(f"\n[full] config {cfg} seed {seed} bs={w.block_size} B={w.num_seqs} H={w.num_heads} "
          f"Hkv={w.num_kv_heads} tokens={w.attended_tokens} fused={fused}", flush=True)
    dw = DeviceWorkload(w)
    got = dw.step_fused() if fused else dw.step()
    assert np.all(np.isfinite(got))
    # every head of the sampled sequences (the oracle gathers each
    # (sequence, kv-head)'s K/V once and serves all its heads from it)
    seqs = sample_seqs(w, 5, seed) if cfg != 1 else list(range(w.num_seqs))
    samples = [(b, h) for b in seqs for h in range(w.num_heads)]
    caches = oracle_caches(w, seqs)
    ref = oracle_out(w, samples=samples, caches=caches)
    kind = w.kv_dtype
    for b in seqs:
        assert_parity(got[b], ref[b], kind, f"config {cfg} seed {seed} fused={fused} (b={b}, all heads)")
    # the step's cache write landed bit-exactly in every sampled sequence's tail slot
    bs_ = w.block_size
    for b in seqs:
        s = int(w.slot_new[b])
        blk, r = s // bs_, s % bs_
        if kind == "bf16":
            assert np.array_equal(bf16_bits_of(dw.k_cache[blk, :, r, :]), caches[0][blk, :, r, :])
            assert np.array_equal(bf16_bits_of(dw.v_cache[blk, :, r // 4, :, r % 4]), caches[1][blk, :, r // 4, :, r % 4])
        elif kind in ("i8", "fp8", "e5m2", "i4"):
            for j in range(int(np.ceil(w.context_lens[b] / bs_))):
                pb = int(w.block_tables[b][j])
                assert np.array_equal(dw.k_cache[pb].view(torch.uint8).cpu().numpy(),
                                      caches[0][pb].view(np.uint8))
                assert np.array_equal(dw.v_cache[pb].view(torch.uint8).cpu().numpy(),
                                      caches[1][pb].view(np.uint8))
                rows = min(bs_, int(w.context_lens[b]) - j * bs_)
                assert np.array_equal(dw.k_scale[pb, :, :rows].cpu().numpy(), caches[2][pb, :, :rows])
                assert np.array_equal(dw.v_scale[pb, :, :rows].cpu().numpy(), caches[3][pb, :, :rows])
    torch.cuda.synchronize()
