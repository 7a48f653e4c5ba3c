"""Child process of test_gpu_debug_mode.py: runs with PKV_DEBUG=1 set before
the library is loaded (the flag is read once per process).

Valid calls must give the oracle's results; two invalid calls must be
rejected before anything is launched.  Both invalid inputs stay inside the
pool (a slot used twice; a group member whose shared table entry names
another valid block), so even a launch would read and write only valid
memory.
"""

import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from oracle import cache as ocache  # noqa: E402
import paged_kv_cache_29_amd as pkv  # noqa: E402
from paged_kv_cache_29_amd import blocks, workloads  # noqa: E402

from gpu_helpers import DEV, assert_parity, bf16_bits_of, out_f64, to_dev  # noqa: E402


def expect_rejected(fn, frag):
    try:
        fn()
    except ValueError as e:
        assert frag in str(e), str(e)
        return
    raise AssertionError(f"not rejected: {frag}")


def main():
    assert os.environ.get("PKV_DEBUG") == "1"
    bs, NB, Hkv, G, D = 16, 64, 2, 4, 128
    H = G * Hkv
    scale = 1 / np.sqrt(D)
    rng = np.random.default_rng(11)
    bm = pkv.BlockManager(NB, bs, order=rng.permutation(NB))
    kc_np = np.zeros((NB, Hkv, bs, D), np.uint16)
    vc_np = np.zeros((NB, Hkv, bs // 4, D, 4), np.uint16)
    kc, vc = to_dev(kc_np, "bf16"), to_dev(vc_np, "bf16")

    def rows(n):
        return workloads.bf16_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32))

    def write(seq_slots, copies):
        nonlocal kc_np, vc_np
        for src, dst, nrows in copies:
            pkv.copy_blocks((kc, vc), (kc, vc), torch.tensor([[src, dst]], dtype=torch.int32, device=DEV))
            kc_np[dst, :, :nrows] = kc_np[src, :, :nrows]
            for r in range(nrows):
                vc_np[dst, :, r // 4, :, r % 4] = vc_np[src, :, r // 4, :, r % 4]
        k, v = rows(len(seq_slots)), rows(len(seq_slots))
        pkv.kv_cache_write(to_dev(k, "bf16"), to_dev(v, "bf16"), kc, vc, torch.from_numpy(seq_slots).to(DEV))
        kc_np, vc_np = ocache.cache_write(k, v, kc_np, vc_np, seq_slots, bs)

    root = bm.new_sequence()
    write(*bm.append(root, 3 * bs + 5))
    seqs = [root] + [bm.fork(root) for _ in range(3)]
    for n in (bs - 3, 2 * bs + 7):
        s = bm.new_sequence()
        write(*bm.append(s, n))
        seqs.append(s)
    slots, copies = [], []
    for s in seqs:
        sl, cp = bm.append(s, 1)
        slots.append(sl[0])
        copies += cp
    slots = np.array(slots, np.int64)
    write(slots, copies)
    torch.cuda.synchronize()
    print("valid writes accepted", flush=True)

    # a slot used twice: rejected, the pool untouched
    before = (bf16_bits_of(kc), bf16_bits_of(vc))
    dup = slots.copy()
    dup[1] = dup[0]
    z = torch.zeros((len(dup), Hkv, D), dtype=torch.bfloat16, device=DEV)
    expect_rejected(lambda: pkv.kv_cache_write(z, z, kc, vc, torch.from_numpy(dup).to(DEV)),
                    "tokens 0 and 1 share slot")
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_of(kc), before[0]) and np.array_equal(bf16_bits_of(vc), before[1])
    print("shared slot rejected, pool unchanged", flush=True)

    lens = np.array([bm.length(s) for s in seqs], np.int32)
    B = len(seqs)
    MB = int(max((L + bs - 1) // bs for L in lens))
    tables = bm.tables(seqs, MB)
    bt, cl = torch.from_numpy(tables).to(DEV), torch.from_numpy(lens).to(DEV)
    q = workloads.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32))
    ref = oracle.decode_attention(q, kc_np, vc_np, tables, lens, scale, H, Hkv, D, bs, "bf16", "bf16")

    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=DEV)
    pkv.paged_attention_decode(out, to_dev(q, "bf16"), kc, vc, bt, cl, scale, H, Hkv, D, bs)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, "bf16", "decode under PKV_DEBUG")
    print("decode parity", flush=True)

    gs, gsb, mg, ms = blocks.cascade_groups(tables, lens, bs)
    assert mg == 4 and ms >= 3
    gs_d, gsb_d = torch.from_numpy(gs).to(DEV), torch.from_numpy(gsb).to(DEV)
    out.zero_()
    pkv.paged_attention_decode_cascade(out, to_dev(q, "bf16"), kc, vc, bt, cl, gs_d, gsb_d,
                                       scale, H, Hkv, D, bs, mg, ms)
    torch.cuda.synchronize()
    assert_parity(out_f64(out), ref, "bf16", "cascade under PKV_DEBUG")
    # member 2's first shared entry names another sequence's (valid) block
    bad = tables.copy()
    bad[2, 0] = tables[4, 0]
    expect_rejected(lambda: pkv.paged_attention_decode_cascade(
        out, to_dev(q, "bf16"), kc, vc, torch.from_numpy(bad).to(DEV), cl, gs_d, gsb_d,
        scale, H, Hkv, D, bs, mg, ms), "sequence 2 of group 0")
    print("cascade parity; differing member rejected", flush=True)
    # the fused step: a member whose new token would land inside its
    # group's shared span (context ending exactly at it) is rejected
    bad_lens = lens.copy()
    bad_lens[1] = 3 * bs
    kz = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device=DEV)
    expect_rejected(lambda: pkv.paged_attention_decode_cascade(
        out, to_dev(q, "bf16"), kc, vc, bt, torch.from_numpy(bad_lens).to(DEV), gs_d, gsb_d,
        scale, H, Hkv, D, bs, mg, ms, k_new=kz, v_new=kz), "shared span")
    print("fused cascade step into a shared span rejected", flush=True)

    n_per = np.minimum(3, lens)
    qs = np.concatenate([[0], np.cumsum(n_per)]).astype(np.int32)
    T = int(qs[-1])
    qm = workloads.bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    om = torch.empty((T, H, D), dtype=torch.bfloat16, device=DEV)
    pkv.paged_attention_multi_query(om, to_dev(qm, "bf16"), kc, vc, bt, cl, torch.from_numpy(qs).to(DEV),
                                    scale, H, Hkv, D, bs, 3)
    torch.cuda.synchronize()
    refm = oracle.multi_query_attention(qm, kc_np, vc_np, tables, lens, qs, scale, H, Hkv, D, bs, "bf16", "bf16")
    assert_parity(out_f64(om), refm, "bf16", "multi-query under PKV_DEBUG")
    print("multi-query parity", flush=True)
    print("PKV_DEBUG child: all passed", flush=True)


if __name__ == "__main__":
    main()
