#!/usr/bin/env python3
"""Decode-step benchmark for paged KV-cache attention on one MI355X.

One step = the hot path once over one batch: write each sequence's new
token into its tail-block slot, then attend every sequence's new query over
its whole paged context.  It is timed through the fused entry point, one
call per step (paged_attention_decode_step: the partition kernel appends
the token and attends, then the split-context reduce runs when a context
spans several partitions), and again as two calls (kv_cache_write or the
quantising write, then paged_attention_decode), reported under
``unfused``.  Inputs are seeded synthetic data already resident in HBM.

Prints ONE JSON line.  ``value`` is the KV bytes a step must read divided by
the measured step time (GB/s) on the 7B-shaped MHA workload (batch 32,
2048-token contexts, 32 heads x 128 dims, bf16, 16-token blocks).  Every
other workload is reported under ``secondary``, one entry each: the
70B-shaped GQA workloads (bf16; int8, FP8 E4M3, FP8 E5M2 and INT4 KV), the
shared-prefix workload at block size 16 and at 32 (with its cascade-decode
leg), and the tiny fp32 workload (microseconds only).  Per-kernel times come
from HIP events recorded on the stream the kernels run on: each kernel is
also run alone, back to back, and its average duration is the roofline's
time.  Every workload carries ``cpu_baseline``: the oracle on the host's
cores over a bounded sample of the same workload.

Before each workload's warm-up steps the step also runs, untimed, for
--settle-seconds (0.3 s): the GPU's clocks drop while the host builds a
workload, and the first timed loop would otherwise measure their ramp.

Options: --steps K --warmup W (timed / untimed steps), --gpus N (only 1),
--configs (which workloads: ids, with @bs for the shared-prefix workload's
block size), --partition-tokens, --cpu-seconds / --cpu-seconds-secondary
(bound of the CPU oracle baseline of the headline / of each other workload;
0 disables it), --copy-calibration (only run a 1 GiB device copy, for
scaling rocprofv3 byte counters), --counter-pass (per workload only fill
the cache and run the fused step warm-up + steps times, so that a counter
run's partition-kernel dispatches are all fused steps).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "paged decode-attn KV read GB/s (% of HBM peak) + µs/step, 7B & 70B shapes"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
KERNEL_SOURCES = ["decode_mfma.hip", "decode_tile.hpp", "decode_append.hpp", "pkv_device.hpp",
                  "pkv_kernels.hpp", "prefix_body.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_traffic.txt")
CODED = ("i8", "fp8", "e5m2", "i4")  # caches of codes with per-(token, kv-head) scales
CODE_BYTES = {"i8": 1.0, "fp8": 1.0, "e5m2": 1.0, "i4": 0.5, "bf16": 2.0, "f32": 4.0}  # per element
DEFAULT_CONFIGS = "2,3,5,6,7,8,4@16,4@32,1"

DESCRIPTIONS = {
    1: "tiny_f32: B=4 L={47,200,16,1} H=Hkv=4 D=64 bs=16 fp32",
    2: "mha7b_bf16: B=32 L=2048 H=Hkv=32 D=128 bs=16 bf16",
    3: "gqa70b_bf16: B=50 L~logU[1024,32768] H=64 Hkv=8 D=128 bs=16 bf16",
    4: "prefix_bf16: B=256 shared 2000-token prefix + U{50..500} H=32 Hkv=8 D=128",
    5: "int8_gqa70b: B=64 L=8192 H=64 Hkv=8 D=128 bs=16 int8 KV, bf16 q",
    6: "fp8_gqa70b: B=64 L=8192 H=64 Hkv=8 D=128 bs=16 FP8 E4M3 KV, bf16 q",
    7: "int4_gqa70b: B=64 L=8192 H=64 Hkv=8 D=128 bs=16 INT4 KV, bf16 q",
    8: "e5m2_gqa70b: B=64 L=8192 H=64 Hkv=8 D=128 bs=16 FP8 E5M2 KV, bf16 q",
}


def code_only(text):
    """C++ source without its comments and blank lines, so that a comment
    edit does not read as a kernel change (string literals in these sources
    hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_sha():
    """Hash of the partition kernel's sources (code only, comments dropped)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_29_amd", "csrc", f)) as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload_name):
    """HBM bytes per launch of the partition kernel from the committed counter
    summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = kernel_source_sha()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            m = re.match(r"^TRAFFIC\s+(\S+)\s+(\S+)\s+(\d+)\s+(\d+)\s*$", line.strip())
            if m and m.group(1) == workload_name and m.group(2) == sha:
                return int(m.group(3)) + int(m.group(4))
    return None


def kv_bytes(w):
    elem = CODE_BYTES[w.kv_dtype]
    scale = 4 if w.kv_dtype in CODED else 0
    return int(2 * w.num_kv_heads * (w.head_dim * elem + scale) * w.attended_tokens)


def torch_kv_dtype(torch, kind):
    """The torch element type of a cache of kind ``kind``."""
    return {"bf16": torch.bfloat16, "i8": torch.int8, "fp8": torch.float8_e4m3fn,
            "e5m2": torch.float8_e5m2, "i4": torch.uint8, "f32": torch.float32}[kind]


def run_workload(cfg, args, torch, pkv, workloads, block_size=None, counter_only=False):
    w = workloads.make_config(cfg, seed=0, block_size=block_size)
    dev = torch.device("cuda:0")
    store = "bf16" if w.kv_dtype == "bf16" else "f32"

    def up(a, kind):
        import numpy as np
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if kind == "bf16" else torch.from_numpy(a)
        return t.to(dev)

    q = up(w.q, w.q_dtype)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    slot = torch.from_numpy(w.slot_new).to(dev)
    k_new, v_new = up(w.k_new, store), up(w.v_new, store)
    ks = vs = None
    write_codes = {"fp8": pkv.kv_cache_write_fp8, "e5m2": pkv.kv_cache_write_fp8_e5m2,
                   "i4": pkv.kv_cache_write_int4}.get(w.kv_dtype, pkv.kv_cache_write_int8)
    if w.kv_dtype in CODED:
        NB, Hkv, bs, D = w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim
        cd = {"fp8": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2,
              "i4": torch.uint8}.get(w.kv_dtype, torch.int8)
        Dw = D // 2 if w.kv_dtype == "i4" else D   # INT4: two dims per byte
        kc = torch.zeros((NB, Hkv, bs, Dw), dtype=torch.uint8, device=dev).view(cd)
        vc = torch.zeros((NB, Hkv, bs // 4, Dw, 4), dtype=torch.uint8, device=dev).view(cd)
        ks = torch.zeros((NB, Hkv, bs), dtype=torch.float32, device=dev)
        vs = torch.zeros((NB, Hkv, bs), dtype=torch.float32, device=dev)
        kf, vf, sf = up(w.k_fill, "f32"), up(w.v_fill, "f32"), torch.from_numpy(w.slot_fill).to(dev)
        write_codes(kf, vf, kc, vc, ks, vs, sf)   # fill the cache once
        torch.cuda.synchronize()
        # the same fill again, timed: the quantising write at bulk size
        fill = None if counter_only else time_fill(
            torch, lambda: write_codes(kf, vf, kc, vc, ks, vs, sf), read_bytes=2 * kf.numel() * 4,
            write_bytes=int(2 * kf.shape[0] * Hkv * (D * CODE_BYTES[w.kv_dtype] + 4)), tokens=kf.shape[0])
        del kf, vf, sf
    else:
        kc, vc = up(w.k_cache, store), up(w.v_cache, store)
        fill = None
        if w.name == "mha7b_bf16" and not counter_only:
            fill = bulk_fill_bf16(torch, pkv, w, kc, vc)
    out = torch.empty_like(q)
    pt = args.partition_tokens
    need = pkv.workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                              w.block_tables.shape[1], pt)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    dargs = (out, q, kc, vc, bt, cl, w.scale, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size)
    dkw = dict(k_scale=ks, v_scale=vs, partition_tokens=pt, workspace=ws)

    def write():
        if w.kv_dtype in CODED:
            write_codes(k_new, v_new, kc, vc, ks, vs, slot)
        else:
            pkv.kv_cache_write(k_new, v_new, kc, vc, slot)

    sargs = (out, q, k_new, v_new, kc, vc, bt, cl, w.scale, w.num_heads, w.num_kv_heads,
             w.head_dim, w.block_size)

    def step_fused():
        # one step, one call: append the new tokens and attend (the
        # partition kernel, then the reduce when a context was split)
        pkv.paged_attention_decode_step(*sargs, **dkw)

    def step_unfused():
        # the same step as the cache write, then decode (partitions + reduce)
        write()
        pkv.paged_attention_decode(*dargs, **dkw)

    def loop_time(fn):
        """Average duration of fn over K back-to-back launches (events on the launch stream)."""
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps * 1e3  # us

    def graph_time(fn, per_graph=20):
        """Average duration of fn replayed from a HIP graph of per_graph
        back-to-back calls (events on the replay stream): the step without
        the host's per-call cost (the binding's argument marshalling), as a
        serving loop that captures its decode step would run it."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        reps = max(2, (args.steps + per_graph - 1) // per_graph)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (reps * per_graph) * 1e3
        del g
        return us

    def per_step(fn):
        """Per-step durations: one event between consecutive steps."""
        n = max(args.steps, 2)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        evs[0].record()
        for i in range(n):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        d = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
        q = lambda f: d[min(n - 1, int(round(f * (n - 1))))]
        return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9)}

    # Clocks drop while the host builds a workload; run untimed steps for a
    # while so the first timed loop does not measure the ramp back up.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(10):
            step_fused()
        torch.cuda.synchronize()

    if counter_only:
        # the fused step alone, warm-up + timed count, for counter runs: the
        # partition kernel's dispatches are then all fused-step launches
        for _ in range(args.warmup + args.steps):
            step_fused()
        torch.cuda.synchronize()
        return {"config": cfg, "name": w.name, "fused_steps": args.warmup + args.steps,
                "algorithmic_bytes": unique_tile_bytes(w) if w.meta.get("prefix") else kv_bytes(w)}

    ms_per_step = loop_time(step_fused) / 1e3
    ms_u = loop_time(step_unfused) / 1e3
    # the partition kernels alone, back to back (every launch is idempotent:
    # the append and the cache write store the same token to the same slot).
    # The few-microsecond kernels (reduce, cache write) are given as their
    # share of the step: looped alone they would time the host's launch rate.
    part_avg = loop_time(lambda: pkv.paged_attention_decode_step_partitions(*sargs, **dkw))
    part_u_us = loop_time(lambda: pkv.paged_attention_decode_partitions(*dargs, **dkw))
    red_us = max(0.0, ms_per_step * 1e3 - part_avg)
    write_us = max(0.0, ms_u * 1e3 - part_u_us - red_us)
    dist = per_step(step_fused)
    us_graph = graph_time(step_fused)
    nbytes = kv_bytes(w)
    uniq = unique_tile_bytes(w)
    res = {
        "workload": DESCRIPTIONS[cfg] + (f" bs={block_size}" if block_size else ""),
        "name": w.name,
        "kv_bytes_per_step": nbytes,
        "attended_tokens": w.attended_tokens,
        "us_per_step": ms_per_step * 1e3,
        "kv_gbs": nbytes / (ms_per_step * 1e-3) / 1e9,
        "pct_hbm_peak": 100.0 * nbytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "tokens_per_s": w.attended_tokens / (ms_per_step * 1e-3),
        "us_per_step_events": dist,
        "us_per_step_graph": us_graph,
        "kernel_us": {"decode_step_partitions": part_avg, "decode_reduce_share": red_us},
        "unfused": {"us_per_step": ms_u * 1e3,
                    "kv_gbs": nbytes / (ms_u * 1e-3) / 1e9,
                    "kernel_us": {"kv_cache_write_share": write_us, "decode_partitions": part_u_us,
                                  "decode_reduce_share": red_us}},
        "unique_tile_bytes": uniq,
        "unique_gbs": uniq / (ms_per_step * 1e-3) / 1e9,
        "partition_tokens": pkv.partition_tokens(w.num_seqs, w.num_kv_heads, w.block_size,
                                                 w.block_tables.shape[1], pt),
    }
    # Roofline of the step's dominant kernel, the partition kernel of the
    # fused step, timed alone (back-to-back launches).  Its algorithmic
    # bytes are the KV bytes a step must read; with shared blocks (the
    # prefix workload) those are the distinct tiles, which is all HBM has
    # to deliver; the logical bytes are reported beside it.
    shared = bool(w.meta.get("prefix"))
    alg = uniq if shared else nbytes
    achieved = alg / (part_avg * 1e-6) / 1e9
    res["roofline"] = {"bound": "latency" if w.kv_dtype == "f32" else "hbm",
                       "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": read_traffic(w.name),
                       "kernel": "decode_mfma_kernel (fused step: append + attend)"
                       if w.kv_dtype != "f32" else "decode_f32_kernel (fused step)",
                       "basis": ("unique tile bytes" if shared else "KV bytes")
                       + " / partition-kernel time (the kernel alone, back-to-back launches)",
                       "step_frac": alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if shared:
        res["roofline"]["logical_gbs"] = nbytes / (part_avg * 1e-6) / 1e9
        res["pct_hbm_peak"] = 100.0 * uniq / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
        res["pct_hbm_peak_basis"] = "unique tile bytes"
    if w.kv_dtype == "f32":
        res["roofline"]["note"] = ("the whole workload (540 KB of KV) stays in the caches: the step "
                                   "is bound by launch and dependent-load latency, so only us/step counts")

    res["roofline"]["load_policy"] = "non-temporal" if pkv.streams_cache(
        w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, torch_kv_dtype(torch, w.kv_dtype)) else "default"
    res["shares"] = pkv.balanced_shares(w.num_seqs, w.num_kv_heads, w.block_size,
                                        w.block_tables.shape[1], torch_kv_dtype(torch, w.kv_dtype), pt) \
        if w.kv_dtype != "f32" else 0
    if w.name == "gqa70b_bf16":
        res["speculative_verify"] = run_multi_query(w, args, torch, pkv, loop_time, q, kc, vc, bt, cl,
                                                    nbytes, ms_per_step)
    if w.meta.get("prefix"):
        res["cascade"] = run_cascade(w, args, torch, pkv, loop_time, write, out, q, kc, vc, bt, cl,
                                     ks, vs, nbytes, uniq, ms_per_step, k_new, v_new)
    res["bulk_fill"] = fill
    res["_w"] = w
    return res


def time_fill(torch, fn, read_bytes, write_bytes, tokens, iters=5):
    """Average duration of a bulk cache write (HIP events on the launch
    stream) and its rate over the bytes it must read and write."""
    fn()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(iters):
        fn()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / iters * 1e3
    return {"tokens": int(tokens), "us": us, "read_bytes": int(read_bytes), "write_bytes": int(write_bytes),
            "gbs_read_plus_write": (read_bytes + write_bytes) / (us * 1e-6) / 1e9}


def bulk_fill_bf16(torch, pkv, w, kc, vc):
    """kv_cache_write of every cached token of the workload at once (a
    prefill: each sequence's tokens in order, so consecutive tokens fill
    consecutive rows of a block), from random bf16 rows; the cache is
    rewritten with the values it is re-read with only after the timing."""
    import numpy as np
    bs = w.block_size
    slots = []
    for b, L in enumerate(w.context_lens):
        pos = np.arange(int(L), dtype=np.int64)
        slots.append(w.block_tables[b][pos // bs].astype(np.int64) * bs + pos % bs)
    slot = torch.from_numpy(np.concatenate(slots)).to("cuda:0")
    T, Hkv, D = slot.numel(), w.num_kv_heads, w.head_dim
    k = torch.randn((T, Hkv, D), dtype=torch.bfloat16, device="cuda:0")
    v = torch.randn((T, Hkv, D), dtype=torch.bfloat16, device="cuda:0")
    k0, v0 = kc.clone(), vc.clone()
    res = time_fill(torch, lambda: pkv.kv_cache_write(k, v, kc, vc, slot),
                    read_bytes=2 * k.numel() * 2, write_bytes=2 * k.numel() * 2, tokens=T)
    kc.copy_(k0)
    vc.copy_(v0)
    torch.cuda.synchronize()
    return res


def run_multi_query(w, args, torch, pkv, loop_time, q, kc, vc, bt, cl, nbytes, ms_decode, n=5):
    """A speculative-decoding verification on the same contexts: the last
    n = k + 1 tokens of every sequence scored in one call (causal), timed
    like the decode step; the pages' point is that when decode is
    memory-bound this costs about as much as one decode step."""
    import numpy as np
    dev = q.device
    B = w.num_seqs
    qs = torch.from_numpy((np.arange(B + 1) * n).astype(np.int32)).to(dev)
    qm = q.repeat_interleave(n, dim=0).contiguous()
    om = torch.empty_like(qm)
    need = pkv.multi_query_workspace_size(B, B * n, n, w.num_heads, w.num_kv_heads, w.head_dim,
                                          w.block_size, w.block_tables.shape[1], 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def verify():
        pkv.paged_attention_multi_query(om, qm, kc, vc, bt, cl, qs, w.scale, w.num_heads,
                                        w.num_kv_heads, w.head_dim, w.block_size, n, workspace=ws)

    us = loop_time(verify)
    return {"tokens_per_seq": n, "us_per_call": us, "kv_gbs": nbytes / (us * 1e-6) / 1e9,
            "cost_vs_one_token_step": us / (ms_decode * 1e3),
            "query_tokens_per_s": B * n / (us * 1e-6)}


def run_cascade(w, args, torch, pkv, loop_time, write, out, q, kc, vc, bt, cl, ks, vs, nbytes,
                uniq, ms_fused, k_new, v_new):
    """The same step with the shared blocks attended once per group: the
    fused cascade step (one launch attends the shared blocks once per group
    and each sequence's own tokens, writing its new token first; then the
    reduce), and for reference the cache write followed by the plain cascade
    call."""
    from paged_kv_cache_29_amd import blocks
    gs, gsb, mg, msb = blocks.cascade_groups(w.block_tables, w.context_lens, w.block_size)
    dev = q.device
    gs_d, gsb_d = torch.from_numpy(gs).to(dev), torch.from_numpy(gsb).to(dev)
    need = pkv.cascade_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                      w.block_size, w.block_tables.shape[1], len(gsb), mg, msb,
                                      args.partition_tokens, 0)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def cascade(fused=False):
        pkv.paged_attention_decode_cascade(out, q, kc, vc, bt, cl, gs_d, gsb_d, w.scale,
                                           w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                           mg, msb, k_scale=ks, v_scale=vs,
                                           partition_tokens=args.partition_tokens, workspace=ws,
                                           k_new=k_new if fused else None, v_new=v_new if fused else None)

    def unfused():
        write()
        cascade()

    us = loop_time(lambda: cascade(True))
    us_unfused = loop_time(unfused)
    us_attn = loop_time(cascade)
    return {"us_per_step": us, "us_per_step_write_then_cascade": us_unfused,
            "logical_kv_gbs": nbytes / (us * 1e-6) / 1e9,
            "unique_gbs": uniq / (us * 1e-6) / 1e9,
            "frac_hbm_unique": uniq / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "attention_us": us_attn,
            "speedup_vs_fused_step": ms_fused * 1e3 / us,
            "groups": int(len(gsb)), "max_group_size": int(mg), "shared_blocks": int(msb)}


def unique_tile_bytes(w):
    """K and V bytes of the distinct (block, kv-head) tiles the step touches:
    what a step must read at least when shared blocks are read once."""
    import numpy as np
    bs = w.block_size
    ids = set()
    for b, L in enumerate(w.context_lens):
        n = (int(L) + bs - 1) // bs
        ids.update(int(x) for x in w.block_tables[b, :n])
    elem = CODE_BYTES[w.kv_dtype]
    scale = 4 if w.kv_dtype in CODED else 0
    return int(len(ids) * 2 * w.num_kv_heads * bs * (w.head_dim * elem + scale))


def read_ceiling(torch, pkv, steps=20):
    """The device's read rate for the decode kernel's access pattern: 2 GiB
    of 4 KB tiles gathered in a shuffled order by the tile-read probe (run
    after the workloads, so the clocks are up; ids range-checked once), with
    the default load policy (``gbs``) and with the non-temporal hint that
    decode takes over a large pool (``gbs_non_temporal``)."""
    import numpy as np
    n = 2 << 30
    pool = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    ids = torch.from_numpy(np.random.default_rng(0).permutation(n // 4096).astype(np.int32)).to("cuda:0")
    pkv.probe_tile_read(pool, ids, torch.empty(256, dtype=torch.int32, device="cuda:0"), 1, check_ids=True)
    out = {}
    for streaming in (False, True):
        best = None
        for grid in (2048, 4096, 8192):
            sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda:0")
            for _ in range(3):
                pkv.probe_tile_read(pool, ids, sink, grid, check_ids=False, streaming=streaming)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                pkv.probe_tile_read(pool, ids, sink, grid, check_ids=False, streaming=streaming)
            t1.record()
            torch.cuda.synchronize()
            gbs = n / (t0.elapsed_time(t1) / steps * 1e-3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, grid)
        key = "non_temporal" if streaming else ""
        out["gbs" + ("_" + key if key else "")] = best[0]
        out["grid" + ("_" + key if key else "")] = best[1]
    del pool, ids
    torch.cuda.empty_cache()
    out["probe"] = "pkv_probe_tile_read: 2 GiB of shuffled 4 KB tiles, best grid, each load policy"
    return out


def block_moves(torch, pkv, steps=10):
    """Whole-block copies of a 70B-shaped pool (8 kv-heads x 16 tokens x 128
    dims, bf16: 64 KB of K + V per block): copy-on-write copies inside HBM,
    and swapping blocks out to pinned host memory and back."""
    import numpy as np
    dev = torch.device("cuda:0")
    Hkv, bs, D, NB, NH, n = 8, 16, 128, 12288, 4096, 4096
    kc = torch.empty((NB, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((NB, Hkv, bs // 4, D, 4), dtype=torch.bfloat16, device=dev)
    hk = torch.empty((NH, Hkv, bs, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((NH, Hkv, bs // 4, D, 4), dtype=torch.bfloat16).pin_memory()
    rng = np.random.default_rng(0)
    perm = rng.permutation(NB)
    cow = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int32)).to(dev)
    out = torch.from_numpy(np.stack([perm[:n], rng.permutation(NH)[:n]], 1).astype(np.int32)).to(dev)
    back = torch.from_numpy(np.stack([out[:, 1].cpu().numpy(), perm[2 * n:3 * n]], 1).astype(np.int32)).to(dev)
    block_bytes = 2 * Hkv * bs * D * 2

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e-3

    t_cow = timed(lambda: pkv.copy_blocks((kc, vc), (kc, vc), cow))
    t_out = timed(lambda: pkv.copy_blocks((hk, hv), (kc, vc), out))
    t_in = timed(lambda: pkv.copy_blocks((kc, vc), (hk, hv), back))
    moved = n * block_bytes
    res = {"blocks_per_call": n, "block_bytes": block_bytes,
           "copy_on_write": {"us": t_cow * 1e6, "gbs_read_plus_write": 2 * moved / t_cow / 1e9,
                             "frac_of_hbm_peak": 2 * moved / t_cow / 1e9 / HBM_PEAK_GBS},
           "swap_out_gbs": moved / t_out / 1e9, "swap_in_gbs": moved / t_in / 1e9,
           "note": "swap rates are over the host link (PCIe Gen5 x16, 64 GB/s per direction nominal)"}
    del kc, vc, hk, hv
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, seconds, with_writes=False):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole sequences (all heads), in order, repeated until `seconds` of
    oracle decode time have passed.  For a coded cache the oracle first
    quantises each sampled sequence's tokens into its own cache (untimed:
    that is the cache write's oracle, not decode's)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from oracle import cache as ocache
    from oracle import fp8 as ofp8
    from oracle import int4 as oint4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    bs = w.block_size
    ks = vs = None
    if w.kv_dtype in CODED:
        NB, Hkv, D = w.num_blocks, w.num_kv_heads, w.head_dim
        Dw = D // 2 if w.kv_dtype == "i4" else D
        code_t = np.int8 if w.kv_dtype == "i8" else np.uint8
        kc = np.zeros((NB, Hkv, bs, Dw), code_t)   # untouched pages stay unallocated
        vc = np.zeros((NB, Hkv, bs // 4, Dw, 4), code_t)
        ks = np.full((NB, Hkv, bs), np.nan, np.float32)
        vs = np.full((NB, Hkv, bs), np.nan, np.float32)
        write = {"i8": ocache.cache_write_int8, "fp8": ofp8.cache_write_fp8,
                 "e5m2": ofp8.cache_write_fp8_e5m2, "i4": oint4.cache_write_int4}[w.kv_dtype]
        per_seq = w.meta.get("fill_per_sequence", True)
        starts = np.concatenate([[0], np.cumsum(np.maximum(w.context_lens.astype(np.int64) - 1, 0))])
        ready = set()
    else:
        kc, vc = ocache.cache_write(w.k_new, w.v_new, w.k_cache, w.v_cache, w.slot_new, bs)
    done_tokens = 0
    done_seqs = 0
    timed = 0.0
    t_wall = time.perf_counter()
    while timed < seconds and time.perf_counter() - t_wall < 4 * seconds + 30:
        b = done_seqs % w.num_seqs
        if w.kv_dtype in CODED and b not in ready:
            if per_seq:
                a, e = int(starts[b]), int(starts[b + 1])
                kc, vc, ks, vs = write(w.k_fill[a:e], w.v_fill[a:e], kc, vc, ks, vs, w.slot_fill[a:e], bs)
            elif not ready:
                kc, vc, ks, vs = write(w.k_fill, w.v_fill, kc, vc, ks, vs, w.slot_fill, bs)
            kc, vc, ks, vs = write(w.k_new[b:b + 1], w.v_new[b:b + 1], kc, vc, ks, vs, w.slot_new[b:b + 1], bs)
            ready.add(b)
        t0 = time.perf_counter()
        oracle.decode_attention(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.num_heads,
                                w.num_kv_heads, w.head_dim, w.block_size, w.kv_dtype, w.q_dtype,
                                k_scale=ks, v_scale=vs, samples=[(b, h) for h in range(w.num_heads)])
        timed += time.perf_counter() - t0
        done_tokens += int(w.context_lens[b])
        done_seqs += 1
    per_tok = 2 * w.num_kv_heads * (w.head_dim * CODE_BYTES[w.kv_dtype] + (4 if w.kv_dtype in CODED else 0))
    nbytes = per_tok * done_tokens
    res = {"value": nbytes / timed / 1e9 if timed > 0 else None, "unit": "GB/s", "cores": int(threads),
           "kind": "oracle",
           "us_per_step_equiv": timed / max(done_tokens, 1) * w.attended_tokens * 1e6,
           "sample": f"{done_seqs} sequence passes ({done_seqs / w.num_seqs:.2f} x all {w.num_seqs} "
                     f"sequences) x all {w.num_heads} heads ({done_tokens} context tokens) of "
                     f"{w.name}, {timed:.1f} s of oracle decode; "
                     f"cpu_count={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}, "
                     f"blas_threads={threads}"}
    if with_writes:
        res["cache_writes"] = cpu_cache_writes(w)
    return res


def cpu_cache_writes(w, tokens=4096, blocks=512):
    """The cache-write oracles (slot scatter, int8 quantiser) on a bulk write
    of `tokens` rows of the workload's kv-head shape into a pool of `blocks`
    blocks (prefill order): rate over the bytes read and written, as the
    GPU's bulk_fill reports it."""
    import numpy as np
    from oracle import cache as ocache
    rng = np.random.default_rng(0)
    Hkv, D, bs = w.num_kv_heads, w.head_dim, w.block_size
    slots = rng.permutation(blocks)[:tokens // bs].repeat(bs) * bs + np.tile(np.arange(bs), tokens // bs)
    k = rng.standard_normal((tokens, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((tokens, Hkv, D)).astype(np.float32)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)   # bf16 bit patterns (truncated: any
    vb = (v.view(np.uint32) >> 16).astype(np.uint16)   # pattern times the same)
    kc = np.zeros((blocks, Hkv, bs, D), np.uint16)
    vc = np.zeros((blocks, Hkv, bs // 4, D, 4), np.uint16)
    t0 = time.perf_counter()
    ocache.cache_write(kb, vb, kc, vc, slots, bs)
    t_bf16 = time.perf_counter() - t0
    kc8 = np.zeros((blocks, Hkv, bs, D), np.int8)
    vc8 = np.zeros((blocks, Hkv, bs // 4, D, 4), np.int8)
    sc = np.zeros((blocks, Hkv, bs), np.float32)
    t0 = time.perf_counter()
    ocache.cache_write_int8(k, v, kc8, vc8, sc, sc.copy(), slots, bs)
    t_i8 = time.perf_counter() - t0
    n = tokens * Hkv * D
    return {"sample": f"{tokens} tokens x {Hkv} kv-heads x {D} dims into a {blocks}-block pool",
            "kv_cache_write_bf16_gbs": 2 * (2 * n * 2) / t_bf16 / 1e9,
            "kv_cache_write_int8_gbs": (2 * n * 4 + 2 * (n + tokens * Hkv * 4)) / t_i8 / 1e9,
            "seconds": t_bf16 + t_i8}


def copy_calibration(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_dispatch": n,
                      "copy_calibration_bytes_written_per_dispatch": n}))


def parse_configs(spec):
    """'2,3,4@32' -> [(2, None), (3, None), (4, 32)]: workload ids, with the
    shared-prefix workload's block size after '@'."""
    out = []
    for item in spec.split(","):
        item = item.strip()
        if not item:
            continue
        cfg, _, bs = item.partition("@")
        out.append((int(cfg), int(bs) if bs else (16 if int(cfg) == 4 else None)))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="workload ids, the first is the headline; 4@32 = the shared-prefix workload at bs 32")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle time on the headline workload")
    ap.add_argument("--cpu-seconds-secondary", type=float, default=4.0,
                    help="oracle time on each other workload")
    ap.add_argument("--settle-seconds", type=float, default=0.3,
                    help="untimed steps before each workload's first warm-up, so clocks have settled")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="per workload only fill the cache and run warm-up + steps fused steps "
                         "(for rocprofv3 counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no "
              "multi-GPU path; the per-GPU kernel is what is measured.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    sys.path.insert(0, ROOT)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(torch)
        return 0
    import paged_kv_cache_29_amd as pkv
    from paged_kv_cache_29_amd import workloads
    pkv.load_library()
    if args.counter_pass:
        runs = []
        for c, bs in parse_configs(args.configs):
            r = run_workload(c, args, torch, pkv, workloads, bs if c == 4 else None, counter_only=True)
            print(f"[bench] config {c}: counter pass, {r['fused_steps']} fused steps", file=sys.stderr, flush=True)
            runs.append(r)
            torch.cuda.empty_cache()
        print(json.dumps({"counter_pass": runs, "kernel_source_sha": kernel_source_sha()}))
        return 0
    results = []
    for i, (c, bs) in enumerate(parse_configs(args.configs)):
        tag = f"{c}" + (f"@{bs}" if c == 4 else "")
        print(f"[bench] config {tag} ...", file=sys.stderr, flush=True)
        r = run_workload(c, args, torch, pkv, workloads, bs if c == 4 else None)
        r["config_id"] = tag
        print(f"[bench] config {tag}: {r['us_per_step']:.1f} us/step, {r['kv_gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        secs = args.cpu_seconds if i == 0 else args.cpu_seconds_secondary
        w = r.pop("_w")
        if secs > 0:
            print(f"[bench] config {tag}: cpu baseline (oracle) ...", file=sys.stderr, flush=True)
            r["cpu_baseline"] = cpu_baseline(w, secs, with_writes=(i == 0))
        else:
            r["cpu_baseline"] = None
        r["_shape"] = {"num_seqs": w.num_seqs, "context_len": int(w.context_lens.max()),
                       "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                       "block_size": w.block_size, "kv_dtype": w.kv_dtype}
        del w
        results.append(r)
    print("[bench] read ceiling probe ...", file=sys.stderr, flush=True)
    ceiling = read_ceiling(torch, pkv)
    print("[bench] block moves ...", file=sys.stderr, flush=True)
    moves = block_moves(torch, pkv)
    for r in results:
        nt = r["roofline"].get("load_policy") == "non-temporal"
        r["roofline"]["frac_of_read_ceiling"] = r["roofline"]["achieved"] / ceiling[
            "gbs_non_temporal" if nt else "gbs"]
    head = results[0]
    shp = head.pop("_shape")
    for r in results[1:]:
        r.pop("_shape")
    line = {
        "metric": METRIC,
        "value": round(head["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "i8": "i8", "fp8": "fp8_e4m3", "e5m2": "fp8_e5m2", "i4": "i4",
                  "f32": "f32"}[shp["kv_dtype"]],
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled block tables)",
        "config": {"workload": head["workload"], "num_seqs": shp["num_seqs"],
                   "context_len": shp["context_len"], "num_heads": shp["num_heads"],
                   "num_kv_heads": shp["num_kv_heads"], "head_dim": shp["head_dim"],
                   "block_size": shp["block_size"], "partition_tokens": head["partition_tokens"]},
        "us_per_step": head["us_per_step"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "kv_bytes_per_step": head["kv_bytes_per_step"],
        "kernel_us": head["kernel_us"],
        "unfused": head["unfused"],
        "bulk_fill": head.get("bulk_fill"),
        "roofline": head["roofline"],
        "us_per_step_events": head["us_per_step_events"],
        "us_per_step_graph": head["us_per_step_graph"],
        "read_ceiling": ceiling,
        "block_moves": moves,
        "kernel_source_sha": kernel_source_sha(),
        "cpu_baseline": head["cpu_baseline"],
        **({"speculative_verify": head["speculative_verify"]} if "speculative_verify" in head else {}),
        "secondary": results[1:],
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
