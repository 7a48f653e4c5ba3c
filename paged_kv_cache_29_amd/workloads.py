"""Seeded synthetic inputs for paged decode attention.

This module builds inputs only: it draws values, lays out block tables with
the host block allocator, and poisons memory that no valid token occupies.
It holds none of the method's arithmetic (no attention, no cache write, no
quantisation), so both the HIP path and the CPU oracle can consume its
output without sharing any of the computation.

Workloads (shapes from the pages' 7B and 70B examples: [LAYERS] 2.1 gives
the 7B shape, 32 heads x 128 dims at 2048 tokens; [ENG5] "KV cache" gives
the 70B shape, 8 KV heads x 128 dims at up to 32K tokens):

=====  =====================  =============================================
id     name                   shape
=====  =====================  =============================================
1      tiny_f32               B=4, L={47,200,16,1}, H=Hkv=4, D=64, bs=16,
                              pool 32, fp32, scale 1/8
2      mha7b_bf16             B=32, L=2048, H=Hkv=32, D=128, bs=16, pool 4608
3      gqa70b_bf16            B=50, L log-uniform in [1024, 32768], H=64,
                              Hkv=8, D=128, bs=16, pool = blocks + 12.5%
4      prefix_bf16_bs{16,32}  B=256 sharing a 2000-token prefix, suffix
                              U{50..500}, H=32, Hkv=8, D=128
5      int8_gqa70b            B=64, L=8192, H=64, Hkv=8, D=128, bs=16,
                              fp32 N(0,1) K/V to be quantised to int8
6      fp8_gqa70b             the same shape and draws, quantised to FP8
                              (E4M3) instead
7      int4_gqa70b            the same shape and draws, quantised to INT4
8      e5m2_gqa70b            the same shape and draws, quantised to FP8
                              in the E5M2 format
=====  =====================  =============================================

Draw order with ``numpy.random.default_rng(seed)`` (PCG64): lengths, the
block-id permutation, q, the K pool, the V pool, the new tokens' k then v.
Values are iid N(0,1) drawn in fp32; bf16 inputs are those draws rounded to
nearest-even.  The last token of every sequence is the step's new token: its
slot is poisoned in the pool and its K/V come in ``k_new`` / ``v_new`` with
``slot_new``, to be written by the cache write before attention reads it.

Layouts: ``k_cache[NB, Hkv, bs, D]``, ``v_cache[NB, Hkv, bs/4, D, 4]``
(token ``r``, dim ``d`` of a V tile at ``[r // 4, d, r % 4]``),
``q[B, H, D]``, ``block_tables[B, MB]`` int32 (-1 past the last block),
``context_lens[B]`` int32, slots int64.  bf16 arrays hold uint16 bit
patterns.  Unused blocks, unused rows and the new-token slots hold NaN.
For the int8, FP8 and INT4 workloads the pool is not materialised: ``k_fill`` /
``v_fill`` ``[T, Hkv, D]`` fp32 with ``slot_fill`` list every cached token but the
new ones, for the consumer to quantise into its own coded cache (per sequence in
order; with a shared prefix, once per distinct slot instead).

A shared prefix (``prefix`` tokens) is held by every sequence, or by each
consecutive group of ``prefix_group_size`` sequences with its own prefix
blocks: the group's first sequence holds them and the others fork it.
"""

from dataclasses import dataclass, field
import math

import numpy as np

from .blocks import BlockAllocator

BF16_NAN = np.uint16(0x7FC0)
CODED_KINDS = ("i8", "fp8", "e5m2", "i4")  # caches of codes with per-(token, kv-head) scales
_CHUNK = 1 << 24  # elements drawn per RNG call when filling large pools


def bf16_bits(x):
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    return np.where(np.isnan(x), BF16_NAN, r).astype(np.uint16)


@dataclass
class Workload:
    name: str
    seed: int
    kv_dtype: str            # "f32" | "bf16" | "i8" | "fp8" | "e5m2" | "i4"
    q_dtype: str             # "f32" | "bf16"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_new: np.ndarray
    k_cache: np.ndarray = None   # f32 / bf16 pools
    v_cache: np.ndarray = None
    k_fill: np.ndarray = None    # i8 / fp8 / i4 workload: fp32 rows of every cached token
    v_fill: np.ndarray = None
    slot_fill: np.ndarray = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(len(self.context_lens))

    @property
    def attended_tokens(self):
        return int(np.sum(self.context_lens, dtype=np.int64))


def _draw(rng, shape, kind):
    """iid N(0,1) in fp32, rounded to bf16 bits when kind == 'bf16'."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if kind == "bf16" else np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = bf16_bits(x) if kind == "bf16" else x
    return out.reshape(shape)


def _poison(alloc, k_cache, v_cache, slots_new, kind):
    nan = BF16_NAN if kind == "bf16" else np.float32(np.nan)
    bs = alloc.block_size
    unused = np.nonzero(alloc.refcount == 0)[0]
    k_cache[unused] = nan
    v_cache[unused] = nan
    for blk in np.nonzero((alloc.refcount > 0) & (alloc.fill < bs))[0]:
        f = int(alloc.fill[blk])
        k_cache[blk, :, f:, :] = nan
        for r in range(f, bs):
            v_cache[blk, :, r // 4, :, r % 4] = nan
    for s in np.asarray(slots_new).tolist():
        k_cache[s // bs, :, s % bs, :] = nan
        v_cache[s // bs, :, (s % bs) // 4, :, s % 4] = nan


def _copy_rows(pool_k, pool_v, src, dst, rows):
    """Copy-on-write duplicate: the first ``rows`` tokens of block ``src``."""
    pool_k[dst, :, :rows, :] = pool_k[src, :, :rows, :]
    for r in range(rows):
        pool_v[dst, :, r // 4, :, r % 4] = pool_v[src, :, r // 4, :, r % 4]


def _allocate(lens, bs, num_blocks, order, prefix=0, prefix_group_size=None):
    """Allocate sequences; returns (alloc, sids, fill slots per seq, new slots).

    With a prefix, consecutive groups of ``prefix_group_size`` sequences (all
    sequences by default) each fork from a root holding its own prefix."""
    alloc = BlockAllocator(num_blocks, bs, order=order)
    sids = []
    fill_slots = []
    if prefix > 0:
        size = len(lens) if prefix_group_size is None else int(prefix_group_size)
        for start in range(0, len(lens), size):
            root = alloc.new_sequence()
            prefix_slots = alloc.append(root, prefix)
            n = min(size, len(lens) - start)
            group = [root] + [alloc.fork(root) for _ in range(n - 1)]
            sids += group
            fill_slots += [prefix_slots.copy() for _ in group]
    else:
        sids = [alloc.new_sequence() for _ in lens]
        fill_slots = [np.empty(0, dtype=np.int64) for _ in sids]
    new_slots = np.empty(len(lens), dtype=np.int64)
    for i, (sid, L) in enumerate(zip(sids, lens)):
        L = int(L)
        if L == 0 and prefix == 0:         # empty context: no blocks, no new token
            new_slots[i] = -1
            continue
        have = alloc.length(sid)
        if L - 1 > have:
            fill_slots[i] = np.concatenate([fill_slots[i], alloc.append(sid, L - 1 - have)])
        elif L - 1 < have:
            raise ValueError("context shorter than the shared prefix")
        new_slots[i] = alloc.append(sid, 1)[0] if L > 0 else -1
    return alloc, sids, fill_slots, new_slots


def _blocks_needed(lens, bs, prefix=0, prefix_group_size=None):
    probe_pool = int(sum((int(L) + bs - 1) // bs for L in lens)) + 8
    alloc, _, _, _ = _allocate(lens, bs, probe_pool, None, prefix, prefix_group_size)
    return int(np.count_nonzero(alloc.refcount))


def build(name, seed, lens, num_heads, num_kv_heads, head_dim, block_size,
          kv_dtype, q_dtype, scale=None, num_blocks=None, spare=0.125,
          prefix=0, rng=None, max_blocks_per_seq=None, meta=None, prefix_group_size=None):
    """Build a workload for the given context lengths (already drawn)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B, H, Hkv, D, bs = len(lens), num_heads, num_kv_heads, head_dim, block_size
    if num_blocks is None:
        need = _blocks_needed(lens, bs, prefix, prefix_group_size)
        num_blocks = max(1, int(math.ceil(need * (1.0 + spare))))
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(max((int(L) + bs - 1) // bs for L in lens)))
    perm = rng.permutation(num_blocks)
    alloc, sids, fill_slots, new_slots = _allocate(lens, bs, num_blocks, perm, prefix,
                                                   prefix_group_size)
    alloc.check()
    tables = alloc.tables(sids, max_blocks_per_seq)
    store = "bf16" if kv_dtype == "bf16" else "f32"
    q = _draw(rng, (B, H, D), "bf16" if q_dtype == "bf16" else "f32")
    w = Workload(
        name=name, seed=seed, kv_dtype=kv_dtype, q_dtype=q_dtype,
        num_heads=H, num_kv_heads=Hkv, head_dim=D, block_size=bs,
        num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        context_lens=lens.astype(np.int32), block_tables=tables, q=q,
        k_new=None, v_new=None, slot_new=new_slots, meta=dict(meta or {}))
    w.meta.update(prefix=prefix, copies=list(alloc.copies), prefix_group_size=prefix_group_size)
    if kv_dtype in CODED_KINDS and prefix:
        # shared blocks: fp32 pools as for bf16 (copy-on-write duplicates
        # included), then one fill row per distinct used slot
        k_pool = _draw(rng, (num_blocks, Hkv, bs, D), "f32")
        v_pool = _draw(rng, (num_blocks, Hkv, bs // 4, D, 4), "f32")
        for src, dst, rows in alloc.copies:
            _copy_rows(k_pool, v_pool, src, dst, rows)
        used = [np.asarray(f, np.int64) for f in fill_slots]
        used += [np.arange(dst * bs, dst * bs + rows, dtype=np.int64) for _, dst, rows in alloc.copies]
        slot_fill = np.unique(np.concatenate(used)) if used else np.empty(0, np.int64)
        w.k_fill = np.ascontiguousarray(k_pool[slot_fill // bs, :, slot_fill % bs, :])
        w.v_fill = np.ascontiguousarray(v_pool[slot_fill // bs, :, (slot_fill % bs) // 4, :, slot_fill % 4])
        w.slot_fill = slot_fill
        w.meta["fill_per_sequence"] = False
    elif kv_dtype in ("f32", "bf16"):
        k_cache = _draw(rng, (num_blocks, Hkv, bs, D), store)
        v_cache = _draw(rng, (num_blocks, Hkv, bs // 4, D, 4), store)
        for src, dst, rows in alloc.copies:        # copy-on-write duplicates
            _copy_rows(k_cache, v_cache, src, dst, rows)
        _poison(alloc, k_cache, v_cache, new_slots[new_slots >= 0], store)
        w.k_cache, w.v_cache = k_cache, v_cache
    elif kv_dtype in CODED_KINDS:
        w.meta["fill_per_sequence"] = True
        slot_fill = np.concatenate(fill_slots) if fill_slots else np.empty(0, np.int64)
        T = len(slot_fill)
        w.k_fill = _draw(rng, (T, Hkv, D), "f32")
        w.v_fill = _draw(rng, (T, Hkv, D), "f32")
        w.slot_fill = slot_fill
    else:
        raise ValueError(kv_dtype)
    w.k_new = _draw(rng, (B, Hkv, D), store)
    w.v_new = _draw(rng, (B, Hkv, D), store)
    return w


CONFIG_NAMES = {
    1: "tiny_f32",
    2: "mha7b_bf16",
    3: "gqa70b_bf16",
    4: "prefix_bf16",
    5: "int8_gqa70b",
    6: "fp8_gqa70b",
    7: "int4_gqa70b",
    8: "e5m2_gqa70b",
}


def make_config(config, seed=0, block_size=None):
    """The workloads listed in the module docstring."""
    rng = np.random.default_rng(seed)
    if config == 1:
        return build("tiny_f32", seed, [47, 200, 16, 1], 4, 4, 64, 16, "f32", "f32",
                     scale=1.0 / 8.0, num_blocks=32, rng=rng)
    if config == 2:
        return build("mha7b_bf16", seed, [2048] * 32, 32, 32, 128, 16, "bf16", "bf16",
                     num_blocks=4608, rng=rng)
    if config == 3:
        u = rng.uniform(math.log(1024.0), math.log(32768.0), size=50)
        lens = np.clip(np.rint(np.exp(u)), 1024, 32768).astype(np.int64)
        return build("gqa70b_bf16", seed, lens, 64, 8, 128, 16, "bf16", "bf16",
                     rng=rng, max_blocks_per_seq=2048)
    if config == 4:
        bs = 16 if block_size is None else int(block_size)
        suffix = rng.integers(50, 501, size=256)
        lens = 2000 + suffix
        return build(f"prefix_bf16_bs{bs}", seed, lens, 32, 8, 128, bs, "bf16", "bf16",
                     prefix=2000, rng=rng, max_blocks_per_seq=(2500 + bs - 1) // bs)
    if config == 5:
        return build("int8_gqa70b", seed, [8192] * 64, 64, 8, 128, 16, "i8", "bf16",
                     num_blocks=32768 + 4096, rng=rng)
    if config == 6:
        return build("fp8_gqa70b", seed, [8192] * 64, 64, 8, 128, 16, "fp8", "bf16",
                     num_blocks=32768 + 4096, rng=rng)
    if config == 7:
        return build("int4_gqa70b", seed, [8192] * 64, 64, 8, 128, 16, "i4", "bf16",
                     num_blocks=32768 + 4096, rng=rng)
    if config == 8:
        return build("e5m2_gqa70b", seed, [8192] * 64, 64, 8, 128, 16, "e5m2", "bf16",
                     num_blocks=32768 + 4096, rng=rng)
    raise ValueError(f"unknown config {config}")


def make_custom(seed, lens, num_heads, num_kv_heads, head_dim, block_size,
                kv_dtype="bf16", q_dtype=None, spare=0.25, prefix=0, scale=None,
                prefix_group_size=None):
    """Small workload of arbitrary shape for tests (same recipe as above)."""
    if q_dtype is None:
        q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    return build(f"custom_s{seed}", seed, lens, num_heads, num_kv_heads, head_dim,
                 block_size, kv_dtype, q_dtype, spare=spare, prefix=prefix, scale=scale,
                 prefix_group_size=prefix_group_size)
