"""Host checks of the device-data preconditions (include/pagedkv_debug.h).

The checkers run on host arrays, so every accept and reject case runs here
without a GPU.  Valid inputs come from the block manager and the group
finder; each reject case breaks one precondition of paged addressing
("LLM Engineering (5)", "Paged attention" and "Block manager: how paging
works") or of the group / query-range arrays.
"""

import re

import numpy as np
import pytest

import paged_kv_cache_29_amd as pkv
from paged_kv_cache_29_amd import blocks


def _served_pool(bs=16, NB=64, seed=0):
    """Tables and lengths of a pool with forks (shared prefixes) and two
    independent sequences, padded with entries no context uses."""
    rng = np.random.default_rng(seed)
    bm = blocks.BlockAllocator(NB, bs, order=rng.permutation(NB))
    root = bm.new_sequence()
    bm.append(root, 3 * bs + 5)
    seqs = [root] + [bm.fork(root) for _ in range(3)]
    for n in (bs - 3, 2 * bs + 7):
        s = bm.new_sequence()
        bm.append(s, n)
        seqs.append(s)
    for s in seqs:
        bm.append(s, 1)
    lens = np.array([bm.length(s) for s in seqs], np.int32)
    MB = int(max((L + bs - 1) // bs for L in lens)) + 2
    tables = np.full((len(seqs), MB), -7, np.int32)      # unused entries: never read
    for i, s in enumerate(seqs):
        t = bm.block_table(s)
        tables[i, :len(t)] = t
    return tables, lens, bs, NB


# ---- block tables ---------------------------------------------------------

def test_tables_accept_served_pool():
    tables, lens, bs, NB = _served_pool()
    pkv.check_block_tables(tables, lens, bs, NB)


def test_tables_accept_edges():
    bs, NB, MB = 16, 8, 3
    tables = np.array([[7, 0, 3], [-1, -1, -1], [5, 9999, -3]], np.int32)
    lens = np.array([MB * bs, 0, bs], np.int32)          # full row; empty; one block
    pkv.check_block_tables(tables, lens, bs, NB)
    pkv.check_block_tables(np.zeros((0, MB), np.int32), np.zeros(0, np.int32), bs, NB)


@pytest.mark.parametrize("where,value,frag", [
    ("len", -1, "context_lens[2] = -1"),
    ("len", None, "outside [0, "),                        # one past the row
    ("blk", -1, "block_tables[2]"),
    ("blk", None, "outside [0, 64)"),                    # == num_blocks
])
def test_tables_reject(where, value, frag):
    tables, lens, bs, NB = _served_pool()
    if where == "len":
        lens[2] = tables.shape[1] * bs + 1 if value is None else value
    else:
        last = (lens[2] - 1) // bs                        # the last entry sequence 2 uses
        tables[2, last] = NB if value is None else value
    with pytest.raises(ValueError, match=re.escape(frag)):
        pkv.check_block_tables(tables, lens, bs, NB)


# ---- slot mapping ---------------------------------------------------------

def test_slots_accept():
    bs, NB = 16, 8
    rng = np.random.default_rng(1)
    slots = rng.permutation(NB * bs)[:100].astype(np.int64)
    slots[::7] = -1                                       # skipped tokens may repeat
    slots[3] = NB * bs - 1
    pkv.check_slot_mapping(slots, bs, NB)
    pkv.check_slot_mapping(np.zeros(0, np.int64), bs, NB)


def test_slots_reject_past_pool():
    with pytest.raises(ValueError, match=r"slot_mapping\[1\] = 128 outside \[0, 128\)"):
        pkv.check_slot_mapping(np.array([0, 128, 5], np.int64), 16, 8)


def test_slots_reject_shared_slot():
    slots = np.array([4, 17, -1, 90, 17, -1], np.int64)
    with pytest.raises(ValueError, match="tokens 1 and 4 share slot 17"):
        pkv.check_slot_mapping(slots, 16, 8)


# ---- query ranges ---------------------------------------------------------

def test_query_start_accept():
    lens = np.array([40, 3, 17, 1], np.int32)
    qs = np.array([0, 5, 5, 8, 9], np.int32)              # 5, 0, 3, 1 new tokens
    pkv.check_query_start(qs, lens, 9, 5)
    pkv.check_query_start(np.zeros(1, np.int32), np.zeros(0, np.int32), 0, 1)


@pytest.mark.parametrize("qs,T,maxq,frag", [
    ([1, 5, 5, 8, 9], 9, 5, r"query_start\[0\] = 1"),
    ([0, 5, 4, 8, 9], 9, 5, "decreases at 2"),
    ([0, 5, 5, 8, 9], 10, 5, r"query_start\[4\] = 9, not num_query_tokens = 10"),
    ([0, 5, 5, 8, 9], 9, 4, "sequence 0 has 5 new tokens, max_queries_per_seq is 4"),
    ([0, 5, 9, 12, 13], 13, 5, "sequence 1 has 4 new tokens in a context of 3"),
])
def test_query_start_reject(qs, T, maxq, frag):
    lens = np.array([40, 3, 17, 1], np.int32)
    with pytest.raises(ValueError, match=frag):
        pkv.check_query_start(np.array(qs, np.int32), lens, T, maxq)


# ---- shared-prefix groups -------------------------------------------------

def test_groups_accept_found_groups():
    tables, lens, bs, NB = _served_pool()
    gs, gsb, mg, ms = blocks.cascade_groups(tables, lens, bs)
    assert mg == 4 and ms >= 3                            # the forks form one group
    pkv.check_groups(gs, gsb, tables, lens, bs, mg, ms)
    # a smaller cap on the shared span is still valid (the rest is the members' own)
    pkv.check_groups(gs, gsb, tables, lens, bs, mg, 1)
    # so is every sequence on its own
    B = len(lens)
    pkv.check_groups(np.arange(B + 1, dtype=np.int32), np.zeros(B, np.int32), tables, lens, bs, 1, 0)


def _groups():
    tables, lens, bs, NB = _served_pool()
    gs, gsb, mg, ms = blocks.cascade_groups(tables, lens, bs)
    return tables, lens, bs, gs, gsb, mg, ms


def test_groups_reject_bad_ranges():
    tables, lens, bs, gs, gsb, mg, ms = _groups()
    B = len(lens)
    for bad, frag in ((np.r_[1, gs[1:]], r"group_start\[0\] = 1"),
                      (np.r_[gs[:-1], B - 1], "not num_seqs"),
                      (np.array([0, 3, 2, B], np.int32), "decreases at 2")):
        with pytest.raises(ValueError, match=frag):
            pkv.check_groups(bad.astype(np.int32), np.zeros(len(bad) - 1, np.int32), tables, lens, bs,
                             B, ms)
    with pytest.raises(ValueError, match="max_group_size is 3"):
        pkv.check_groups(gs, gsb, tables, lens, bs, 3, ms)


def test_groups_reject_member_that_differs():
    tables, lens, bs, gs, gsb, mg, ms = _groups()
    tables = tables.copy()
    tables[2, 1] = tables[0, 1] + 1                       # inside the shared span
    with pytest.raises(ValueError, match=r"sequence 2 of group 0: block_tables\[2\]\[1\]"):
        pkv.check_groups(gs, gsb, tables, lens, bs, mg, ms)
    # past the capped span the difference is allowed
    pkv.check_groups(gs, gsb, tables, lens, bs, mg, 1)


def test_groups_reject_member_shorter_than_the_span():
    tables, lens, bs, gs, gsb, mg, ms = _groups()
    lens = lens.copy()
    S = int(min(gsb[0], ms, lens[0] // bs)) * bs
    lens[3] = S - 1
    with pytest.raises(ValueError, match=f"sequence 3 of group 0 has {S - 1} tokens, fewer than the {S} shared"):
        pkv.check_groups(gs, gsb, tables, lens, bs, mg, ms)


# ---- the checkers' own argument checks, through the C ABI -------------------

def test_checkers_reject_bad_arguments():
    import ctypes
    lib = pkv.load_library()
    one = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    slots = (ctypes.c_int64 * 2)(0, 1)
    INVALID = 1
    cases = [
        (lambda: lib.pkv_check_block_tables(one, one, -1, 1, 16, 8), "invalid sizes"),
        (lambda: lib.pkv_check_block_tables(one, one, 1, 0, 16, 8), "invalid sizes"),
        (lambda: lib.pkv_check_block_tables(None, one, 1, 1, 16, 8), "null array"),
        (lambda: lib.pkv_check_slot_mapping(slots, 2, 0, 8), "invalid sizes"),
        (lambda: lib.pkv_check_slot_mapping(None, 2, 16, 8), "null array"),
        (lambda: lib.pkv_check_query_start(one, one, -1, 0, 1), "invalid sizes"),
        (lambda: lib.pkv_check_query_start(None, one, 1, 0, 1), "null array"),
        (lambda: lib.pkv_check_groups(one, one, one, one, 1, 1, 16, -1, 1, 0), "invalid sizes"),
        (lambda: lib.pkv_check_groups(one, None, one, one, 1, 1, 16, 1, 1, 0), "null array"),
    ]
    for call, frag in cases:
        assert call() == INVALID
        assert frag in lib.pkv_last_error().decode()
    # nothing to check is valid, and clears the last error
    assert lib.pkv_check_slot_mapping(None, 0, 16, 8) == 0
    assert lib.pkv_last_error() == b""
