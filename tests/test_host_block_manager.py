"""The library's native block manager, on the host (no GPU needed).

Random sequences of new / fork / append / free are replayed on the native
manager and on the Python allocator (``blocks.BlockAllocator``) with the same
free-list order: tables, slots, copy-on-write copies and reference counts
must agree after every operation.  Swapping, all-or-nothing failure and the
argument checks are tested against the invariants they promise.
"""

import numpy as np
import pytest

from paged_kv_cache_29_amd import BlockManager
from paged_kv_cache_29_amd.blocks import BlockAllocator, OutOfBlocks


def _invariants(bm, live, swapped=()):
    """refcount of a block = number of live device tables holding it; the
    free count = blocks with refcount 0."""
    ref = np.zeros(bm.num_blocks, dtype=np.int64)
    for sid in live:
        if sid in swapped:
            continue
        for b in bm.block_table(sid):
            ref[b] += 1
    assert np.array_equal(ref, bm.refcounts())
    assert bm.num_free == int((ref == 0).sum())


@pytest.mark.parametrize("seed,bs", [(0, 16), (1, 32), (2, 16), (3, 1)])
def test_native_manager_matches_python_allocator(seed, bs):
    rng = np.random.default_rng(seed)
    NB = 400
    order = rng.permutation(NB)
    nat = BlockManager(NB, bs, order=order)
    py = BlockAllocator(NB, bs, order=order)
    ids = {}  # native id -> python id
    live = []
    for step in range(600):
        op = rng.choice(["new", "fork", "append", "append", "append", "free"])
        if op == "new" or not live:
            a, b = nat.new_sequence(), py.new_sequence()
            ids[a] = b
            live.append(a)
        elif op == "fork":
            src = live[rng.integers(len(live))]
            a, b = nat.fork(src), py.fork(ids[src])
            ids[a] = b
            live.append(a)
        elif op == "append":
            sid = live[rng.integers(len(live))]
            n = int(rng.integers(0, 3 * bs + 2))
            need = n // bs + 2
            if need > nat.num_free:  # keep both in the no-exhaustion regime
                continue
            before = len(py.copies)
            slots, copies = nat.append(sid, n)
            ref = py.append(ids[sid], n)
            assert np.array_equal(slots, ref)
            assert copies == [tuple(c) for c in py.copies[before:]]
        else:
            sid = live.pop(int(rng.integers(len(live))))
            nat.free_sequence(sid)
            py.free_sequence(ids[sid])
        for sid in live:
            assert nat.block_table(sid) == py.block_table(ids[sid])
            assert nat.length(sid) == py.length(ids[sid])
        assert np.array_equal(nat.refcounts(), py.refcount)
        assert nat.num_free == py.num_free
    _invariants(nat, live)


def test_append_is_all_or_nothing():
    bm = BlockManager(4, 16)
    a = bm.new_sequence()
    bm.append(a, 40)                       # 3 blocks
    b = bm.fork(a)
    table, refs = bm.block_table(a), bm.refcounts()
    with pytest.raises(OutOfBlocks):
        bm.append(b, 30)                   # copy-on-write of the tail + 1 more block: 2 > 1 free
    assert bm.block_table(a) == table and bm.block_table(b) == table
    assert np.array_equal(bm.refcounts(), refs) and bm.length(b) == 40
    slots, copies = bm.append(b, 8)        # fits: the private copy takes the last block
    assert copies == [(table[-1], bm.block_table(b)[-1], 8)]
    assert slots.tolist() == [bm.block_table(b)[-1] * 16 + r for r in range(8, 16)]
    with pytest.raises(OutOfBlocks):
        bm.append(b, 1)
    _invariants(bm, [a, b])


def test_copy_on_write_only_for_a_shared_partial_tail():
    bm = BlockManager(16, 16)
    a = bm.new_sequence()
    bm.append(a, 32)                       # two full blocks
    b = bm.fork(a)
    slots, copies = bm.append(b, 1)        # full tail: a new block, no copy
    assert copies == [] and bm.block_table(b)[:2] == bm.block_table(a)
    c = bm.fork(b)
    _, copies = bm.append(c, 1)            # shared partial tail (1 row): copied
    assert copies == [(bm.block_table(b)[2], bm.block_table(c)[2], 1)]
    _, copies = bm.append(b, 1)            # b's tail is private again
    assert copies == []
    _invariants(bm, [a, b, c])


def test_swap_out_and_in():
    bm = BlockManager(10, 16, num_host_blocks=6, order=np.arange(10)[::-1])
    a = bm.new_sequence()
    bm.append(a, 50)                       # 4 blocks
    b = bm.fork(a)
    bm.append(b, 5)                        # b: copy of the tail + shared first 3
    ta, tb = bm.block_table(a), bm.block_table(b)
    free0 = bm.num_free
    pairs = bm.swap_out(b)
    assert pairs[:, 0].tolist() == tb and len(set(pairs[:, 1].tolist())) == len(tb)
    assert bm.num_free_host == 6 - len(tb)
    assert bm.num_free == free0 + 1        # only b's private tail is freed; shared blocks stay with a
    assert bm.block_table(a) == ta
    with pytest.raises(ValueError):
        bm.block_table(b)
    with pytest.raises(ValueError):
        bm.append(b, 1)
    with pytest.raises(ValueError):
        bm.fork(b)
    with pytest.raises(ValueError):
        bm.swap_out(b)
    _invariants(bm, [a, b], swapped={b})
    back = bm.swap_in(b)
    assert back[:, 0].tolist() == pairs[:, 1].tolist()
    tb2 = bm.block_table(b)
    assert back[:, 1].tolist() == tb2 and len(tb2) == len(tb) and bm.length(b) == 55
    assert not set(tb2) & set(ta)          # swapped-in blocks are private
    assert bm.num_free_host == 6
    _invariants(bm, [a, b])
    # host pool too small: nothing changes
    c = bm.new_sequence()
    bm.append(c, 16 * 2)
    assert bm.num_free == 0
    pairs_c = bm.swap_out(c)
    assert len(pairs_c) == 2
    d = bm.new_sequence()
    bm.append(d, 16 * 2)                   # takes c's freed blocks
    with pytest.raises(OutOfBlocks):
        bm.swap_in(c)                      # no device block free
    bm.free_sequence(c)                    # a swapped-out sequence returns host blocks
    assert bm.num_free_host == 6
    _invariants(bm, [a, b, d])


def test_argument_checks():
    with pytest.raises(ValueError):
        BlockManager(0, 16)
    with pytest.raises(ValueError):
        BlockManager(4, 16, order=[0, 1, 1, 3])
    bm = BlockManager(4, 16)
    with pytest.raises(ValueError):
        bm.append(99, 1)
    with pytest.raises(ValueError):
        bm.free_sequence(99)
    a = bm.new_sequence()
    bm.free_sequence(a)
    with pytest.raises(ValueError):
        bm.free_sequence(a)
    assert bm.length(a) == -1
    with pytest.raises(OutOfBlocks):
        bm.append(bm.new_sequence(), 16 * 5)
    # an empty sequence swaps with no pairs
    e = bm.new_sequence()
    assert len(bm.swap_out(e)) == 0 and len(bm.swap_in(e)) == 0
