"""Host-side block allocator for a paged KV cache.

Implements the block manager of [ENG5] "Block manager: how paging works"
("LLM Engineering (5): core techniques of inference optimization",
chenk.top): a pool of fixed-size physical blocks, a free list, one block
table per sequence, and reference-counted sharing with copy-on-write.

* ``append`` grows a sequence: when its tail block is full a block is popped
  from the free list and appended to the table; the new tokens' slots
  (``physical_block * block_size + row``) are returned.
* ``fork`` makes a new sequence that shares every block of an existing one
  (refcount + 1 per block), as for a shared prompt prefix ([ENG5] "Paged
  attention": requests with a common prefix share physical blocks).
* Writing into a tail block whose refcount is above one first copies it to a
  private block (copy-on-write); the copy is logged in ``copies`` as
  ``(src, dst, rows)`` so the caller can copy the cached K/V rows.
* ``free_sequence`` drops one reference per block; a block returns to the
  free list only when its count reaches zero.

This module does bookkeeping only; it never touches K/V data.
"""

from dataclasses import dataclass, field

import numpy as np


class OutOfBlocks(RuntimeError):
    """The free list is empty."""


@dataclass
class _Seq:
    table: list = field(default_factory=list)
    length: int = 0


class BlockAllocator:
    """Free list + refcounts + copy-on-write over ``num_blocks`` blocks."""

    def __init__(self, num_blocks, block_size, order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if order is None:
            order = np.arange(self.num_blocks)
        order = [int(b) for b in order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        # pop() takes from the end; reverse so blocks are handed out in `order`
        self._free = order[::-1]
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)
        # rows of each block that hold written tokens (high-water mark)
        self.fill = np.zeros(self.num_blocks, dtype=np.int64)
        self._seqs = {}
        self._next_id = 0
        self.copies = []

    # -- pool -----------------------------------------------------------
    @property
    def num_free(self):
        return len(self._free)

    def _pop(self):
        if not self._free:
            raise OutOfBlocks("no free KV blocks")
        blk = self._free.pop()
        assert self.refcount[blk] == 0
        self.refcount[blk] = 1
        self.fill[blk] = 0
        return blk

    def _release(self, blk):
        self.refcount[blk] -= 1
        assert self.refcount[blk] >= 0
        if self.refcount[blk] == 0:
            self._free.append(blk)

    # -- sequences ------------------------------------------------------
    def new_sequence(self):
        sid = self._next_id
        self._next_id += 1
        self._seqs[sid] = _Seq()
        return sid

    def fork(self, sid):
        """New sequence sharing all of ``sid``'s blocks."""
        src = self._seqs[sid]
        nid = self.new_sequence()
        self._seqs[nid].table = list(src.table)
        self._seqs[nid].length = src.length
        for blk in src.table:
            self.refcount[blk] += 1
        return nid

    def free_sequence(self, sid):
        seq = self._seqs.pop(sid)
        for blk in seq.table:
            self._release(blk)

    def length(self, sid):
        return self._seqs[sid].length

    def block_table(self, sid):
        return list(self._seqs[sid].table)

    def append(self, sid, n=1):
        """Append ``n`` tokens to ``sid``; return their slots (int64)."""
        seq = self._seqs[sid]
        bs = self.block_size
        out = np.empty(int(n), dtype=np.int64)
        done = 0
        while done < n:
            row = seq.length % bs
            if row == 0:
                seq.table.append(self._pop())
            else:
                tail = seq.table[-1]
                if self.refcount[tail] > 1:
                    fresh = self._pop()
                    self.copies.append((tail, fresh, row))
                    self.fill[fresh] = row
                    self._release(tail)
                    seq.table[-1] = fresh
            blk = seq.table[-1]
            take = min(bs - row, n - done)
            out[done:done + take] = blk * bs + row + np.arange(take, dtype=np.int64)
            self.fill[blk] = max(self.fill[blk], row + take)
            seq.length += take
            done += take
        return out

    def tables(self, sids, max_blocks):
        """Block tables of ``sids`` as int32 ``[len(sids), max_blocks]``, -1 padded."""
        t = np.full((len(sids), int(max_blocks)), -1, dtype=np.int32)
        for i, sid in enumerate(sids):
            tab = self._seqs[sid].table
            if len(tab) > max_blocks:
                raise ValueError("sequence has more blocks than max_blocks")
            t[i, :len(tab)] = tab
        return t

    def check(self):
        """Internal consistency: refcounts equal table references; free list exact."""
        ref = np.zeros(self.num_blocks, dtype=np.int64)
        for seq in self._seqs.values():
            for blk in seq.table:
                ref[blk] += 1
        assert np.array_equal(ref, self.refcount), "refcount mismatch"
        free = set(self._free)
        assert len(free) == len(self._free), "block on free list twice"
        assert free == {b for b in range(self.num_blocks) if ref[b] == 0}, "free list mismatch"
        return True


def cascade_groups(block_tables, context_lens, block_size, min_shared_blocks=1):
    """Groups of consecutive sequences that share leading blocks.

    A group starts at a sequence (its first member); the next sequence
    joins when it shares at least ``min_shared_blocks`` leading table
    entries with the first member, which fixes the group's shared count; a
    later sequence joins while it shares at least that many.  Only whole
    blocks inside both contexts count.  Returns ``(group_start int32
    [NG + 1], group_shared_blocks int32 [NG], max_group_size,
    max_shared_blocks)``, the arguments of the shared-prefix decode
    ([ENG5] "Paged attention": requests with a common prefix hold the same
    physical blocks).  Sequences that share nothing are groups of one with
    0 shared blocks.
    """
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens, dtype=np.int64)
    B = len(lens)
    full = lens // int(block_size)

    def common(a, b):
        n = int(min(full[a], full[b]))
        ta, tb = tables[a, :n], tables[b, :n]
        diff = np.nonzero(ta != tb)[0]
        return int(diff[0]) if len(diff) else n

    starts, shared = [], []
    b = 0
    while b < B:
        lead, cnt, size = b, 0, 1
        b += 1
        if b < B:
            c = common(lead, b)
            if c >= max(1, int(min_shared_blocks)):
                cnt = c
                while b < B and common(lead, b) >= cnt:
                    b += 1
                    size += 1
        starts.append(lead)
        shared.append(cnt)
    group_start = np.array(starts + [B], dtype=np.int32)
    group_shared = np.array(shared, dtype=np.int32)
    sizes = np.diff(group_start)
    return (group_start, group_shared, int(sizes.max()) if B else 0,
            int(group_shared.max()) if B else 0)
