"""fp64 definition of single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages fix it:

* The KV cache lives in fixed-size physical blocks of ``block_size`` tokens,
  and each sequence owns a block table mapping its logical blocks to physical
  ones, like OS page tables ([ENG5] "Paged attention").  A request of 47 tokens
  occupies 3 blocks filled 16+16+15; only the last block can be partial
  ([ENG5] "Paged attention", worked example and the near-zero-waste remark).
* A decode step attends the one new query token of each sequence over all of
  that sequence's cached keys and values ([ENG5] "Two phases with very
  different characteristics": every decode step reads the whole KV cache).
* Attention itself is the textbook ``out = softmax(scale * K q) V`` per query
  head, over the sequence's ``context_len`` tokens.

Readings taken where the pages are silent (each is listed in the design doc):

* Cache layout (the pages print sizes, not an order): ``k_cache`` is
  ``[num_blocks, num_kv_heads, block_size, head_dim]`` (each token a row) and
  ``v_cache`` is ``[num_blocks, num_kv_heads, block_size / 4, head_dim, 4]``
  (each tile in groups of 4 consecutive tokens, dim-major inside a group:
  token ``r``, dim ``d`` at ``[r // 4, d, r % 4]``).  The oracle reads both
  by index, token by token within a block, so its arithmetic does not
  depend on the layout.
* GQA grouping: query head ``h`` reads kv-head ``h // (H / Hkv)``.
* ``context_len == 0`` gives an all-zero output row.
* int8 cache: the value of a stored code ``c`` with scale ``s`` is ``c * s``
  ([LAYERS] 2.3, per-token scales; [ENG5] "KV-cache quantization",
  per-token-per-head scales), evaluated exactly in fp64.
* INT4 cache: two codes per byte (layout and quantiser in ``int4.py``); the
  value of code ``c`` with scale ``s`` is again ``c * s``, exactly.
* bf16 elements are given as their 16-bit patterns (``uint16``); their value
  is the fp32 number whose upper half is that pattern.
"""

import numpy as np

from . import fp8 as _fp8
from . import int4 as _int4

KV_DTYPES = ("f32", "bf16", "i8", "fp8", "e5m2", "i4")
CODED = ("i8", "fp8", "e5m2", "i4")  # codes with one scale per (token, kv-head)


def n_blocks(context_len, block_size):
    """Number of physical blocks a sequence of ``context_len`` tokens occupies.

    ceil(L / bs): 47 tokens -> 3 blocks, 200 tokens -> 13 blocks at bs = 16
    ([ENG5] "Paged attention", worked example).
    """
    context_len = int(context_len)
    block_size = int(block_size)
    if context_len <= 0:
        return 0
    return (context_len + block_size - 1) // block_size


def rows_in_block(context_len, block_size, j):
    """Valid token rows held by logical block ``j`` of a sequence.

    Every block but the last is full; the last holds ``L - (n - 1) * bs``
    ([ENG5] "Paged attention": only the last block may be partial).
    """
    n = n_blocks(context_len, block_size)
    if j < 0 or j >= n:
        return 0
    if j < n - 1:
        return int(block_size)
    return int(context_len) - (n - 1) * int(block_size)


def token_location(t, block_table, block_size):
    """(physical block, row) that holds logical token ``t`` of a sequence.

    The block table maps logical block ``t // bs`` to a physical block; the
    token sits at row ``t % bs`` inside it ([ENG5] "Paged attention").
    """
    t = int(t)
    block_size = int(block_size)
    return int(block_table[t // block_size]), t % block_size


def kv_head_of(h, num_heads, num_kv_heads):
    """KV head read by query head ``h``: contiguous groups of ``H / Hkv``."""
    group = int(num_heads) // int(num_kv_heads)
    return int(h) // group


def widen(x, kind):
    """Exact fp64 value of stored elements ``x`` of element type ``kind``."""
    x = np.asarray(x)
    if kind == "bf16":
        bits = x.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if kind == "f32":
        return x.astype(np.float32).astype(np.float64)
    if kind == "i8":
        return x.astype(np.int8).astype(np.float64)
    if kind == "fp8":
        return _fp8.e4m3_decode(x.astype(np.uint8))
    if kind == "e5m2":
        return _fp8.e5m2_decode(x.astype(np.uint8))
    raise ValueError(f"unknown element type {kind!r}")


def gather_kv(k_cache, v_cache, block_table, context_len, block_size, kv_head,
              kv_dtype, k_scale=None, v_scale=None):
    """Contiguous fp64 ``K[L, D]`` and ``V[L, D]`` of one sequence and kv-head.

    Walks the sequence's logical blocks in order; logical block ``j`` lives in
    physical block ``block_table[j]`` and contributes its first
    ``rows_in_block(L, bs, j)`` rows.  Table entries past the last logical
    block are never read.  For an int8, FP8 or INT4 cache each element's
    value is its code's value times its token's scale; INT4 tiles hold two
    dims per byte (``k_cache[..., D/2]``, ``v_cache[..., D/2, 4]``).
    """
    L = int(context_len)
    bs = int(block_size)
    D = k_cache.shape[-1] * (2 if kv_dtype == "i4" else 1)
    K = np.zeros((L, D), dtype=np.float64)
    V = np.zeros((L, D), dtype=np.float64)
    for j in range(n_blocks(L, bs)):
        rows = rows_in_block(L, bs, j)
        blk = int(block_table[j])
        # V token rows: token r of the tile is [r // 4, :, r % 4]; swapping
        # the last two axes and merging the first two lists them in order
        v_tile = np.asarray(v_cache[blk, kv_head])                          # [bs/4, D(/2), 4]
        v_tok = np.swapaxes(v_tile, 1, 2).reshape(bs, v_tile.shape[1])[:rows]
        if kv_dtype == "i4":
            k_rows = _int4.unpack_int4(k_cache[blk, kv_head, :rows, :], axis=-1).astype(np.float64)
            v_rows = _int4.unpack_int4(v_tok, axis=-1).astype(np.float64)
        else:
            k_rows = widen(k_cache[blk, kv_head, :rows, :], kv_dtype)        # [rows, D]
            v_rows = widen(v_tok, kv_dtype)                                  # [rows, D]
        if kv_dtype in CODED:
            ks = np.asarray(k_scale[blk, kv_head, :rows], dtype=np.float32).astype(np.float64)
            vs = np.asarray(v_scale[blk, kv_head, :rows], dtype=np.float32).astype(np.float64)
            k_rows = k_rows * ks[:, None]
            v_rows = v_rows * vs[:, None]
        K[j * bs: j * bs + rows] = k_rows
        V[j * bs: j * bs + rows] = v_rows
    return K, V


def attend_one(q_vec, K, V, scale):
    """Textbook attention of one query vector over contiguous K, V (fp64).

    ``s = scale * K q``; ``p = exp(s - max s)``; ``out = (p V) / sum(p)``.
    Subtracting the maximum does not change the result and keeps exp finite.
    An empty context gives zeros.
    """
    q_vec = np.asarray(q_vec, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = float(scale) * (K @ q_vec)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                     num_heads, num_kv_heads, head_dim, block_size,
                     kv_dtype, q_dtype, k_scale=None, v_scale=None,
                     samples=None):
    """fp64 decode attention for a batch of sequences (one query token each).

    Shapes: ``q[B, H, D]``; ``k_cache[NB, Hkv, bs, D]``;
    ``v_cache[NB, Hkv, bs/4, D, 4]``; ``block_tables[B, MB]``; ``context_lens[B]``;
    scales ``[NB, Hkv, bs]`` (int8, FP8, INT4; INT4 tiles hold two dims per
    byte).  ``q_dtype`` / ``kv_dtype`` name the stored element types ("f32",
    "bf16", "i8", "fp8" (E4M3), "e5m2", "i4").

    Returns ``out[B, H, D]`` in fp64.  With ``samples`` (an iterable of
    ``(b, h)`` pairs) only those rows are computed and the others are NaN.
    """
    if kv_dtype not in KV_DTYPES:
        raise ValueError(kv_dtype)
    H, Hkv, D = int(num_heads), int(num_kv_heads), int(head_dim)
    if H % Hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    B = len(context_lens)
    if samples is None:
        out = np.zeros((B, H, D), dtype=np.float64)
        wanted = {(b, h) for b in range(B) for h in range(H)}
    else:
        out = np.full((B, H, D), np.nan, dtype=np.float64)
        wanted = {(int(b), int(h)) for b, h in samples}
    by_group = {}
    for b, h in wanted:
        by_group.setdefault((b, kv_head_of(h, H, Hkv)), []).append(h)
    for (b, g), heads in sorted(by_group.items()):
        K, V = gather_kv(k_cache, v_cache, block_tables[b], context_lens[b],
                         block_size, g, kv_dtype, k_scale, v_scale)
        for h in heads:
            q_vec = widen(q[b, h, :D], q_dtype)
            out[b, h] = attend_one(q_vec, K, V, scale)
    return out


def multi_query_attention(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                          num_heads, num_kv_heads, head_dim, block_size, kv_dtype, q_dtype,
                          k_scale=None, v_scale=None, samples=None):
    """fp64 causal attention of several new query tokens per sequence.

    A verification step of speculative decoding scores k + 1 proposed
    positions in one pass, and a prefill chunk scores a run of new tokens,
    instead of one token per step ([ENG5] "Speculative decoding", "Orca's
    iteration-level scheduling": chunked prefill).  Reading taken: sequence
    ``b`` has ``n_b = query_start[b+1] - query_start[b]`` new tokens, the last
    ``n_b`` of its ``L_b = context_lens[b]`` cached tokens (their K/V already
    written); its query row ``query_start[b] + i`` sits at position
    ``p = L_b - n_b + i`` and attends to tokens ``0 .. p`` (causal), through
    the block table exactly as decode does.

    Shapes: ``q[T, H, D]`` with ``T = query_start[B]``; caches, tables and
    scales as for ``decode_attention``.  Returns ``out[T, H, D]`` in fp64;
    with ``samples`` (``(row, h)`` pairs) only those rows are computed, the
    others are NaN.
    """
    if kv_dtype not in KV_DTYPES:
        raise ValueError(kv_dtype)
    H, Hkv, D = int(num_heads), int(num_kv_heads), int(head_dim)
    if H % Hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    qs = [int(x) for x in query_start]
    T = qs[-1]
    if samples is None:
        out = np.zeros((T, H, D), dtype=np.float64)
        wanted = {(r, h) for r in range(T) for h in range(H)}
    else:
        out = np.full((T, H, D), np.nan, dtype=np.float64)
        wanted = {(int(r), int(h)) for r, h in samples}
    rows_of = {}
    for b in range(len(qs) - 1):
        for r in range(qs[b], qs[b + 1]):
            rows_of[r] = b
    by_group = {}
    for r, h in wanted:
        by_group.setdefault((rows_of[r], kv_head_of(h, H, Hkv)), []).append((r, h))
    for (b, g), pairs in sorted(by_group.items()):
        L = int(context_lens[b])
        n = qs[b + 1] - qs[b]
        if n > L:
            raise ValueError("more new tokens than the context holds")
        K, V = gather_kv(k_cache, v_cache, block_tables[b], L, block_size, g, kv_dtype,
                         k_scale, v_scale)
        for r, h in pairs:
            pos = L - n + (r - qs[b])
            q_vec = widen(q[r, h, :D], q_dtype)
            out[r, h] = attend_one(q_vec, K[:pos + 1], V[:pos + 1], scale)
    return out
