"""Definitions of the KV-cache writes: the slot scatter and the int8 quantiser.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Slot scatter.  When a sequence grows by a token, the block manager hands
  out the next slot in its tail block (appending a fresh block when the tail
  is full) and the token's K and V go there ([ENG5] "Block manager: how
  paging works").  A slot is the flat index ``physical_block * bs + row``
  (the block/row model of [ENG5] "Paged attention").  Reading taken: a
  negative slot means "no write" for that token.  Layout as in
  ``attention.py``: K rows at ``k_cache[blk, h, row, :]``, V at
  ``v_cache[blk, h, row // 4, :, row % 4]``.  The write is a bit copy.

* int8 quantiser.  Symmetric int8 with one scale per (token, kv-head)
  ([ENG5] "KV-cache quantization": per-token-per-head scales computed online;
  [LAYERS] 2.3: per-token scales, K and V quantized separately), using
  ``q = round(x / s)`` ([ENG5] "INT8 weight-only quantization") with
  ``s = absmax / 127``.  Readings taken: fp32 throughout (IEEE division);
  round half to even; clamp to [-127, 127]; a row whose scale is zero
  (all-zero, or so tiny that absmax / 127 underflows) gets ``s = 0`` and
  codes 0.  Inputs are assumed finite.
"""

import numpy as np


def cache_write(k, v, k_cache, v_cache, slot_mapping, block_size):
    """Return copies of ``(k_cache, v_cache)`` with the new tokens written.

    ``k, v: [T, Hkv, D]`` in the caches' element type; ``slot_mapping: [T]``.
    Token ``t`` with slot ``s >= 0`` goes to block ``s // bs``, row ``s % bs``,
    for every kv-head.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    bs = int(block_size)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, row = s // bs, s % bs
        k_out[blk, :, row, :] = k[t]
        v_out[blk, :, row // 4, :, row % 4] = v[t]
    return k_out, v_out


def quantize_int8(x):
    """Quantise the last axis of fp32 ``x`` to int8 codes with one fp32 scale.

    Returns ``(codes int8[..., D], scale float32[...])`` with
    ``scale = absmax / 127`` and ``codes = clip(rint(x / scale), -127, 127)``.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)                       # exact in fp32
    s = (a / np.float32(127.0)).astype(np.float32)       # IEEE fp32 division
    nz = s > 0                                           # a == 0, or a/127 underflowed
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)     # IEEE fp32 division
    codes = np.clip(np.rint(ratio), -127, 127)           # rint: half to even
    codes = np.where(nz[..., None], codes, 0).astype(np.int8)
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return codes, s


def cache_write_int8(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping,
                     block_size):
    """Quantise new fp32 ``k, v: [T, Hkv, D]`` and scatter codes and scales.

    Returns copies of ``(k_cache, v_cache, k_scale, v_scale)``.  Each
    (token, kv-head) row of K and of V is quantised on its own.
    """
    kq, ks = quantize_int8(k)
    vq, vs = quantize_int8(v)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    ks_out = np.array(k_scale, copy=True)
    vs_out = np.array(v_scale, copy=True)
    bs = int(block_size)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, row = s // bs, s % bs
        k_out[blk, :, row, :] = kq[t]
        v_out[blk, :, row // 4, :, row % 4] = vq[t]
        ks_out[blk, :, row] = ks[t]
        vs_out[blk, :, row] = vs[t]
    return k_out, v_out, ks_out, vs_out
