"""INT4 KV-cache codes: the per-(token, kv-head) quantiser and nibble packing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

An INT4 KV cache keeps a 4-bit code per element and one scale per
(token, kv-head).  [ENG5] "KV-cache quantization": INT4 KV caches cost
little quality when calibrated per token, and the recommended scheme
scales per token and per head.  [LAYERS] 2.3: KV quantisation with
per-token scales, K and V quantised separately; 4 bits is possible but
harder on accuracy than 8.

Readings taken where the pages are silent:

* Codes are symmetric signed integers in [-7, 7]: ``s = absmax / 7`` (IEEE
  fp32 division), ``c = clip(rint(x / s), -7, 7)`` with ``rint`` rounding
  half to even; a row whose scale is 0 gets ``s = 0`` and codes 0.  This
  is the int8 quantiser with 7 in place of 127 (code -8 is never produced).
* Two codes share a byte, as 4-bit two's complement: each byte holds two
  consecutive head dims of one token, dim ``2j`` in the low nibble and dim
  ``2j + 1`` in the high nibble.  K tiles are ``[num_blocks, num_kv_heads,
  block_size, head_dim / 2]`` (byte ``j`` of a token's row) and V tiles
  ``[num_blocks, num_kv_heads, block_size / 4, head_dim / 2, 4]`` (byte
  ``[r // 4, j, r % 4]`` holds dims ``2j, 2j + 1`` of token ``r``), so no
  byte mixes two tokens.
* The outlier retention the pages pair with per-token-per-head scales
  (about 1% of channels kept in high precision) is not part of this format:
  the pages say neither how those channels are chosen nor how they are
  stored.
"""

import numpy as np

INT4_MAX = 7


def pack_int4(codes, axis=-1):
    """Pack int codes in [-8, 7] two per byte along ``axis`` (even length):
    element ``2j`` in the low nibble of byte ``j``, ``2j + 1`` in the high
    nibble, both as 4-bit two's complement.  Returns uint8 with that axis
    halved."""
    c = np.moveaxis(np.asarray(codes).astype(np.int64), axis, -1)
    if c.shape[-1] % 2:
        raise ValueError("packing needs an even number of elements")
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("codes outside [-8, 7]")
    nib = c & 0xF                                  # two's complement nibble
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return np.moveaxis(packed, -1, axis)


def unpack_int4(packed, axis=-1):
    """Inverse of ``pack_int4``: int8 codes with ``axis`` doubled."""
    b = np.moveaxis(np.asarray(packed, dtype=np.uint8).astype(np.int64), axis, -1)
    lo = b & 0xF
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return np.moveaxis(out, -1, axis)


def quantize_int4(x):
    """Quantise the last axis of fp32 ``x`` to codes in [-7, 7] with one fp32
    scale.  Returns ``(codes int8[..., D], scale float32[...])`` with
    ``scale = absmax / 7`` and ``codes = clip(rint(x / scale), -7, 7)``
    (unpacked)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)                       # exact in fp32
    s = (a / np.float32(INT4_MAX)).astype(np.float32)    # IEEE fp32 division
    nz = s > 0
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)     # IEEE fp32 division
    codes = np.clip(np.rint(ratio), -INT4_MAX, INT4_MAX) # rint: half to even
    codes = np.where(nz[..., None], codes, 0).astype(np.int8)
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return codes, s


def cache_write_int4(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, block_size):
    """Quantise new fp32 ``k, v: [T, Hkv, D]`` to INT4 and scatter packed
    codes and scales into copies of the caches (layouts above; slots as for
    the other writes, negative = no write).  Returns ``(k_cache, v_cache,
    k_scale, v_scale)``."""
    kq, ks = quantize_int4(k)
    vq, vs = quantize_int4(v)
    kp = pack_int4(kq, axis=-1)                          # [T, Hkv, D/2]
    vp = pack_int4(vq, axis=-1)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    ks_out = np.array(k_scale, copy=True)
    vs_out = np.array(v_scale, copy=True)
    bs = int(block_size)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, row = s // bs, s % bs
        k_out[blk, :, row, :] = kp[t]
        v_out[blk, :, row // 4, :, row % 4] = vp[t]
        ks_out[blk, :, row] = ks[t]
        vs_out[blk, :, row] = vs[t]
    return k_out, v_out, ks_out, vs_out
