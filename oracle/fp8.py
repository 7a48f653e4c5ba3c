"""FP8 codes (E4M3 and E5M2) and the FP8 KV-cache quantisers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

An FP8 KV cache keeps one 8-bit float per element plus one scale per
(token, kv-head), computed online from the row itself ([ENG5] "KV-cache
quantization": FP8 KV caches with per-token scales, which cost almost
nothing because the scale is computed on the fly; [LAYERS] 2.3: per-token
scales, K and V quantised separately).

Readings taken where the pages are silent:

* The 8-bit format is E4M3 in its OCP form: sign, 4 exponent bits (bias 7),
  3 mantissa bits, no infinities, codes 0x7F / 0xFF are NaN.  Code
  ``s eeee mmm`` is ``(-1)^s 2^(e-7) (1 + m/8)`` for ``e >= 1`` and
  ``(-1)^s 2^-6 (m/8)`` for ``e = 0``; the largest finite value is 448.
* The scale maps the row's absolute maximum onto the largest finite code,
  ``s = absmax / 448`` (IEEE fp32 division), as the int8 scale maps it onto
  127; elements are ``x / s`` (fp32 division) rounded to the nearest E4M3
  value, ties to the even code (mantissa LSB 0), magnitudes beyond 448
  (possible only through the rounding of ``s``) saturate to 448; the sign of
  a zero is kept.  A row whose scale is 0 gets ``s = 0`` and codes 0.
* The other common FP8 format, E5M2 (sign, 5 exponent bits with bias 15,
  2 mantissa bits: ``(-1)^s 2^(e-15) (1 + m/4)``, subnormals
  ``(-1)^s 2^-14 (m/4)``, ``e = 31`` infinities (m = 0) and NaNs), is read
  the same way: the scale maps the row maximum onto its largest finite
  value, ``s = absmax / 57344``; codes are the nearest E5M2 value of
  ``x / s``, ties to the even code, saturating at 57344 (never infinity).
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one E4M3 code (int 0..255) as a Python float; NaN for 0x7F / 0xFF."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite values, codes 0x00 .. 0x7E, in increasing order
_POS = _TABLE[:0x7F]


def e4m3_decode(codes):
    """Exact fp64 values of E4M3 codes (uint8 array)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """Nearest E4M3 code of each fp32 value (ties to the even code,
    saturating at 448, sign kept).  Inputs must not be NaN."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    neg = np.signbit(v)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)          # saturate
    code = np.where(a <= _POS[0], 0, code)              # exact zero
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


E5M2_MAX = 57344.0


def e5m2_value(code):
    """Value of one E5M2 code (int 0..255) as a Python float: +-inf for
    0x7C / 0xFC, NaN for 0x7D..0x7F and 0xFD..0xFF."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (2.0 ** -14) * (m / 4.0)
    return sign * (2.0 ** (e - 15)) * (1.0 + m / 4.0)


_TABLE5 = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite values, codes 0x00 .. 0x7B, in increasing order
_POS5 = _TABLE5[:0x7C]


def e5m2_decode(codes):
    """Exact fp64 values of E5M2 codes (uint8 array)."""
    return _TABLE5[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode(v):
    """Nearest finite E5M2 code of each fp32 value (ties to the even code,
    saturating at 57344, sign kept).  Inputs must not be NaN."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    neg = np.signbit(v)
    hi = np.searchsorted(_POS5, a, side="left")         # first value >= a
    hi = np.minimum(hi, 0x7B)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS5[lo]
    d_hi = _POS5[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E5M2_MAX, 0x7B, code)          # saturate
    code = np.where(a <= _POS5[0], 0, code)             # exact zero
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_fp8(x):
    """Quantise the last axis of fp32 ``x`` to E4M3 codes with one fp32 scale.

    Returns ``(codes uint8[..., D], scale float32[...])``, ``scale = absmax /
    448`` and ``codes = e4m3_encode(x / scale)``.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)                       # exact in fp32
    s = (a / np.float32(E4M3_MAX)).astype(np.float32)    # IEEE fp32 division
    nz = s > 0
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)     # IEEE fp32 division
    codes = np.where(nz[..., None], e4m3_encode(ratio), 0).astype(np.uint8)
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return codes, s


def quantize_fp8_e5m2(x):
    """Quantise the last axis of fp32 ``x`` to E5M2 codes with one fp32 scale:
    ``scale = absmax / 57344``, ``codes = e5m2_encode(x / scale)``."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(E5M2_MAX)).astype(np.float32)    # IEEE fp32 division
    nz = s > 0
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    ratio = (x / safe[..., None]).astype(np.float32)     # IEEE fp32 division
    codes = np.where(nz[..., None], e5m2_encode(ratio), 0).astype(np.uint8)
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return codes, s


def cache_write_fp8(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, block_size,
                    quantize=None):
    """Quantise new fp32 ``k, v: [T, Hkv, D]`` to E4M3 (or with ``quantize``,
    e.g. ``quantize_fp8_e5m2``) and scatter codes and scales into copies of
    the caches (same slots and layout as the int8 write).  Returns
    ``(k_cache, v_cache, k_scale, v_scale)``."""
    q = quantize_fp8 if quantize is None else quantize
    kq, ks = q(k)
    vq, vs = q(v)
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


def cache_write_fp8_e5m2(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, block_size):
    """The FP8 cache write with E5M2 codes."""
    return cache_write_fp8(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, block_size,
                           quantize=quantize_fp8_e5m2)
