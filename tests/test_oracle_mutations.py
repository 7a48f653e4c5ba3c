"""Plant plausible mistakes in the oracle (on the CPU) and require a pin to fail.

A pin suite that passes a broken oracle proves nothing; each mutation below is
an error a careful reader could still make (a transposed operand, a dropped
term, an off-by-one, a wrong rounding rule), and at least one check in
``oracle_pin_checks.ALL_CHECKS`` must reject it.
"""

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import fp8 as ofp8
from oracle import int4 as oint4
from oracle_pin_checks import ALL_CHECKS


def _gather_table_off_by_one(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                             kv_dtype, k_scale=None, v_scale=None):
    L, bs = int(context_len), int(block_size)
    D = k_cache.shape[-1]
    K = np.zeros((L, D))
    V = np.zeros((L, D))
    for j in range(oatt.n_blocks(L, bs)):
        rows = oatt.rows_in_block(L, bs, j)
        blk = int(block_table[min(j + 1, len(block_table) - 1)])
        K[j * bs:j * bs + rows] = oatt.widen(k_cache[blk, kv_head, :rows, :], kv_dtype)
        v_tok = np.swapaxes(v_cache[blk, kv_head], 1, 2).reshape(bs, D)[:rows]
        V[j * bs:j * bs + rows] = oatt.widen(v_tok, kv_dtype)
    return K, V


def _gather_no_v_scale(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                       kv_dtype, k_scale=None, v_scale=None):
    if kv_dtype == "i8":
        v_scale = np.ones_like(v_scale)
    return _orig_gather(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                        kv_dtype, k_scale, v_scale)


def _gather_v_rows_as_columns(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                              kv_dtype, k_scale=None, v_scale=None):
    # reads V tiles as if they were stored token-major like K (a transposed operand)
    K, _ = _orig_gather(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                        kv_dtype, k_scale, v_scale)
    L, bs = int(context_len), int(block_size)
    D = v_cache.shape[3]
    V = np.zeros((L, D))
    for j in range(oatt.n_blocks(L, bs)):
        rows = oatt.rows_in_block(L, bs, j)
        blk = int(block_table[j])
        flat = oatt.widen(v_cache[blk, kv_head], kv_dtype).reshape(-1)   # [D * bs]
        V[j * bs:j * bs + rows] = flat.reshape(bs, D)[:rows]
    return K, V


def _gather_v_group_index_swapped(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                                  kv_dtype, k_scale=None, v_scale=None):
    # reads token r of a V tile at [r % (bs/4), :, r // (bs/4)]: the group and
    # in-group indices exchanged
    K, _ = _orig_gather(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                        kv_dtype, k_scale, v_scale)
    L, bs = int(context_len), int(block_size)
    D = v_cache.shape[3]
    V = np.zeros((L, D))
    for j in range(oatt.n_blocks(L, bs)):
        rows = oatt.rows_in_block(L, bs, j)
        blk = int(block_table[j])
        tile = v_cache[blk, kv_head]
        for r in range(rows):
            V[j * bs + r] = oatt.widen(tile[r % (bs // 4), :, r // (bs // 4)], kv_dtype)
    return K, V


def _attend_no_scale(q_vec, K, V, scale):
    return _orig_attend(q_vec, K, V, 1.0)


def _attend_mean_norm(q_vec, K, V, scale):
    s = scale * (K @ np.asarray(q_vec, np.float64))
    p = np.exp(s - s.max())
    return (p @ V) / len(p)


def _attend_keys_as_values(q_vec, K, V, scale):
    return _orig_attend(q_vec, K, K, scale)


def _quant_half_away(x):
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(127)).astype(np.float32)
    safe = np.where(a > 0, s, np.float32(1)).astype(np.float32)
    r = (x / safe[..., None]).astype(np.float32)
    c = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127)
    c = np.where(a[..., None] > 0, c, 0).astype(np.int8)
    return c, np.where(a > 0, s, 0).astype(np.float32)


def _quant_scale_128(x):
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(128)).astype(np.float32)
    safe = np.where(a > 0, s, np.float32(1)).astype(np.float32)
    c = np.clip(np.rint((x / safe[..., None]).astype(np.float32)), -127, 127)
    c = np.where(a[..., None] > 0, c, 0).astype(np.int8)
    return c, np.where(a > 0, s, 0).astype(np.float32)


def _cache_write_row_shift(k, v, k_cache, v_cache, slot_mapping, block_size):
    shifted = np.where(np.asarray(slot_mapping) >= 0, np.asarray(slot_mapping) + 1, -1)
    return _orig_cache_write(k, v, k_cache, v_cache, shifted, block_size)


def _widen_bf16_shift15(x, kind):
    if kind == "bf16":
        bits = np.asarray(x).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return _orig_widen(x, kind)


def _fp8_table(bias=7, sub_exp=-6):
    vals = []
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 0xF and m == 7:
            vals.append(float("nan"))
        elif e == 0:
            vals.append(sign * 2.0 ** sub_exp * m / 8.0)
        else:
            vals.append(sign * 2.0 ** (e - bias) * (1 + m / 8.0))
    return np.array(vals)


_T_BIAS8 = _fp8_table(bias=8, sub_exp=-7)
_T_SUB = _fp8_table(sub_exp=-7)


def _fp8_encode_ties_away(v):
    v = np.asarray(v, dtype=np.float32)
    out = _orig_e4m3_encode(v)
    pos = _orig_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(v).astype(np.float64)
    for i in np.ndindex(v.shape):
        c = int(out[i]) & 0x7F
        for lo in (c - 1, c):  # a tie resolved toward the smaller neighbour moves up
            if 0 <= lo < 0x7E and a[i] == (pos[lo] + pos[lo + 1]) / 2:
                out[i] = (out[i] & 0x80) | (lo + 1)
    return out


def _fp8_encode_truncate(v):
    v = np.asarray(v, dtype=np.float32)
    pos = _orig_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    code = np.searchsorted(pos, a, side="right") - 1
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _fp8_quant_over_240(x):
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(240.0)).astype(np.float32)
    nz = s > 0
    safe = np.where(nz, s, np.float32(1.0)).astype(np.float32)
    codes = np.where(nz[..., None], ofp8.e4m3_encode((x / safe[..., None]).astype(np.float32)), 0)
    return codes.astype(np.uint8), np.where(nz, s, 0).astype(np.float32)


def _gather_fp8_no_v_scale(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                           kv_dtype, k_scale=None, v_scale=None):
    if kv_dtype == "fp8":
        v_scale = np.ones_like(v_scale)
    return _orig_gather(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                        kv_dtype, k_scale, v_scale)


def _mq_variant(shift=0, top_left=False, causal=True):
    def mq(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_heads, num_kv_heads,
           head_dim, block_size, kv_dtype, q_dtype, k_scale=None, v_scale=None, samples=None):
        H, Hkv, D = int(num_heads), int(num_kv_heads), int(head_dim)
        qs = [int(x) for x in query_start]
        out = np.zeros((qs[-1], H, D))
        for b in range(len(qs) - 1):
            L, n = int(context_lens[b]), qs[b + 1] - qs[b]
            for h in range(H):
                K, V = oatt.gather_kv(k_cache, v_cache, block_tables[b], L, block_size, oatt.kv_head_of(h, H, Hkv),
                                      kv_dtype, k_scale, v_scale)
                for i in range(n):
                    pos = (i if top_left else L - n + i) + shift
                    stop = L if not causal else max(1, min(L, pos + 1))
                    out[qs[b] + i, h] = oatt.attend_one(oatt.widen(q[qs[b] + i, h], q_dtype), K[:stop], V[:stop], scale)
        return out
    return mq


def _int4_unpack_swapped(packed, axis=-1):
    # high nibble taken as the lower dim
    b = np.moveaxis(np.asarray(packed, np.uint8).astype(np.int64), axis, -1)
    lo, hi = b >> 4, b & 0xF
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return np.moveaxis(out, -1, axis)


def _int4_unpack_unsigned(packed, axis=-1):
    b = np.moveaxis(np.asarray(packed, np.uint8).astype(np.int64), axis, -1)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return np.moveaxis(out, -1, axis)


def _int4_pack_swapped(codes, axis=-1):
    c = np.moveaxis(np.asarray(codes).astype(np.int64), axis, -1) & 0xF
    return np.moveaxis((c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8), -1, axis)


def _int4_quant_over_8(x):
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(8)).astype(np.float32)
    safe = np.where(a > 0, s, np.float32(1)).astype(np.float32)
    c = np.clip(np.rint((x / safe[..., None]).astype(np.float32)), -8, 7)
    c = np.where(a[..., None] > 0, c, 0).astype(np.int8)
    return c, np.where(a > 0, s, 0).astype(np.float32)


def _gather_int4_no_v_scale(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                            kv_dtype, k_scale=None, v_scale=None):
    if kv_dtype == "i4":
        v_scale = np.ones_like(v_scale)
    return _orig_gather(k_cache, v_cache, block_table, context_len, block_size, kv_head,
                        kv_dtype, k_scale, v_scale)


_T5_BIAS16 = np.array([ofp8.e5m2_value(c) / 2.0 for c in range(256)])


def _e5m2_encode_ties_away(v):
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    pos = ofp8.e5m2_decode(np.arange(0x7C, dtype=np.uint8))
    hi = np.minimum(np.searchsorted(pos, a, side="left"), 0x7B)
    lo = np.maximum(hi - 1, 0)
    code = np.where(pos[hi] - a <= a - pos[lo], hi, lo)
    code = np.where(a >= 57344.0, 0x7B, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _e5m2_quant_over_448(x):
    x = np.asarray(x, np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(448)).astype(np.float32)
    safe = np.where(a > 0, s, np.float32(1)).astype(np.float32)
    c = np.where(a[..., None] > 0, ofp8.e5m2_encode((x / safe[..., None]).astype(np.float32)), 0)
    return c.astype(np.uint8), np.where(a > 0, s, 0).astype(np.float32)


def _widen_e5m2_as_e4m3(x, kind):
    if kind == "e5m2":
        return ofp8.e4m3_decode(np.asarray(x).astype(np.uint8))
    return _orig_widen(x, kind)


_orig_e4m3_encode = ofp8.e4m3_encode
_orig_e4m3_decode = ofp8.e4m3_decode
_orig_gather = oatt.gather_kv
_orig_attend = oatt.attend_one
_orig_widen = oatt.widen
_orig_cache_write = ocache.cache_write

MUTATIONS = {
    "gqa_interleaved_heads": [(oatt, "kv_head_of", lambda h, H, Hkv: int(h) % int(Hkv))],
    "last_block_one_row_too_many": [
        (oatt, "rows_in_block",
         lambda L, bs, j: 0 if (j < 0 or j >= oatt.n_blocks(L, bs)) else min(int(bs), int(L) - j * int(bs) + 1))],
    "block_count_floor": [(oatt, "n_blocks", lambda L, bs: int(L) // int(bs))],
    "block_table_off_by_one": [(oatt, "gather_kv", _gather_table_off_by_one)],
    "v_tile_read_token_major": [(oatt, "gather_kv", _gather_v_rows_as_columns)],
    "v_group_index_swapped": [(oatt, "gather_kv", _gather_v_group_index_swapped)],
    "int8_v_scale_dropped": [(oatt, "gather_kv", _gather_no_v_scale)],
    "scale_dropped": [(oatt, "attend_one", _attend_no_scale)],
    "normalised_by_length": [(oatt, "attend_one", _attend_mean_norm)],
    "keys_used_as_values": [(oatt, "attend_one", _attend_keys_as_values)],
    "bf16_widen_wrong_shift": [(oatt, "widen", _widen_bf16_shift15)],
    "quant_round_half_away": [(ocache, "quantize_int8", _quant_half_away)],
    "quant_scale_over_128": [(ocache, "quantize_int8", _quant_scale_128)],
    "cache_write_row_shift": [(ocache, "cache_write", _cache_write_row_shift)],
    "fp8_exponent_bias_8": [(ofp8, "e4m3_decode", lambda c: _T_BIAS8[np.asarray(c, np.uint8)])],
    "fp8_subnormal_scale": [(ofp8, "e4m3_decode", lambda c: _T_SUB[np.asarray(c, np.uint8)])],
    "fp8_round_ties_away": [(ofp8, "e4m3_encode", _fp8_encode_ties_away)],
    "fp8_truncate": [(ofp8, "e4m3_encode", _fp8_encode_truncate)],
    "fp8_scale_over_240": [(ofp8, "quantize_fp8", _fp8_quant_over_240)],
    "fp8_v_scale_dropped": [(oatt, "gather_kv", _gather_fp8_no_v_scale)],
    "e5m2_exponent_bias_16": [(ofp8, "e5m2_decode", lambda c: _T5_BIAS16[np.asarray(c, np.uint8)])],
    "e5m2_round_ties_away": [(ofp8, "e5m2_encode", _e5m2_encode_ties_away)],
    "e5m2_scale_over_448": [(ofp8, "quantize_fp8_e5m2", _e5m2_quant_over_448)],
    "e5m2_read_as_e4m3": [(oatt, "widen", _widen_e5m2_as_e4m3)],
    "int4_nibbles_swapped": [(oint4, "unpack_int4", _int4_unpack_swapped)],
    "int4_no_sign_extension": [(oint4, "unpack_int4", _int4_unpack_unsigned)],
    "int4_pack_high_first": [(oint4, "pack_int4", _int4_pack_swapped)],
    "int4_scale_over_8": [(oint4, "quantize_int4", _int4_quant_over_8)],
    "int4_v_scale_dropped": [(oatt, "gather_kv", _gather_int4_no_v_scale)],
    "mq_excludes_own_token": [(oatt, "multi_query_attention", _mq_variant(shift=-1))],
    "mq_top_left_causal": [(oatt, "multi_query_attention", _mq_variant(top_left=True))],
    "mq_not_causal": [(oatt, "multi_query_attention", _mq_variant(causal=False))],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for module, attr, repl in MUTATIONS[name]:
        monkeypatch.setattr(module, attr, repl)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, repl)
    failed = []
    for check in ALL_CHECKS:
        try:
            check()
        except Exception:  # AssertionError or a shape error caused by the mistake
            failed.append(check.__name__)
    assert failed, f"mutation {name!r} passed every pin"
