"""ctypes binding of libpagedkv.so (argument marshalling only).

Every call here checks tensor shapes, dtypes and devices, then hands raw
device pointers, sizes and the current HIP stream to the C ABI declared in
``include/pagedkv.h``.  All computation happens in the library's kernels;
if the library is missing, every entry point raises.
"""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_ERR_NO_BLOCKS = range(6)
PKV_F32, PKV_BF16, PKV_I8, PKV_FP8, PKV_I4, PKV_FP8_E5M2 = range(6)

# INT4 caches are uint8 tensors holding two codes per byte
_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.int8: PKV_I8,
           torch.float8_e4m3fn: PKV_FP8, torch.float8_e5m2: PKV_FP8_E5M2, torch.uint8: PKV_I4}
_CODED = (PKV_I8, PKV_FP8, PKV_FP8_E5M2, PKV_I4)  # codes with per-(token, kv-head) scales


def _tile_shapes(kd, Hkv, bs, D):
    """Per-block K and V tile shapes of a cache of kind kd: [Hkv, bs, D] and
    [Hkv, bs/4, D, 4] (V in groups of 4 tokens: token r, dim d at
    [r // 4, d, r % 4]), or [Hkv, bs, D/2] and [Hkv, bs/4, D/2, 4] for INT4."""
    w = D // 2 if kd == PKV_I4 else D
    return (Hkv, bs, w), (Hkv, bs // 4, w, 4)

_lib = None
_lib_lock = threading.Lock()

c_i32, c_i64, c_f32, c_size, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                     ctypes.c_size_t, ctypes.c_void_p)

_DECODE_ARGS = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_f32,
                c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32, c_i32, c_i32,
                c_vp, c_size, c_vp]

SIGNATURES = {
    "pkv_kv_cache_write": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32,
                                   c_i64, c_i32, c_vp]),
    "pkv_kv_cache_write_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32,
                                       c_i32, c_i32, c_i64, c_vp]),
    "pkv_kv_cache_write_int8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32,
                                        c_i32, c_i32, c_i64, c_vp]),
    "pkv_kv_cache_write_fp8_e5m2": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32,
                                            c_i32, c_i32, c_i64, c_vp]),
    "pkv_kv_cache_write_int4": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32,
                                        c_i32, c_i32, c_i64, c_vp]),
    "pkv_paged_attention_workspace_size": (c_size, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                    c_i32]),
    "pkv_paged_attention_partition_tokens": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pkv_paged_attention_shares": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pkv_paged_attention_streams_cache": (c_i32, [c_i64, c_i32, c_i32, c_i32, c_i32]),
    "pkv_paged_attention_decode": (c_i32, _DECODE_ARGS),
    "pkv_paged_attention_decode_partitions": (c_i32, _DECODE_ARGS),
    "pkv_paged_attention_decode_noalloc": (c_i32, _DECODE_ARGS[:18] + [c_vp]),
    "pkv_paged_attention_decode_reduce": (c_i32, _DECODE_ARGS),
    "pkv_paged_attention_decode_step": (c_i32, _DECODE_ARGS[:2] + [c_vp, c_vp] + _DECODE_ARGS[2:]),
    "pkv_paged_attention_decode_step_partitions": (c_i32, _DECODE_ARGS[:2] + [c_vp, c_vp] + _DECODE_ARGS[2:]),
    "pkv_paged_attention_decode_cascade": (c_i32, _DECODE_ARGS[:8] + [c_vp, c_vp] + _DECODE_ARGS[8:16]
                                           + [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                              c_vp, c_size, c_vp]),
    "pkv_paged_attention_decode_cascade_step": (c_i32, _DECODE_ARGS[:2] + [c_vp, c_vp] + _DECODE_ARGS[2:8]
                                                + [c_vp, c_vp] + _DECODE_ARGS[8:16]
                                                + [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                   c_vp, c_size, c_vp]),
    "pkv_paged_attention_cascade_workspace_size": (c_size, [c_i32] * 11),
    "pkv_paged_attention_multi_query": (c_i32, _DECODE_ARGS[:8] + [c_vp] + _DECODE_ARGS[8:16]
                                        + [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_size, c_vp]),
    "pkv_paged_attention_multi_query_workspace_size": (c_size, [c_i32] * 9),
    "pkv_probe_tile_read": (c_i32, [c_vp, c_vp, c_i64, c_i32, c_i32, c_vp, c_vp]),
    "pkv_bm_create": (c_i32, [c_i64, c_i32, c_i64, c_vp, ctypes.POINTER(c_vp)]),
    "pkv_bm_destroy": (None, [c_vp]),
    "pkv_bm_num_free": (c_i64, [c_vp]),
    "pkv_bm_num_free_host": (c_i64, [c_vp]),
    "pkv_bm_new_sequence": (c_i32, [c_vp, ctypes.POINTER(c_i64)]),
    "pkv_bm_fork": (c_i32, [c_vp, c_i64, ctypes.POINTER(c_i64)]),
    "pkv_bm_free_sequence": (c_i32, [c_vp, c_i64]),
    "pkv_bm_append": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_i32, ctypes.POINTER(c_i32)]),
    "pkv_bm_length": (c_i64, [c_vp, c_i64]),
    "pkv_bm_block_table": (c_i32, [c_vp, c_i64, c_vp, c_i32, ctypes.POINTER(c_i32)]),
    "pkv_bm_refcounts": (c_i32, [c_vp, c_vp]),
    "pkv_bm_swap_out": (c_i32, [c_vp, c_i64, c_vp, c_i32, ctypes.POINTER(c_i32)]),
    "pkv_bm_swap_in": (c_i32, [c_vp, c_i64, c_vp, c_i32, ctypes.POINTER(c_i32)]),
    "pkv_copy_blocks": (c_i32, [c_vp] * 9 + [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "pkv_check_block_tables": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_i64]),
    "pkv_check_slot_mapping": (c_i32, [c_vp, c_i64, c_i32, c_i64]),
    "pkv_check_query_start": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32]),
    "pkv_check_groups": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}


def load(path=None):
    """Load (once) and return the ctypes handle of libpagedkv.so."""
    global _lib
    with _lib_lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is not built; run `python -m paged_kv_cache_29_amd.build` "
                "(the HIP library is required: there is no fallback path)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


class PagedKVError(RuntimeError):
    pass


def _check(status, what):
    if status == PKV_OK:
        return
    msg = load().pkv_last_error().decode(errors="replace")
    text = f"{what}: {msg}"
    if status in (PKV_ERR_INVALID, PKV_ERR_WORKSPACE):
        raise ValueError(text)
    if status == PKV_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    if status == PKV_ERR_NO_BLOCKS:
        from .blocks import OutOfBlocks
        raise OutOfBlocks(text)
    raise PagedKVError(text)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dense_on(t, device, name):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.device == device, f"{name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


# ------------------------------------------------------------------ writes
def kv_cache_write(k, v, k_cache, v_cache, slot_mapping):
    """Scatter new tokens' K/V rows ``[T, Hkv, D]`` into their cache slots."""
    dev = k_cache.device
    for n, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("slot_mapping", slot_mapping)):
        _dense_on(t, dev, n)
    _need(k_cache.dim() == 4 and v_cache.dim() == 5, "k_cache must be 4-D and v_cache 5-D")
    NB, Hkv, bs, D = k_cache.shape
    _need(tuple(v_cache.shape) == (NB, Hkv, bs // 4, D, 4), "v_cache must be [NB, Hkv, bs/4, D, 4]")
    _need(k.dim() == 3 and tuple(k.shape[1:]) == (Hkv, D) and k.shape == v.shape,
          "k, v must be [T, Hkv, D]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k.shape[0],),
          "slot_mapping must be int64 [T]")
    _need(k.dtype == v.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    dt = _DTYPES.get(k.dtype)
    _need(dt in (PKV_F32, PKV_BF16), "kv_cache_write takes float32 or bfloat16")
    st = load().pkv_kv_cache_write(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(slot_mapping), k.shape[0], Hkv, D, bs, NB, dt,
                                   _stream(dev))
    _check(st, "kv_cache_write")


def kv_cache_write_int8(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping):
    """Quantise fp32 K/V rows to int8 + per-(token, kv-head) scale and scatter."""
    _write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, torch.int8,
                 "pkv_kv_cache_write_int8")


def kv_cache_write_fp8(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping):
    """Quantise fp32 K/V rows to FP8 (E4M3) + per-(token, kv-head) scale and
    scatter; the caches are ``torch.float8_e4m3fn`` tensors."""
    _write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, torch.float8_e4m3fn,
                 "pkv_kv_cache_write_fp8")


def kv_cache_write_fp8_e5m2(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping):
    """Quantise fp32 K/V rows to FP8 in the E5M2 format + per-(token,
    kv-head) scale and scatter; the caches are ``torch.float8_e5m2``."""
    _write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, torch.float8_e5m2,
                 "pkv_kv_cache_write_fp8_e5m2")


def kv_cache_write_int4(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping):
    """Quantise fp32 K/V rows to INT4 codes in [-7, 7] + per-(token, kv-head)
    scale and scatter; the caches are uint8 tensors ``[NB, Hkv, bs, D/2]``
    (K) and ``[NB, Hkv, bs/4, D/2, 4]`` (V), two consecutive dims per byte."""
    _write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, torch.uint8,
                 "pkv_kv_cache_write_int4")


def _write_codes(k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, cache_dtype, entry):
    dev = k_cache.device
    for n, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("k_scale", k_scale), ("v_scale", v_scale), ("slot_mapping", slot_mapping)):
        _dense_on(t, dev, n)
    _need(k_cache.dim() == 4, "k_cache must be 4-d")
    NB, Hkv, bs, D = k_cache.shape
    kd = _DTYPES[cache_dtype]
    if kd == PKV_I4:
        D *= 2
    kt, vt = _tile_shapes(kd, Hkv, bs, D)
    _need(tuple(v_cache.shape) == (NB,) + vt, f"v_cache must be [NB, {', '.join(map(str, vt))}]")
    _need(k_cache.dtype == v_cache.dtype == cache_dtype, f"{cache_dtype} caches expected")
    _need(k.dtype == v.dtype == torch.float32, "k, v must be float32")
    _need(k.dim() == 3 and tuple(k.shape[1:]) == (Hkv, D) and k.shape == v.shape,
          "k, v must be [T, Hkv, D]")
    _need(tuple(k_scale.shape) == (NB, Hkv, bs) and k_scale.shape == v_scale.shape
          and k_scale.dtype == v_scale.dtype == torch.float32, "scales must be float32 [NB, Hkv, bs]")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (k.shape[0],),
          "slot_mapping must be int64 [T]")
    st = getattr(load(), entry)(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                _ptr(v_scale), _ptr(slot_mapping), k.shape[0], Hkv, D, bs, NB,
                                _stream(dev))
    _check(st, entry[4:])


# ------------------------------------------------------------------ decode
def partition_tokens(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, requested=0):
    return int(load().pkv_paged_attention_partition_tokens(num_seqs, num_kv_heads, block_size,
                                                           max_blocks_per_seq, requested))


def balanced_shares(num_seqs, num_kv_heads, block_size, max_blocks_per_seq, kv_dtype, requested=0):
    """Balanced shares decode uses for a cache of torch dtype ``kv_dtype``
    (0: fixed partitions)."""
    return int(load().pkv_paged_attention_shares(num_seqs, num_kv_heads, block_size, max_blocks_per_seq,
                                                 requested, _DTYPES[kv_dtype]))


def streams_cache(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype):
    """Whether one-query decode reads a cache pool of these sizes (torch
    dtype ``kv_dtype``; for INT4 ``head_dim`` is the unpacked width) with the
    non-temporal load hint."""
    return bool(load().pkv_paged_attention_streams_cache(int(num_blocks), num_kv_heads, block_size, head_dim,
                                                         _DTYPES[kv_dtype]))


def workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   partition_tokens=0):
    return int(load().pkv_paged_attention_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                         head_dim, block_size, max_blocks_per_seq,
                                                         partition_tokens))


_ws_cache = {}
_NO_WORKSPACE = object()


def _workspace(device, nbytes):
    key = (device.type, device.index)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _marshal_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_heads,
                    num_kv_heads, head_dim, block_size, k_scale=None, v_scale=None,
                    partition_tokens=0, workspace=None):
    dev = q.device
    for n, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                 ("block_tables", block_tables), ("context_lens", context_lens)):
        _dense_on(t, dev, n)
    _need(q.dim() == 3 and tuple(q.shape[1:]) == (num_heads, head_dim), "q must be [B, H, D]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(k_cache.dim() == 4, "k_cache must be [NB, Hkv, bs, D]")
    NB = k_cache.shape[0]
    kt, vt = _tile_shapes(_DTYPES.get(k_cache.dtype), num_kv_heads, block_size, head_dim)
    _need(tuple(k_cache.shape) == (NB,) + kt,
          "k_cache must be [NB, Hkv, bs, D] ([NB, Hkv, bs, D/2] for INT4)")
    _need(tuple(v_cache.shape) == (NB,) + vt,
          "v_cache must be [NB, Hkv, bs/4, D, 4] ([NB, Hkv, bs/4, D/2, 4] for INT4)")
    _need(k_cache.dtype == v_cache.dtype, "k_cache and v_cache dtypes differ")
    B = q.shape[0]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == B,
          "block_tables must be int32 [B, MB]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (B,),
          "context_lens must be int32 [B]")
    qd, kd = _DTYPES.get(q.dtype), _DTYPES.get(k_cache.dtype)
    _need(qd is not None and kd is not None, "unsupported dtype")
    if kd in _CODED:
        for n, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            _dense_on(t, dev, n)
            _need(t.dtype == torch.float32 and tuple(t.shape) == (NB, num_kv_heads, block_size),
                  f"{n} must be float32 [NB, Hkv, bs]")
    MB = block_tables.shape[1]
    if workspace is _NO_WORKSPACE:  # the caller sizes its own workspace
        return (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                _ptr(k_scale if kd in _CODED else None), _ptr(v_scale if kd in _CODED else None),
                _ptr(block_tables), _ptr(context_lens), float(scale), B, num_heads, num_kv_heads,
                head_dim, block_size, MB, NB, qd, kd, int(partition_tokens), None, 0, _stream(dev))
    need = workspace_size(B, num_heads, num_kv_heads, head_dim, block_size, MB, partition_tokens)
    if workspace is None:
        workspace = _workspace(dev, need) if need else None
    else:
        _dense_on(workspace, dev, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale if kd in _CODED else None), _ptr(v_scale if kd in _CODED else None),
            _ptr(block_tables), _ptr(context_lens), float(scale), B, num_heads, num_kv_heads,
            head_dim, block_size, MB, NB, qd, kd, int(partition_tokens), _ptr(workspace),
            ws_bytes, _stream(dev))


def cascade_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, num_groups, max_group_size, max_shared_blocks,
                           partition_tokens=0, prefix_partition_tokens=0):
    return int(load().pkv_paged_attention_cascade_workspace_size(
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_groups,
        max_group_size, max_shared_blocks, partition_tokens, prefix_partition_tokens))


def paged_attention_decode_cascade(out, q, k_cache, v_cache, block_tables, context_lens,
                                   group_start, group_shared_blocks, scale, num_heads,
                                   num_kv_heads, head_dim, block_size, max_group_size,
                                   max_shared_blocks, k_scale=None, v_scale=None,
                                   partition_tokens=0, prefix_partition_tokens=0,
                                   workspace=None, k_new=None, v_new=None):
    """Decode attention with each group's shared blocks read once for the group.

    ``group_start`` (int32 ``[num_groups + 1]``) and ``group_shared_blocks``
    (int32 ``[num_groups]``) are device tensors; ``max_group_size`` and
    ``max_shared_blocks`` are host-side bounds on them (see
    ``blocks.cascade_groups``, which computes all four from block tables).
    With ``k_new`` and ``v_new`` ([B, Hkv, D], as for the fused step) it is
    the fused step: each sequence's new token is written at position L-1
    first (``pkv_paged_attention_decode_cascade_step``)."""
    dev = q.device
    for n, t in (("group_start", group_start), ("group_shared_blocks", group_shared_blocks)):
        _dense_on(t, dev, n)
        _need(t.dtype == torch.int32 and t.dim() == 1, f"{n} must be int32 1-D")
    G = group_shared_blocks.numel()
    _need(group_start.numel() == G + 1, "group_start must have num_groups + 1 entries")
    args = list(_marshal_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                num_heads, num_kv_heads, head_dim, block_size, k_scale, v_scale,
                                partition_tokens, workspace=_NO_WORKSPACE))
    B, MB = q.shape[0], block_tables.shape[1]
    need = cascade_workspace_size(B, num_heads, num_kv_heads, head_dim, block_size, MB, G,
                                  max_group_size, max_shared_blocks, partition_tokens,
                                  prefix_partition_tokens)
    if workspace is None:
        workspace = _workspace(dev, need) if need else None
    else:
        _dense_on(workspace, dev, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    # decode's arguments up to num_blocks, then the cascade's
    tail = (*args[8:16], G, int(max_group_size), int(max_shared_blocks), args[16], args[17], args[18],
            int(prefix_partition_tokens), _ptr(workspace), ws_bytes, args[21])
    groups = (_ptr(group_start), _ptr(group_shared_blocks))
    if k_new is None and v_new is None:
        st = load().pkv_paged_attention_decode_cascade(*args[:8], *groups, *tail)
        _check(st, "paged_attention_decode_cascade")
        return
    want = torch.float32 if _DTYPES.get(k_cache.dtype) in _CODED else k_cache.dtype
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t is not None, "the fused step needs both k_new and v_new")
        _dense_on(t, dev, n)
        _need(tuple(t.shape) == (B, num_kv_heads, head_dim), f"{n} must be [B, Hkv, D]")
        _need(t.dtype == want, f"{n} must be {want}")
    st = load().pkv_paged_attention_decode_cascade_step(*args[:2], _ptr(k_new), _ptr(v_new), *args[2:8],
                                                        *groups, *tail)
    _check(st, "paged_attention_decode_cascade (fused step)")


def multi_query_workspace_size(num_seqs, num_query_tokens, max_queries_per_seq, num_heads,
                               num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               partition_tokens=0):
    return int(load().pkv_paged_attention_multi_query_workspace_size(
        num_seqs, num_query_tokens, max_queries_per_seq, num_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, partition_tokens))


def paged_attention_multi_query(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                                scale, num_heads, num_kv_heads, head_dim, block_size,
                                max_queries_per_seq, k_scale=None, v_scale=None,
                                partition_tokens=0, workspace=None):
    """Causal attention of each sequence's new tokens (rows ``query_start[b]
    .. query_start[b+1]-1`` of ``q`` / ``out``, ``[T, H, D]``), the last of its
    context, over its paged context; ``query_start`` is a device int32
    ``[B + 1]`` tensor and ``max_queries_per_seq`` a host bound on the
    per-sequence counts."""
    dev = q.device
    for n, t in (("out", out), ("q", q), ("block_tables", block_tables),
                 ("context_lens", context_lens), ("query_start", query_start)):
        _dense_on(t, dev, n)
    B = context_lens.shape[0]
    _need(query_start.dtype == torch.int32 and tuple(query_start.shape) == (B + 1,),
          "query_start must be int32 [B + 1]")
    _need(q.dim() == 3 and tuple(q.shape[1:]) == (num_heads, head_dim), "q must be [T, H, D]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    T = q.shape[0]
    # decode's checks on the caches and tables, with a stand-in [B, H, D] query
    stand = torch.empty((B, num_heads, head_dim), dtype=q.dtype, device=dev) if B else q[:0]
    args = list(_marshal_decode(stand, stand, k_cache, v_cache, block_tables, context_lens, scale,
                                num_heads, num_kv_heads, head_dim, block_size, k_scale, v_scale,
                                partition_tokens, workspace=_NO_WORKSPACE))
    MB = block_tables.shape[1]
    need = multi_query_workspace_size(B, T, max_queries_per_seq, num_heads, num_kv_heads, head_dim,
                                      block_size, MB, partition_tokens)
    if workspace is None:
        workspace = _workspace(dev, need) if need else None
    else:
        _dense_on(workspace, dev, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().pkv_paged_attention_multi_query(
        _ptr(out), _ptr(q), *args[2:8], _ptr(query_start), *args[8:16], T, int(max_queries_per_seq),
        args[16], args[17], int(partition_tokens), _ptr(workspace), ws_bytes, args[21])
    _check(st, "paged_attention_multi_query")


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           num_heads, num_kv_heads, head_dim, block_size, k_scale=None,
                           v_scale=None, partition_tokens=0, workspace=None):
    """One decode step of attention over the paged cache; writes ``out``."""
    args = _marshal_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           num_heads, num_kv_heads, head_dim, block_size, k_scale, v_scale,
                           partition_tokens, workspace)
    _check(load().pkv_paged_attention_decode(*args), "paged_attention_decode")


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                   num_heads, num_kv_heads, head_dim, block_size, k_scale=None,
                                   v_scale=None):
    """paged_attention_decode without a workspace: the split-context
    partials go to the library's own per-GPU scratch (automatic partitions;
    calls that overlap on one GPU race)."""
    args = _marshal_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_heads,
                           num_kv_heads, head_dim, block_size, k_scale, v_scale, 0,
                           workspace=_NO_WORKSPACE)
    _check(load().pkv_paged_attention_decode_noalloc(*args[:18], args[21]),
           "paged_attention_decode_noalloc")


def paged_attention_decode_partitions(*args, **kwargs):
    """First of decode's two launches; same arguments as paged_attention_decode."""
    _check(load().pkv_paged_attention_decode_partitions(*_marshal_decode(*args, **kwargs)),
           "paged_attention_decode_partitions")


def paged_attention_decode_reduce(*args, **kwargs):
    """Second of decode's two launches; same arguments as paged_attention_decode."""
    _check(load().pkv_paged_attention_decode_reduce(*_marshal_decode(*args, **kwargs)),
           "paged_attention_decode_reduce")


def _marshal_step(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                  num_heads, num_kv_heads, head_dim, block_size, k_scale=None, v_scale=None,
                  partition_tokens=0, workspace=None):
    args = _marshal_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_heads,
                           num_kv_heads, head_dim, block_size, k_scale, v_scale, partition_tokens,
                           workspace)
    dev = q.device
    want = torch.float32 if _DTYPES.get(k_cache.dtype) in _CODED else k_cache.dtype
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _dense_on(t, dev, n)
        _need(tuple(t.shape) == (q.shape[0], num_kv_heads, head_dim), f"{n} must be [B, Hkv, D]")
        _need(t.dtype == want, f"{n} must be {want}")
    return args[:2] + (_ptr(k_new), _ptr(v_new)) + args[2:]


def paged_attention_decode_step(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                context_lens, scale, num_heads, num_kv_heads, head_dim,
                                block_size, k_scale=None, v_scale=None, partition_tokens=0,
                                workspace=None):
    """Fused decode step: append each sequence's new token at position L-1
    (through its block table), then attend; writes ``out`` and the caches."""
    args = _marshal_step(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                         num_heads, num_kv_heads, head_dim, block_size, k_scale, v_scale,
                         partition_tokens, workspace)
    _check(load().pkv_paged_attention_decode_step(*args), "paged_attention_decode_step")


def paged_attention_decode_step_partitions(*args, **kwargs):
    """First launch of the fused step; the second is paged_attention_decode_reduce."""
    _check(load().pkv_paged_attention_decode_step_partitions(*_marshal_step(*args, **kwargs)),
           "paged_attention_decode_step_partitions")


def probe_tile_read(pool, tile_ids, sink, grid, check_ids=True, streaming=False):
    """Measurement aid: read the 4096-byte tiles ``pool[4096*id : 4096*(id+1)]``
    for every id in ``tile_ids`` (the decode kernel's access pattern, no
    arithmetic); ``sink`` is uint32-sized ``[grid * 256]`` and is overwritten.
    ``streaming`` loads with the non-temporal hint.

    ``check_ids`` range-checks the ids first (a device reduction and a
    synchronisation); a timing loop checks once and then passes False."""
    dev = pool.device
    for n, t in (("pool", pool), ("tile_ids", tile_ids), ("sink", sink)):
        _dense_on(t, dev, n)
    _need(tile_ids.dtype == torch.int32 and tile_ids.dim() == 1, "tile_ids must be int32 [N]")
    _need(sink.numel() * sink.element_size() >= 4 * 256 * int(grid), "sink must hold grid * 256 uint32")
    pool_tiles = pool.numel() * pool.element_size() // 4096
    _need(pool.numel() * pool.element_size() % 4096 == 0, "pool must be whole 4096-byte tiles")
    if check_ids and tile_ids.numel():  # an id outside the pool would be a memory fault
        _need(int(tile_ids.min()) >= 0 and int(tile_ids.max()) < pool_tiles,
              "tile_ids must name tiles inside pool")
    st = load().pkv_probe_tile_read(_ptr(pool), _ptr(tile_ids), tile_ids.numel(), int(grid),
                                    1 if streaming else 0, _ptr(sink), _stream(dev))
    _check(st, "probe_tile_read")


def copy_blocks(dst, src, pairs):
    """Copy whole blocks from pool ``src`` to pool ``dst``: block ``pairs[i,
    0]`` of ``src`` to block ``pairs[i, 1]`` of ``dst`` (K tiles, V tiles and,
    for int8 / FP8 / INT4 pools, scale rows).  A pool is ``(k_cache, v_cache)`` or
    ``(k_cache, v_cache, k_scale, v_scale)``, on the device or in pinned host
    memory (swapping); ``pairs`` is an int32 ``[n, 2]`` tensor on the device.
    Runs on the current stream of the device pool's GPU."""
    dst, src = tuple(dst), tuple(src)
    _need(len(dst) == len(src) and len(dst) in (2, 4), "pools are (k, v) or (k, v, k_scale, v_scale)")
    dev = pairs.device
    _need(dev.type == "cuda", "pairs must be on the device")
    _need(pairs.dtype == torch.int32 and pairs.dim() == 2 and pairs.shape[1] == 2 and
          pairs.is_contiguous(), "pairs must be contiguous int32 [n, 2]")
    for pool, name in ((dst, "dst"), (src, "src")):
        for t in pool:
            _need(isinstance(t, torch.Tensor) and t.is_contiguous(), f"{name} pool tensors must be contiguous")
            _need(t.device == dev or (t.device.type == "cpu" and t.is_pinned()),
                  f"{name} pool tensors must be on {dev} or in pinned host memory")
    kd = _DTYPES.get(dst[0].dtype)
    _need(kd is not None and all(_DTYPES.get(t.dtype) == kd for t in (dst[1], src[0], src[1])),
          "pool dtypes must match")
    coded = kd in _CODED
    _need(coded == (len(dst) == 4), "int8 / FP8 / INT4 pools carry scales; fp32 / bf16 pools do not")
    k = dst[0]
    _need(k.dim() == 4, "k_cache must be [NB, Hkv, bs, D]")
    _, Hkv, bs, D = k.shape
    if kd == PKV_I4:
        D *= 2
    kt, vt = _tile_shapes(kd, Hkv, bs, D)
    for pool in (dst, src):
        _need(tuple(pool[0].shape[1:]) == kt and tuple(pool[1].shape[1:]) == vt,
              "pools must share Hkv, bs and D")
    sc = (lambda pool: (_ptr(pool[2]), _ptr(pool[3]))) if coded else (lambda pool: (_ptr(None), _ptr(None)))
    st = load().pkv_copy_blocks(_ptr(dst[0]), _ptr(dst[1]), *sc(dst), _ptr(src[0]), _ptr(src[1]),
                                *sc(src), _ptr(pairs), pairs.shape[0], Hkv, D, bs, kd, _stream(dev))
    _check(st, "copy_blocks")


# ---- host checks of the device-data preconditions (include/pagedkv_debug.h)

def _host_i(a, dtype):
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, ctypes.c_void_p(a.ctypes.data if a.size else 0)


def check_block_tables(block_tables, context_lens, block_size, num_blocks):
    """Raise ValueError unless every context fits its table row and every
    block id it uses is in [0, num_blocks) (``pkv_check_block_tables``)."""
    import numpy as np
    bt, pbt = _host_i(block_tables, np.int32)
    cl, pcl = _host_i(context_lens, np.int32)
    _need(bt.ndim == 2 and cl.ndim == 1 and cl.shape[0] == bt.shape[0], "block_tables [B, MB], context_lens [B]")
    _check(load().pkv_check_block_tables(pbt, pcl, bt.shape[0], bt.shape[1], block_size, num_blocks),
           "check_block_tables")


def check_slot_mapping(slot_mapping, block_size, num_blocks):
    """Raise ValueError if a slot is past the pool or two tokens share one
    (``pkv_check_slot_mapping``; negative slots are skipped)."""
    import numpy as np
    sm, psm = _host_i(slot_mapping, np.int64)
    _need(sm.ndim == 1, "slot_mapping must be 1-D")
    _check(load().pkv_check_slot_mapping(psm, sm.shape[0], block_size, num_blocks), "check_slot_mapping")


def check_query_start(query_start, context_lens, num_query_tokens, max_queries_per_seq):
    """Raise ValueError unless query_start is a valid prefix sum of the new
    tokens per sequence (``pkv_check_query_start``)."""
    import numpy as np
    qs, pqs = _host_i(query_start, np.int32)
    cl, pcl = _host_i(context_lens, np.int32)
    _need(qs.ndim == 1 and cl.ndim == 1 and qs.shape[0] == cl.shape[0] + 1,
          "query_start [B + 1], context_lens [B]")
    _check(load().pkv_check_query_start(pqs, pcl, cl.shape[0], num_query_tokens, max_queries_per_seq),
           "check_query_start")


def check_groups(group_start, group_shared_blocks, block_tables, context_lens, block_size,
                 max_group_size, max_shared_blocks):
    """Raise ValueError unless the shared-prefix groups are valid for the
    block tables (``pkv_check_groups``)."""
    import numpy as np
    gs, pgs = _host_i(group_start, np.int32)
    gsb, pgsb = _host_i(group_shared_blocks, np.int32)
    bt, pbt = _host_i(block_tables, np.int32)
    cl, pcl = _host_i(context_lens, np.int32)
    _need(gs.ndim == 1 and gsb.ndim == 1 and gs.shape[0] == gsb.shape[0] + 1,
          "group_start [G + 1], group_shared_blocks [G]")
    _need(bt.ndim == 2 and cl.ndim == 1 and cl.shape[0] == bt.shape[0], "block_tables [B, MB], context_lens [B]")
    _check(load().pkv_check_groups(pgs, pgsb, pbt, pcl, bt.shape[0], bt.shape[1], block_size, gsb.shape[0],
                                   max_group_size, max_shared_blocks), "check_groups")
