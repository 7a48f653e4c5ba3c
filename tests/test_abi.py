"""The C ABI on a host without a GPU: exports, validation and error codes.

Every call here fails validation (or is a size query) before the library
touches the HIP runtime, so nothing is launched.
"""

import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_29_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
F32, BF16, I8, FP8, I4, E5M2 = range(6)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "pkv_paged_attention_decode" in names and "pkv_kv_cache_write" in names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", out))
    for n in names:
        assert n in exported, f"{n} declared in include/ but not exported"
        assert hasattr(lib, n)
    # the binding declares a signature for every exported entry point
    assert set(names) == set(_lib.SIGNATURES)


def test_version(lib):
    assert lib.pkv_version() == b"0.1.0"


def _fake(n):
    # distinct non-null host addresses: never dereferenced, validation fails first
    return ctypes.c_void_p(0x1000 * n)


def _decode(lib, **over):
    a = dict(out=_fake(1), q=_fake(2), k_cache=_fake(3), v_cache=_fake(4), k_scale=None,
             v_scale=None, block_tables=_fake(5), context_lens=_fake(6), scale=0.125,
             num_seqs=4, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
             max_blocks_per_seq=13, num_blocks=32, q_dtype=BF16, kv_dtype=BF16,
             partition_tokens=0, workspace=None, workspace_bytes=0, stream=None)
    a.update(over)
    st = lib.pkv_paged_attention_decode(*a.values())
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("over,code,frag", [
    (dict(out=None), INVALID, "null pointer"),
    (dict(num_seqs=-1), INVALID, "num_seqs"),
    (dict(num_heads=6, num_kv_heads=4), INVALID, "multiple"),
    (dict(num_heads=0), INVALID, "positive"),
    (dict(max_blocks_per_seq=0), INVALID, "max_blocks_per_seq"),
    (dict(num_blocks=0), INVALID, "num_blocks"),
    (dict(scale=float("nan")), INVALID, "finite"),
    (dict(scale=float("inf")), INVALID, "finite"),
    (dict(head_dim=96), UNSUPPORTED, "head_dim"),
    (dict(block_size=8), UNSUPPORTED, "block_size"),
    (dict(num_heads=24, num_kv_heads=8), UNSUPPORTED, "not in {1, 2, 4, 8, 16}"),
    (dict(num_heads=64, num_kv_heads=2), UNSUPPORTED, "not in {1, 2, 4, 8, 16}"),
    (dict(q_dtype=F32, kv_dtype=BF16), UNSUPPORTED, "not supported"),
    (dict(q_dtype=BF16, kv_dtype=F32), UNSUPPORTED, "not supported"),
    (dict(q_dtype=F32, kv_dtype=I8), UNSUPPORTED, "not supported"),
    (dict(kv_dtype=I8), INVALID, "k_scale"),
    (dict(kv_dtype=I4), INVALID, "k_scale"),
    (dict(kv_dtype=E5M2), INVALID, "k_scale"),
    (dict(kv_dtype=6, k_scale=_fake(9), v_scale=_fake(10)), UNSUPPORTED, "not supported"),
    (dict(q_dtype=F32, kv_dtype=I4), UNSUPPORTED, "not supported"),
    (dict(k_scale=_fake(7)), INVALID, "must be NULL"),
    (dict(partition_tokens=48), INVALID, "partition_tokens"),
    (dict(partition_tokens=16), INVALID, "partition_tokens"),
    (dict(partition_tokens=4096), INVALID, "partition_tokens"),
    (dict(max_blocks_per_seq=2048, partition_tokens=256), WORKSPACE, "workspace"),
])
def test_decode_rejects(lib, over, code, frag):
    st, msg = _decode(lib, **over)
    assert st == code, msg
    assert frag in msg


def test_decode_workspace_checks(lib):
    need = lib.pkv_paged_attention_workspace_size(4, 8, 2, 64, 16, 2048, 256)
    assert need > 0
    st, msg = _decode(lib, max_blocks_per_seq=2048, partition_tokens=256,
                      workspace=ctypes.c_void_p(0x100000), workspace_bytes=need - 1)
    assert st == WORKSPACE and "required" in msg
    st, msg = _decode(lib, max_blocks_per_seq=2048, partition_tokens=256,
                      workspace=ctypes.c_void_p(0x100010), workspace_bytes=need)
    assert st == WORKSPACE and "aligned" in msg


def test_decode_empty_batch_is_noop(lib):
    st, msg = _decode(lib, num_seqs=0, out=None, q=None, k_cache=None, v_cache=None,
                      block_tables=None, context_lens=None)
    assert st == OK and msg == ""


def test_workspace_and_partition_queries(lib):
    ws = lib.pkv_paged_attention_workspace_size
    pt = lib.pkv_paged_attention_partition_tokens
    # one partition covers the context -> no workspace
    assert ws(4, 4, 4, 64, 16, 13, 0) == 0
    assert pt(4, 4, 16, 13, 0) == 256
    assert pt(32, 32, 16, 128, 0) == 2048     # 7B shape: one partition per sequence
    assert pt(50, 8, 16, 2048, 0) == 2048
    # explicit partition length: B*H*P rows of (D + 2) floats, 256-byte aligned pieces
    P = 2048 * 16 // 512
    rows = 50 * 64 * P
    expect = -(-rows * 128 * 4 // 256) * 256 + 2 * (-(-rows * 4 // 256) * 256)
    assert ws(50, 64, 8, 128, 16, 2048, 512) == expect
    assert pt(50, 8, 16, 2048, 512) == 512
    assert pt(50, 8, 16, 2048, 100) == 0
    assert ws(50, 64, 8, 96, 16, 2048, 512) == 0       # invalid head_dim
    assert pt(1, 1, 16, 1, 0) >= 32


def _write(lib, **over):
    a = dict(k=_fake(1), v=_fake(2), k_cache=_fake(3), v_cache=_fake(4), slots=_fake(5),
             num_tokens=8, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=64,
             dtype=BF16, stream=None)
    a.update(over)
    st = lib.pkv_kv_cache_write(*a.values())
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("over,code", [
    (dict(k=None), INVALID),
    (dict(slots=None), INVALID),
    (dict(num_tokens=-1), INVALID),
    (dict(num_kv_heads=0), INVALID),
    (dict(num_blocks=0), INVALID),
    (dict(head_dim=80), UNSUPPORTED),
    (dict(block_size=64), UNSUPPORTED),
    (dict(dtype=I8), UNSUPPORTED),
])
def test_write_rejects(lib, over, code):
    st, msg = _write(lib, **over)
    assert st == code and msg


def test_write_zero_tokens_is_noop(lib):
    st, msg = _write(lib, num_tokens=0, k=None, v=None, k_cache=None, v_cache=None, slots=None)
    assert st == OK and msg == ""


def test_write_int8_rejects(lib):
    f = lib.pkv_kv_cache_write_int8
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), None, _fake(6), _fake(7), 4, 8, 128, 16, 8, None)
    assert st == INVALID and b"scale" in lib.pkv_last_error()
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), 4, 8, 48, 16, 8, None)
    assert st == UNSUPPORTED
    st = f(None, None, None, None, None, None, None, 0, 8, 128, 16, 8, None)
    assert st == OK


def test_write_fp8_e5m2_rejects(lib):
    f = lib.pkv_kv_cache_write_fp8_e5m2
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), None, _fake(7), 4, 8, 128, 16, 8, None)
    assert st == INVALID and b"scale" in lib.pkv_last_error()
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), 4, 8, 128, 64, 8, None)
    assert st == UNSUPPORTED
    st = f(None, None, None, None, None, None, None, 0, 8, 128, 16, 8, None)
    assert st == OK


def test_write_int4_rejects(lib):
    f = lib.pkv_kv_cache_write_int4
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), None, _fake(6), _fake(7), 4, 8, 128, 16, 8, None)
    assert st == INVALID and b"scale" in lib.pkv_last_error()
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), 4, 8, 96, 16, 8, None)
    assert st == UNSUPPORTED
    st = f(_fake(1), _fake(2), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), 4, 8, 128, 8, 8, None)
    assert st == UNSUPPORTED
    st = f(None, None, None, None, None, None, None, 0, 8, 128, 16, 8, None)
    assert st == OK


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "missing.so"))


def test_probe_rejects_bad_arguments(lib):
    f = lib.pkv_probe_tile_read
    pool, ids, sink = ctypes.c_void_p(0x10000), _fake(2), _fake(3)
    assert f(None, ids, 1, 1, 0, sink, None) == INVALID
    assert f(pool, None, 1, 1, 0, sink, None) == INVALID
    assert f(pool, ids, 1, 1, 0, None, None) == INVALID
    assert f(ctypes.c_void_p(0x10010), ids, 1, 1, 0, sink, None) == INVALID  # misaligned pool
    assert b"aligned" in lib.pkv_last_error()
    assert f(pool, ids, -1, 1, 0, sink, None) == INVALID
    assert f(pool, ids, 1, 0, 0, sink, None) == INVALID
    assert f(pool, ids, 1, 65537, 0, sink, None) == INVALID
    assert f(pool, ids, 1, 1, 2, sink, None) == INVALID
    assert b"streaming" in lib.pkv_last_error()
    assert f(pool, ids, 0, 1, 0, sink, None) == OK  # nothing to read: no launch
    assert f(pool, ids, 0, 1, 1, sink, None) == OK


MIB = 1 << 20


@pytest.mark.parametrize("kv,per_token", [(F32, 8 * 128), (BF16, 4 * 128), (I8, 2 * 128 + 8),
                                          (FP8, 2 * 128 + 8), (E5M2, 2 * 128 + 8), (I4, 128 + 8)])
def test_streams_cache_threshold(lib, kv, per_token):
    """The non-temporal hint is taken exactly when the pool (K + V codes and
    scales of every token slot of every block) exceeds 512 MiB."""
    f = lib.pkv_paged_attention_streams_cache
    Hkv, bs, D = 8, 16, 128
    per_block = Hkv * bs * per_token
    at = (512 * MIB) // per_block  # largest pool not above the threshold
    assert f(at, Hkv, bs, D, kv) == 0
    assert f(at + 1, Hkv, bs, D, kv) == 1
    # the same byte count laid out with other sizes gives the same answer
    assert f(2 * at, Hkv // 2, bs, D, kv) == 0 and f(2 * at + 2, Hkv // 2, bs, D, kv) == 1
    assert f(at + 1, Hkv, bs, D, kv) == f((at + 1) // 2 + 1, Hkv, 2 * bs, D, kv)


@pytest.mark.parametrize("args", [(-1, 8, 16, 128, BF16), (1 << 30, 0, 16, 128, BF16),
                                  (1 << 30, 8, 8, 128, BF16), (1 << 30, 8, 16, 96, BF16),
                                  (1 << 30, 8, 16, 128, 99)])
def test_streams_cache_invalid_sizes(lib, args):
    assert lib.pkv_paged_attention_streams_cache(*args) == 0


@pytest.mark.parametrize("name,num_blocks,Hkv,kv,expect", [
    ("tiny_f32", 32, 4, F32, 0), ("mha7b_bf16", 4608, 32, BF16, 1), ("gqa70b_bf16", 34658, 8, BF16, 1),
    ("prefix_bf16_bs16", 5407, 8, BF16, 0), ("int8_gqa70b", 36864, 8, I8, 1), ("int4_gqa70b", 36864, 8, I4, 1)])
def test_streams_cache_workloads(lib, name, num_blocks, Hkv, kv, expect):
    """The benchmark workloads' pools (block size 16; head_dim 64 for the
    tiny fp32 one, 128 otherwise): the 7B and 70B-shaped ones (over 1 GiB)
    stream; the 256-sequence shared-prefix pool (about 340 MiB) and the tiny
    one do not."""
    D = 64 if kv == F32 else 128
    assert lib.pkv_paged_attention_streams_cache(num_blocks, Hkv, 16, D, kv) == expect


def _cascade(lib, **over):
    a = dict(out=_fake(1), q=_fake(2), k_cache=_fake(3), v_cache=_fake(4), k_scale=None,
             v_scale=None, block_tables=_fake(5), context_lens=_fake(6), group_start=_fake(7),
             group_shared_blocks=_fake(8), scale=0.125, num_seqs=4, num_heads=8, num_kv_heads=2,
             head_dim=64, block_size=16, max_blocks_per_seq=13, num_blocks=32, num_groups=2,
             max_group_size=3, max_shared_blocks=5, q_dtype=BF16, kv_dtype=BF16,
             partition_tokens=0, prefix_partition_tokens=0, workspace=None, workspace_bytes=0,
             stream=None)
    a.update(over)
    st = lib.pkv_paged_attention_decode_cascade(*a.values())
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("over,code,frag", [
    (dict(q_dtype=F32, kv_dtype=F32), UNSUPPORTED, "bf16, int8, FP8 and INT4"),
    (dict(num_groups=0), INVALID, "num_groups"),
    (dict(num_groups=5), INVALID, "num_groups"),
    (dict(max_group_size=0), INVALID, "max_group_size"),
    (dict(max_group_size=5), INVALID, "max_group_size"),
    (dict(max_shared_blocks=-1), INVALID, "max_shared_blocks"),
    (dict(max_shared_blocks=14), INVALID, "max_shared_blocks"),
    (dict(group_start=None), INVALID, "group_start"),
    (dict(group_shared_blocks=None), INVALID, "group_start"),
    (dict(prefix_partition_tokens=48), INVALID, "prefix_partition_tokens"),
    (dict(prefix_partition_tokens=4096), INVALID, "prefix_partition_tokens"),
    (dict(partition_tokens=40), INVALID, "partition_tokens"),
    (dict(out=None), INVALID, "null pointer"),
    (dict(head_dim=96), UNSUPPORTED, "head_dim"),
    (dict(kv_dtype=I8), INVALID, "k_scale"),
])
def test_cascade_rejects(lib, over, code, frag):
    st, msg = _cascade(lib, **over)
    assert st == code, msg
    assert frag in msg


def test_cascade_workspace(lib):
    need = lib.pkv_paged_attention_cascade_workspace_size(4, 8, 2, 64, 16, 13, 2, 3, 5, 0, 0)
    assert need > 0
    st, msg = _cascade(lib)
    assert st == WORKSPACE and "required" in msg
    st, msg = _cascade(lib, workspace=ctypes.c_void_p(0x100000), workspace_bytes=need - 1)
    assert st == WORKSPACE
    st, msg = _cascade(lib, workspace=ctypes.c_void_p(0x100010), workspace_bytes=need)
    assert st == WORKSPACE and "aligned" in msg
    # no shared blocks: still one partial slot per partition, the reduce always runs
    assert lib.pkv_paged_attention_cascade_workspace_size(4, 8, 2, 64, 16, 13, 4, 1, 0, 0, 0) > 0
    assert lib.pkv_paged_attention_cascade_workspace_size(0, 8, 2, 64, 16, 13, 0, 0, 0, 0, 0) == 0
    assert lib.pkv_paged_attention_cascade_workspace_size(4, 8, 2, 96, 16, 13, 2, 3, 5, 0, 0) == 0
    # slot count = prefix partitions + partitions of the rest
    rows = 4 * 8 * (-(-5 * 16 // 32) + -(-13 * 16 // 64))
    want = -(-rows * 64 * 4 // 256) * 256 + 2 * (-(-rows * 4 // 256) * 256)
    assert lib.pkv_paged_attention_cascade_workspace_size(4, 8, 2, 64, 16, 13, 2, 3, 5, 64, 32) == want


def test_cascade_empty_batch_is_noop(lib):
    st, msg = _cascade(lib, num_seqs=0, num_groups=0, max_group_size=0, max_shared_blocks=0)
    assert st == OK, msg


def _copy(lib, **over):
    a = dict(dst_k=_fake(1), dst_v=_fake(2), dst_ks=None, dst_vs=None, src_k=_fake(3), src_v=_fake(4),
             src_ks=None, src_vs=None, pairs=_fake(5), n=3, num_kv_heads=2, head_dim=64, block_size=16,
             dtype=BF16, stream=None)
    a.update(over)
    st = lib.pkv_copy_blocks(*a.values())
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("over,code,frag", [
    (dict(n=-1), INVALID, "n must be"),
    (dict(dtype=7), UNSUPPORTED, "dtype"),
    (dict(head_dim=96), UNSUPPORTED, "head_dim"),
    (dict(block_size=8), UNSUPPORTED, "block_size"),
    (dict(pairs=None), INVALID, "null pointer"),
    (dict(src_v=None), INVALID, "null pointer"),
    (dict(dtype=I8), INVALID, "scale"),
    (dict(dtype=I4), INVALID, "scale"),
    (dict(dst_ks=_fake(6)), INVALID, "NULL"),
    (dict(n=70000), UNSUPPORTED, "65535"),
])
def test_copy_blocks_rejects(lib, over, code, frag):
    st, msg = _copy(lib, **over)
    assert st == code, msg
    assert frag in msg


def test_copy_blocks_zero_pairs_is_noop(lib):
    st, msg = _copy(lib, n=0, pairs=None)
    assert st == OK, msg


def _mq(lib, **over):
    a = dict(out=_fake(1), q=_fake(2), k_cache=_fake(3), v_cache=_fake(4), k_scale=None, v_scale=None,
             block_tables=_fake(5), context_lens=_fake(6), query_start=_fake(7), scale=0.125,
             num_seqs=4, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, max_blocks_per_seq=13,
             num_blocks=32, num_query_tokens=20, max_queries_per_seq=5, q_dtype=BF16, kv_dtype=BF16,
             partition_tokens=0, workspace=None, workspace_bytes=0, stream=None)
    a.update(over)
    st = lib.pkv_paged_attention_multi_query(*a.values())
    return st, lib.pkv_last_error().decode()


@pytest.mark.parametrize("over,code,frag", [
    (dict(q_dtype=F32, kv_dtype=F32), UNSUPPORTED, "bf16, int8, FP8 and INT4"),
    (dict(num_query_tokens=-1), INVALID, "num_query_tokens"),
    (dict(max_queries_per_seq=0), INVALID, "max_queries_per_seq"),
    (dict(max_queries_per_seq=21), INVALID, "max_queries_per_seq"),
    (dict(query_start=None), INVALID, "query_start"),
    (dict(partition_tokens=40), INVALID, "partition_tokens"),
    (dict(kv_dtype=I8), INVALID, "k_scale"),
    (dict(out=None), INVALID, "null pointer"),
])
def test_multi_query_rejects(lib, over, code, frag):
    st, msg = _mq(lib, **over)
    assert st == code, msg
    assert frag in msg


def test_multi_query_workspace(lib):
    st, msg = _mq(lib)
    assert st == WORKSPACE
    need = lib.pkv_paged_attention_multi_query_workspace_size(4, 20, 5, 8, 2, 64, 16, 13, 64)
    rows = 20 * 8 * -(-13 * 16 // 64)
    assert need == -(-rows * 64 * 4 // 256) * 256 + 2 * (-(-rows * 4 // 256) * 256)
    assert lib.pkv_paged_attention_multi_query_workspace_size(4, 0, 0, 8, 2, 64, 16, 13, 0) == 0
    st, msg = _mq(lib, num_query_tokens=0, max_queries_per_seq=0)
    assert st == OK, msg
