"""Closed forms for KV-cache sizes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``kv_cache_bytes``: ``2 x batch x seq_len x layers x heads x head_dim x
  dtype_bytes`` ([LAYERS] 2.1; its 7B example, 32 layers, 32 heads, head_dim
  128, fp16 at 2048 tokens, is about 1.07 GB, and 34 GB at batch 32).  For
  grouped-query attention ``heads`` is the number of KV heads.
* ``decode_kv_bytes``: the K and V bytes one decode step must read, counted
  token by token from the context lengths (every decode step reads the whole
  cache: [ENG5] "Two phases with very different characteristics"), plus the
  per-token scales of an int8 cache.
"""


def kv_cache_bytes(batch, seq_len, num_layers, num_heads, head_dim, dtype_bytes):
    """KV-cache bytes of ``batch`` sequences of ``seq_len`` tokens."""
    return 2 * int(batch) * int(seq_len) * int(num_layers) * int(num_heads) \
        * int(head_dim) * int(dtype_bytes)


def decode_kv_bytes(context_lens, num_kv_heads, head_dim, kv_elem_bytes,
                    scale_bytes=0):
    """Bytes of K and V (and their per-token scales) one decode step reads."""
    per_token = int(num_kv_heads) * (int(head_dim) * int(kv_elem_bytes) + int(scale_bytes))
    return 2 * per_token * sum(int(L) for L in context_lens)
