"""Closed-form measures (oracle; test infrastructure only).

* ``kv_cache_bytes``: 2 (K and V) x layers x KV heads x head_dim x tokens x batch x bytes
  per value ("KV Cache Optimization and PagedAttention", prose on cache size and the
  worked example in its code listing).
* ``contiguous_waste``: slots reserved but unused when each request reserves its maximum
  length up front (same page, listing; "KV Cache Management", "The Memory Fragmentation
  Problem").
* ``paged_waste``: unused slots in the last, partly filled block when requests take
  fixed-size blocks on demand (same page, listing).
* ``decode_bytes`` / ``kv_write_bytes``: the bytes the method must move -- every request's
  cached K and V once per KV head, plus q, the output, the block-table entries it uses and
  the sequence lengths; for the write, the new rows read and written plus the slot ids.
"""

from __future__ import annotations

import math


def kv_cache_bytes(num_layers, num_kv_heads, head_dim, seq_len, batch, bytes_per_val=2):
    return 2 * num_layers * num_kv_heads * head_dim * seq_len * batch * bytes_per_val


def contiguous_waste(actual_len, max_len):
    return max_len - actual_len


def paged_waste(actual_len, block_size):
    return math.ceil(actual_len / block_size) * block_size - actual_len


def decode_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                 kv_bytes, q_bytes, out_bytes, fp8_scales=False):
    kv = sum(2 * num_kv_heads * L * head_dim * kv_bytes for L in seq_lens)
    qo = len(seq_lens) * num_q_heads * head_dim * (q_bytes + out_bytes)
    table = sum(4 * math.ceil(L / block_size) for L in seq_lens)
    lens = 4 * len(seq_lens)
    scales = 2 * num_kv_heads * 4 if fp8_scales else 0
    return kv + qo + table + lens + scales


def kv_write_bytes(num_tokens, num_kv_heads, head_dim, in_bytes, cache_bytes, fp8_scales=False):
    rows = num_tokens * num_kv_heads * head_dim
    return 2 * rows * (in_bytes + cache_bytes) + 8 * num_tokens + (2 * num_kv_heads * 4 if fp8_scales else 0)
