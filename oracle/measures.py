"""Closed-form measures of a KV cache (oracle; test infrastructure only).

* ``footprint_bytes``: what a cache holds -- a K vector and a V vector of head_dim values
  for every (layer, KV head, token, request) ("KV Cache Optimization and PagedAttention", prose
  on the cache's size and the first value its code listing prints).
* ``slot_budget``: the token slots one request holds and the slots it fills, under the two
  placements the pages compare.  A request that reserves its maximum length up front holds
  that many slots ("KV Cache Management", "The Memory Fragmentation Problem"; the listing's
  second print).  A request that takes fixed-size blocks as its tokens arrive holds its whole
  blocks (the listing's third print; "KV Cache Management", "The Solution: PagedAttention
  (vLLM)").  ``unused_slots`` is the difference.
* ``decode_bytes``: what one decode call must move -- every request's cached K and V once per
  KV head, plus q, the output, the block-table entries it uses and the sequence lengths.
"""

from __future__ import annotations


def footprint_bytes(layers, kv_heads, head_dim, tokens, requests, value_bytes=2):
    """Bytes of a KV cache: vectors_per_request K and V vectors of head_dim values each."""
    vectors_per_request = 2 * layers * kv_heads * tokens       # one K and one V per layer, head, token
    return requests * vectors_per_request * head_dim * value_bytes


def slot_budget(tokens, *, reserve=None, block_size=None):
    """(held, filled) token slots of one request of `tokens` tokens: either `reserve` slots
    reserved up front (reserve >= tokens), or whole blocks of `block_size` slots taken as the
    tokens arrive.  Exactly one of the two keywords is given."""
    if (reserve is None) == (block_size is None):
        raise ValueError("give exactly one of reserve, block_size")
    if reserve is not None:
        if tokens > reserve:
            raise ValueError("a reservation smaller than the request")
        return reserve, tokens
    blocks = -(-tokens // block_size)                          # blocks started, the last maybe partly filled
    return blocks * block_size, tokens


def unused_slots(tokens, **placement):
    """Slots held but not filled (see slot_budget)."""
    held, filled = slot_budget(tokens, **placement)
    return held - filled


def decode_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                 kv_bytes, q_bytes, out_bytes, fp8_scales=False):
    kv = sum(2 * num_kv_heads * L * head_dim * kv_bytes for L in seq_lens)
    qo = len(seq_lens) * num_q_heads * head_dim * (q_bytes + out_bytes)
    table = sum(4 * (-(-L // block_size)) for L in seq_lens)
    lens = 4 * len(seq_lens)
    scales = 2 * num_kv_heads * 4 if fp8_scales else 0
    return kv + qo + table + lens + scales
