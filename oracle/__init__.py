"""Float64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct statement of what
the GPU library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The GPU library
(``paged_kv_cache_408_amd``) never imports, links or calls anything here, and nothing here
imports the GPU library: the two share no kernels, headers, helpers, tables or constants.

Sources (web pages; cited by title and section):

* "KV Cache Optimization and PagedAttention" (cracklab.in) -- cache-size formula, the
  contiguous-vs-paged waste worked example, the page-table analogy, prefix sharing.
* "PagedAttention: Optimizing KV Cache Utilization in Large Language Models"
  (fromzero2ai.dev) -- "The Mechanics of PagedAttention" (logical/physical blocks, page
  table, on-demand allocation), "The Math: Block Attention Calculation" (softmax of scaled
  q.K^T through the page table), "Serving Advantages" (shared prefix blocks),
  "Conclusion" (mid-generation block exhaustion, block-size trade-off).
* "KV Cache Management" (ai360xpert.com) -- "The Solution: PagedAttention (vLLM)"
  (one block at a time, non-adjacent blocks, block table), "The Bonus: Zero-Copy Sharing",
  "Watch Out For" / "What to Read Next" (8-bit KV cache).

Modules:

* ``codecs``     -- bit-level bf16 and OCP E4M3FN (fp8) codecs, written from the formats.
* ``allocator``  -- the block allocator model (FIFO free list, refcounts, fork, COW).
* ``attention``  -- slot-mapped scatter, block-table gather, exact softmax(q.K^T*scale).V,
                    the split-K / log-sum-exp variant and a pure-Python brute force.
* ``measures``   -- cache footprint, slots held and filled (reserved or paged), algorithmic bytes.

Every function is pinned by ``tests/test_oracle_*.py`` to something other than itself
(the pages' worked examples, closed forms, invariants, library routines, brute force).
"""

from . import codecs, allocator, attention, measures  # noqa: F401
