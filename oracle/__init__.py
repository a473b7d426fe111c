"""CPU oracle for paged KV-cache attention (PagedAttention).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may use it.
It shares no code with the HIP library or its Python binding, and it imports
neither of them.

What it computes, and where each step comes from:

* ``paging``        -- slot arithmetic, the append (write) into pool slots, the
                       copy-on-write block copy and the gather of one
                       sequence's blocks through its block table.  All of it is
                       done on raw storage words, so results are bit patterns.
                       Sources: "Paged Attention for Efficient Memory
                       Management" (The Daily Triptych), technical summary and
                       "The story"; "PagedAttention and RadixAttention: Let's
                       Talk About KV Cache", section "PagedAttention: Memory
                       Like an Operating System".
* ``attention``     -- exact softmax attention in float64 over the gathered
                       keys and values: decode (one query token per sequence),
                       extend (new tokens attending causally to a cached prefix
                       plus themselves), per-partition partials and the
                       log-sum-exp merge that recombines them.  Sources: the
                       Triptych page, technical summary and "The surprising
                       detail" (paging leaves the attention scores unchanged);
                       "RadixAttention: Tree-Based KV Cache Reuse in SGLang
                       Guide", section "3. Integrating FlashInfer ..." (split-KV
                       decode along the sequence).
* ``block_manager`` -- a deliberately plain, token-at-a-time model of the
                       reference-counted block manager (allocate on overflow,
                       fork by reference, copy-on-write on the first write to a
                       shared block, free at refcount zero).  Sources: the
                       Triptych page, technical summary and "Sharing is a
                       pointer change"; "PagedAttention 与 RadixAttention"
                       (khotyn.com), section "PagedAttention".

* ``prefix_cache`` -- plain models of the two automatic prefix caches: one
                       keyed by (salt, whole token prefix) for the chained-hash
                       cache, and a radix tree kept as a flat node list searched
                       by scanning.  Sources: "PagedAttention and
                       RadixAttention: Let's Talk About KV Cache", sections
                       "RadixAttention: A Tree That Does Not Forget", "Two
                       Layers, Not Two Rivals" and "Beyond the Two Techniques";
                       "RadixAttention: Tree-Based KV Cache Reuse in SGLang
                       Guide", "Architecture"; "PagedAttention 与
                       RadixAttention", section "RadixAttention".

Numerics: float64 throughout.  bf16 inputs are widened exactly (bits << 16 as
float32, then float64); float32 inputs are widened exactly.

Parity pins: every function here is pinned by tests in ``tests/`` against
closed forms, brute force, library routines on contiguous data and the
invariants the pages state (see ``tests/test_oracle_pins.py``).  No function in
this package is "parity unpinned".
"""

from . import attention, block_manager, numerics, paging, prefix_cache  # noqa: F401
