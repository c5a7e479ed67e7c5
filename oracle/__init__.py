"""CPU fp64 oracle for decode-step paged attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The product path (the C-ABI library and its Python binding) never
routes through it and shares no code with it: the oracle receives raw arrays
(stored bit patterns, block tables, lengths, op logs) and recomputes everything
from the pages' definitions, in plain NumPy / pure Python, in float64.

Modules, and the passages each one follows:

* ``alloc_model``  -- the O(1) LIFO free list and per-sequence block tables
  (PageForge, "Four layers, one pointer moving through all of them" and
  "Five techniques": free-list allocator + block table; mini-infer,
  "Implementation Walkthrough": the free-list stack; PagedAttention blog,
  "Architecture": allocate a new block only when the last one is full), with
  copy-on-write sharing: reference counts, fork, and a grow that copies a
  shared block before writing into it (PagedAttention blog, "Copy-on-Write
  for Parallel Sampling"), and swapping whole sequences to a host backing
  store and back (PagedAttention blog, "Preemption and Swapping").
* ``layout``       -- the pool image: element address of a token's K/V inside
  a page, the scatter of new tokens, and the read-back (gather) of a
  sequence's pages into contiguous K/V (PageFault, "The OS analogy": the
  page-table walk; PageForge, "Four layers": K and V combined in one pool),
  the whole-page copies of copy-on-write and the page <-> host-slot copies of
  swapping.
* ``attention``    -- the plain definition softmax(q.K^T.scale).V on contiguous
  read-back K/V, two-pass, no splitting (PagedAttention blog, "The Attention
  Kernel"; PageFault, "Four stages", stage 1 and 3), plus a pure-Python brute
  force used only to pin it.
* ``accounting``   -- bytes per token, reserved memory, utilization and
  internal fragmentation (PageFault, "Calculate": core formulas).

Pins (``tests/pins.py``, run by ``tests/test_oracle_pins.py``; fixtures in
``tests/golden/``) tie every public function and method here to something other
than itself: worked examples printed on the pages, closed forms, brute force on
tiny inputs and invariants; ``tests/test_oracle_planted.py`` plants plausible
mistakes and checks that a pin catches each.  The dense table export
(``AllocModel.block_tables``) is pinned to the blog's table [7, 13, 2, 41]
exported wider than the table, in request order, with the -1 padding that is
this package's reading.  The rounding of the GPU's fp32 arithmetic is bounded
only by the 2e-3 tolerance (there is no bit-exact attention target).
"""
