"""Oracle O1: the page allocator as a plain Python model (test infrastructure only).

What it follows:

* PageForge, "Four layers, one pointer moving through all of them": a free
  list of page ids plus a per-sequence block table (sequence id -> list of page
  ids), joined behind one object whose ``alloc_for_seq`` / ``free_seq`` are O(1)
  per page.
* mini-infer ("Why Naive KV-Caches Waste >60% VRAM"), "Implementation
  Walkthrough": the free list is a stack built from the page ids in reverse, so
  a fresh pool hands out page 0 first; an empty pool is an error.
* PagedAttention blog, "Architecture": a new physical block is taken only when
  the sequence's last block is full; the table only ever grows, nothing is
  copied.
* PageFault, "Test" (free-list row): exhaustion and double free are errors and
  allocation is all-or-nothing.
* PageForge, "Does the pool actually come back to zero?": every page returns on
  free, and the next batch reuses exactly the pages the previous one returned.

Readings where the pages are silent:

* Order of the free list: LIFO (mini-infer's and the blog's stacks; it is also
  what makes batch 2 reuse batch 1's pages).  Pages of a freed sequence are
  pushed last-page-first, so the first page of its table is on top again.
* A shuffled pool is a permutation given as the initial free order; the model
  holds no random number generator.
* ``alloc(seq, new_len)`` takes the sequence's new total length; a new id
  creates the entry; a shorter length is invalid; on OOM nothing changes.
"""

OK = "ok"
OOM = "oom"
UNKNOWN_SEQ = "unknown_seq"
INVALID = "invalid"


def blocks_for(length, block_size):
    """Number of fixed-size blocks a sequence of ``length`` tokens occupies."""
    return -(-length // block_size)


class AllocModel:
    """LIFO free stack of page ids plus per-sequence block tables."""

    def __init__(self, num_pages, block_size=16, initial_free_order=None):
        if num_pages <= 0 or block_size <= 0:
            raise ValueError("num_pages and block_size must be positive")
        order = list(range(num_pages)) if initial_free_order is None else [int(p) for p in initial_free_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("initial_free_order must be a permutation of 0..num_pages-1")
        self.num_pages = num_pages
        self.block_size = block_size
        # Stack top is the end of the list; reversing makes order[0] pop first.
        self.stack = list(reversed(order))
        self.tables = {}
        self.lengths = {}

    # -- operations -----------------------------------------------------------
    def alloc(self, seq_id, new_len):
        """Grow ``seq_id`` to ``new_len`` tokens.  Returns (status, n_new_pages)."""
        if new_len < 0:
            return INVALID, 0
        table = self.tables.get(seq_id, [])
        current = self.lengths.get(seq_id, 0)
        if new_len < current:
            return INVALID, 0
        need = blocks_for(new_len, self.block_size) - len(table)
        if need > len(self.stack):
            return OOM, 0
        new_pages = [self.stack.pop() for _ in range(need)]
        self.tables[seq_id] = table + new_pages
        self.lengths[seq_id] = new_len
        return OK, need

    def free(self, seq_id):
        """Return every page of ``seq_id`` to the pool and forget the sequence."""
        if seq_id not in self.tables:
            return UNKNOWN_SEQ
        for page in reversed(self.tables[seq_id]):
            self.stack.append(page)
        del self.tables[seq_id]
        del self.lengths[seq_id]
        return OK

    # -- queries --------------------------------------------------------------
    def free_pages(self):
        return len(self.stack)

    def table(self, seq_id):
        return list(self.tables[seq_id])

    def seq_len(self, seq_id):
        return self.lengths[seq_id]

    def block_tables(self, seq_ids, max_blocks):
        """Dense int32-style table rows (padded with -1) and the lengths, as lists."""
        rows, lens = [], []
        for s in seq_ids:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("sequence needs more than max_blocks blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return rows, lens

    # -- invariants (checked by the tests after every op) ----------------------
    def check_invariants(self):
        live = []
        for s, t in self.tables.items():
            n = self.lengths[s]
            assert len(t) == blocks_for(n, self.block_size), "ceil(len/B) blocks per sequence"
            assert self.block_size * len(t) - n <= self.block_size - 1, "waste at most B-1 slots"
            live.extend(t)
        assert len(live) == len(set(live)), "a page is owned by two sequences"
        assert not set(live) & set(self.stack), "a live page is also on the free list"
        assert len(self.stack) + len(live) == self.num_pages, "pages leaked or duplicated"
        assert len(set(self.stack)) == len(self.stack), "page pushed twice"


def replay(num_pages, block_size, initial_free_order, ops):
    """Replay an op log ``[("alloc", seq, new_len) | ("free", seq), ...]``.

    Returns the model and, per op, ``(status, n_new_pages, free_pages)`` so a
    log recorded from another implementation can be compared op by op.
    """
    m = AllocModel(num_pages, block_size, initial_free_order)
    trace = []
    for op in ops:
        if op[0] == "alloc":
            st, nn = m.alloc(op[1], op[2])
        elif op[0] == "free":
            st, nn = m.free(op[1]), 0
        else:
            raise ValueError(op)
        trace.append((st, nn, m.free_pages()))
    return m, trace
