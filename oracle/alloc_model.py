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
* Peak (PageFault, "Project layout": the host free list records its peak;
  PageForge, "Does the pool actually come back to zero?": the paged peak of a
  batch against the naive reservation): the largest number of pages in use
  at any moment since the pool was made or the peak was last reset.

Copy-on-write sharing (PagedAttention blog, "Copy-on-Write for Parallel
Sampling"): several tables may hold the same physical page; a reference count
per page says how many.  ``fork`` gives a new sequence the parent's table,
raising every count by one.  ``free`` lowers the counts and returns a page to
the stack only when its count reaches zero.  A write into a shared page first
copies it: ``grow`` takes a fresh page, reports the (source, destination) copy,
and puts the destination into the writing sequence's table only.  Readings
where the blog is silent:

* Tokens are only ever appended, so the only page a growth writes into is the
  sequence's last page, and only if that page is partly filled; full shared
  pages stay shared for good.  A grow therefore makes at most one copy.
* The copy page is taken from the stack before the new pages of the same
  grow, and it counts towards the all-or-nothing page need.
* Plain ``alloc`` does no copying: if its growth would write into a shared
  page it refuses (SHARED) and changes nothing, so a caller that does not
  know about sharing can never overwrite another sequence's tokens.
* The last holder of a page frees it; pages are pushed in the order the
  freeing sequence's table lists them, last first, skipping pages still held.

Swapping (PagedAttention blog, "Preemption and Swapping": a sequence's blocks
are evicted to CPU memory and copied back when it resumes, block by block).
Readings where the blog is silent:

* The backing store is a set of page-sized host slots with its own LIFO
  stack (slot 0 first), like the device pool.
* A whole sequence is swapped: every page of its table goes to a slot, in
  table order, and the sequence drops its hold on the device pages (a page
  another table still holds stays where it is; the swapped copy is private).
  Its device pages go back to the stack as a free would push them.
* Swapping in takes pages from the device stack in table order, copies the
  slots back and returns the slots to their stack last first, as a free does.
* Both are all or nothing over a batch of sequences (not enough slots, or
  not enough device pages); a swapped sequence cannot grow, fork or be
  exported (SWAPPED) until it is swapped in; freeing it releases its slots.
"""

OK = "ok"
OOM = "oom"
UNKNOWN_SEQ = "unknown_seq"
INVALID = "invalid"
SHARED = "shared"
SWAPPED = "swapped"


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
        self.refs = [0] * num_pages
        self.peak = 0                 # most pages in use at once (see reset_peak)
        self.slot_stack = []          # host swap slots, top at the end
        self.num_slots = 0
        self.swapped = {}             # seq id -> host slots, in table order

    # -- operations -----------------------------------------------------------
    def _writes_shared(self, seq_id, new_len):
        """True if growing to new_len writes into a partly filled last page
        that another table also holds."""
        table = self.tables.get(seq_id, [])
        current = self.lengths.get(seq_id, 0)
        return (new_len > current and current % self.block_size != 0
                and self.refs[table[-1]] > 1)

    def alloc(self, seq_id, new_len):
        """Grow ``seq_id`` to ``new_len`` tokens.  Returns (status, n_new_pages)."""
        if new_len < 0:
            return INVALID, 0
        if seq_id in self.swapped:
            return SWAPPED, 0
        table = self.tables.get(seq_id, [])
        current = self.lengths.get(seq_id, 0)
        if new_len < current:
            return INVALID, 0
        if self._writes_shared(seq_id, new_len):
            return SHARED, 0
        need = blocks_for(new_len, self.block_size) - len(table)
        if need > len(self.stack):
            return OOM, 0
        new_pages = [self.stack.pop() for _ in range(need)]
        for p in new_pages:
            self.refs[p] = 1
        self.tables[seq_id] = table + new_pages
        self.lengths[seq_id] = new_len
        self._note_peak()
        return OK, need

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent``'s table and length, sharing
        every page.  Returns a status."""
        if parent in self.swapped:
            return SWAPPED
        if parent not in self.tables:
            return UNKNOWN_SEQ
        if child in self.tables or child in self.swapped:
            return INVALID
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for p in self.tables[child]:
            self.refs[p] += 1
        return OK

    def grow(self, seq_id, new_len):
        """Copy-on-write growth.  Returns (status, n_new_pages, copy) where
        copy is (source page, destination page) or None; n_new_pages counts
        every page taken from the stack, the copy's destination included."""
        if new_len < 0:
            return INVALID, 0, None
        if seq_id in self.swapped:
            return SWAPPED, 0, None
        table = self.tables.get(seq_id, [])
        current = self.lengths.get(seq_id, 0)
        if new_len < current:
            return INVALID, 0, None
        cow = self._writes_shared(seq_id, new_len)
        need = blocks_for(new_len, self.block_size) - len(table) + (1 if cow else 0)
        if need > len(self.stack):
            return OOM, 0, None
        table = list(table)
        copy = None
        if cow:
            src = table[-1]
            dst = self.stack.pop()
            self.refs[src] -= 1
            self.refs[dst] = 1
            table[-1] = dst
            copy = (src, dst)
        while len(table) < blocks_for(new_len, self.block_size):
            p = self.stack.pop()
            self.refs[p] = 1
            table.append(p)
        self.tables[seq_id] = table
        self.lengths[seq_id] = new_len
        self._note_peak()
        return OK, need, copy

    def grow_many(self, entries):
        """Batch copy-on-write growth, all or nothing: ``entries`` is a list of
        (seq_id, new_len) applied in order.  Returns (status, [n_new_pages],
        [copies in entry order]).  A length below what the earlier entries
        leave is INVALID (checked over the whole batch first); otherwise the
        batch is OOM if the pages run out anywhere.  On failure nothing
        changes."""
        lens = dict(self.lengths)
        for seq_id, new_len in entries:
            if new_len < 0 or new_len < lens.get(seq_id, 0):
                return INVALID, [0] * len(entries), []
            lens[seq_id] = new_len
        if any(seq_id in self.swapped for seq_id, _ in entries):
            return SWAPPED, [0] * len(entries), []
        saved = (self.stack[:], {k: v[:] for k, v in self.tables.items()}, dict(self.lengths), self.refs[:],
                 self.peak)
        counts, copies = [], []
        for seq_id, new_len in entries:
            st, nn, copy = self.grow(seq_id, new_len)
            if st != OK:
                self.stack, self.tables, self.lengths, self.refs, self.peak = saved
                return st, [0] * len(entries), []
            counts.append(nn)
            if copy is not None:
                copies.append(copy)
        return OK, counts, copies

    def free(self, seq_id):
        """Drop ``seq_id``'s hold on its pages, returning those no other table
        holds to the pool, and forget the sequence."""
        if seq_id in self.swapped:
            for slot in reversed(self.swapped.pop(seq_id)):
                self.slot_stack.append(slot)
            del self.lengths[seq_id]
            return OK
        if seq_id not in self.tables:
            return UNKNOWN_SEQ
        self._release(self.tables[seq_id])
        del self.tables[seq_id]
        del self.lengths[seq_id]
        return OK

    def _release(self, table):
        for page in reversed(table):
            self.refs[page] -= 1
            if self.refs[page] == 0:
                self.stack.append(page)

    # -- swapping --------------------------------------------------------------
    def set_swap_space(self, num_slots):
        """A fresh backing store of ``num_slots`` host slots (slot 0 first)."""
        self.num_slots = num_slots
        self.slot_stack = list(reversed(range(num_slots)))

    def swap_out(self, seq_ids):
        """Evict whole sequences.  Returns (status, [(page, slot), ...]) with
        the copies to make, device to host, in order."""
        if len(set(seq_ids)) != len(seq_ids):
            return INVALID, []
        for s in seq_ids:
            if s in self.swapped:
                return SWAPPED, []
            if s not in self.tables:
                return UNKNOWN_SEQ, []
        if sum(len(self.tables[s]) for s in seq_ids) > len(self.slot_stack):
            return OOM, []
        copies = []
        for s in seq_ids:
            slots = []
            for page in self.tables[s]:
                slot = self.slot_stack.pop()
                slots.append(slot)
                copies.append((page, slot))
            self._release(self.tables[s])
            del self.tables[s]
            self.swapped[s] = slots
        return OK, copies

    def swap_in(self, seq_ids):
        """Bring whole sequences back.  Returns (status, [(slot, page), ...])
        with the copies to make, host to device, in order."""
        if len(set(seq_ids)) != len(seq_ids):
            return INVALID, []
        for s in seq_ids:
            if s not in self.swapped:
                return (INVALID if s in self.tables else UNKNOWN_SEQ), []
        if sum(len(self.swapped[s]) for s in seq_ids) > len(self.stack):
            return OOM, []
        copies = []
        for s in seq_ids:
            slots = self.swapped.pop(s)
            table = []
            for slot in slots:
                page = self.stack.pop()
                self.refs[page] = 1
                table.append(page)
                copies.append((slot, page))
            for slot in reversed(slots):
                self.slot_stack.append(slot)
            self.tables[s] = table
        self._note_peak()
        return OK, copies

    # -- queries --------------------------------------------------------------
    def free_pages(self):
        return len(self.stack)

    def table(self, seq_id):
        return list(self.tables[seq_id])

    def seq_len(self, seq_id):
        return self.lengths[seq_id]

    def refcount(self, page):
        return self.refs[page]

    def _note_peak(self):
        self.peak = max(self.peak, self.pages_in_use())

    def reset_peak(self):
        """Restart the peak from the pages in use now."""
        self.peak = self.pages_in_use()

    def pages_in_use(self):
        return self.num_pages - len(self.stack)

    def block_tables(self, seq_ids, max_blocks):
        """Dense table rows and the lengths, as lists, one row per requested id
        in the order requested (PagedAttention blog, "Architecture": a fixed
        array of max_blocks_per_seq int32 entries per sequence whose first
        num_blocks entries map logical blocks to physical ones).  The blog
        zero-fills the unused entries and tracks num_blocks beside them; here
        they hold -1, which names no page (0 is a page id), so a table row
        carries its own block count.  A sequence with more blocks than
        max_blocks raises ValueError."""
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
        holders = [0] * self.num_pages
        for s, t in self.tables.items():
            n = self.lengths[s]
            assert len(t) == blocks_for(n, self.block_size), "ceil(len/B) blocks per sequence"
            assert self.block_size * len(t) - n <= self.block_size - 1, "waste at most B-1 slots"
            assert len(t) == len(set(t)), "a page twice in one table"
            for p in t:
                holders[p] += 1
        assert holders == self.refs, "reference counts differ from the tables holding each page"
        live = {p for p in range(self.num_pages) if holders[p] > 0}
        assert not live & set(self.stack), "a live page is also on the free list"
        assert len(self.stack) + len(live) == self.num_pages, "pages leaked or duplicated"
        assert len(set(self.stack)) == len(self.stack), "page pushed twice"
        held = [slot for slots in self.swapped.values() for slot in slots]
        assert len(held) == len(set(held)), "a host slot held twice"
        assert not set(held) & set(self.slot_stack), "a held slot is also free"
        assert len(held) + len(self.slot_stack) == self.num_slots, "host slots leaked"
        for s, slots in self.swapped.items():
            assert s not in self.tables and len(slots) == blocks_for(self.lengths[s], self.block_size)

