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
are evicted to CPU memory and copied back when it resumes; swapping works on
blocks, so part of a sequence may be on the GPU and the rest on the CPU).
Readings where the blog is silent:

* The backing store is a set of page-sized host slots with its own LIFO
  stack (slot 0 first), like the device pool.
* A block range of one sequence can be swapped out (every block in it on
  the device) or in (every block in it on the host); a whole sequence, or
  every block of a batch of sequences that is on the host, likewise.
* Swapping out takes a slot per block in block order; the sequence drops
  its hold on those pages (a page another table still holds stays where it
  is; the swapped copy is private), which go back to the stack last block
  first, as a free would push them.
* Swapping in takes pages from the device stack in block order, copies the
  slots back and returns the slots to their stack last block first.
* Every swap is all or nothing (not enough slots, or not enough device
  pages); a sequence with any block on the host cannot grow, fork or be
  exported (SWAPPED) until all its blocks are back; freeing it releases its
  device pages and its slots.
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
        # sequences with blocks on the host: id -> (pages, host), pages[b] the
        # device page of block b or None, host[b] the slot of a block on the host
        self.offdev = {}

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
        if seq_id in self.offdev:
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
        if parent in self.offdev:
            return SWAPPED
        if parent not in self.tables:
            return UNKNOWN_SEQ
        if child in self.tables or child in self.offdev:
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
        if seq_id in self.offdev:
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
        if any(seq_id in self.offdev for seq_id, _ in entries):
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
        holds to the pool, return its host slots (last block first), and
        forget the sequence."""
        if seq_id in self.offdev:
            pages, host = self.offdev.pop(seq_id)
            self._release([p for p in pages if p is not None])
            for b in sorted(host, reverse=True):
                self.slot_stack.append(host[b])
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

    @property
    def swapped(self):
        """Sequences with blocks on the host: id -> the slots of those blocks,
        in block order."""
        return {s: [host[b] for b in sorted(host)] for s, (_, host) in self.offdev.items()}

    def _split(self, seq_id):
        """(pages, host) of a live sequence (pages: None for blocks on the host)."""
        if seq_id in self.offdev:
            return self.offdev[seq_id]
        return self.tables[seq_id], {}

    def _move_out(self, seq_id, blocks):
        """Blocks (all on the device) to host slots taken in block order; the
        pages are released last block first.  Returns the (page, slot) copies.
        (A sequence of length 0 swapped out whole moves nothing and is listed
        as swapped all the same.)"""
        pages, host = self._split(seq_id)
        pages, host = list(pages), dict(host)
        copies = []
        for b in blocks:
            slot = self.slot_stack.pop()
            copies.append((pages[b], slot))
            host[b] = slot
        self._release([pages[b] for b in blocks])
        for b in blocks:
            pages[b] = None
        self.tables.pop(seq_id, None)
        self.offdev[seq_id] = (pages, host)
        return copies

    def _move_in(self, seq_id, blocks):
        """Blocks (all on the host) to pages popped in block order; the slots
        return last block first.  Returns the (slot, page) copies."""
        pages, host = self.offdev[seq_id]
        pages, host = list(pages), dict(host)
        copies = []
        for b in blocks:
            page = self.stack.pop()
            self.refs[page] = 1
            copies.append((host[b], page))
            pages[b] = page
        for b in reversed(blocks):
            self.slot_stack.append(host.pop(b))
        if host:
            self.offdev[seq_id] = (pages, host)
        else:
            del self.offdev[seq_id]
            self.tables[seq_id] = pages
        self._note_peak()
        return copies

    def swap_out(self, seq_ids):
        """Evict whole sequences (every block on the device).  Returns
        (status, [(page, slot), ...]) with the copies to make, device to host,
        in order."""
        if len(set(seq_ids)) != len(seq_ids):
            return INVALID, []
        for s in seq_ids:
            if s in self.offdev:
                return SWAPPED, []
            if s not in self.tables:
                return UNKNOWN_SEQ, []
        if sum(len(self.tables[s]) for s in seq_ids) > len(self.slot_stack):
            return OOM, []
        copies = []
        for s in seq_ids:
            copies += self._move_out(s, list(range(len(self.tables[s]))))
        return OK, copies

    def swap_in(self, seq_ids):
        """Bring back every block of these sequences that is on the host.
        Returns (status, [(slot, page), ...]) with the copies to make, host to
        device, in order."""
        if len(set(seq_ids)) != len(seq_ids):
            return INVALID, []
        for s in seq_ids:
            if s not in self.offdev:
                return (INVALID if s in self.tables else UNKNOWN_SEQ), []
        if sum(len(self.offdev[s][1]) for s in seq_ids) > len(self.stack):
            return OOM, []
        copies = []
        for s in seq_ids:
            copies += self._move_in(s, sorted(self.offdev[s][1]))
        return OK, copies

    def _block_range(self, seq_id, first, count):
        """The blocks [first, first + count) of a live sequence, or None if the
        range is empty or leaves its table."""
        pages, _ = self._split(seq_id)
        if count < 1 or first < 0 or first + count > len(pages):
            return None
        return list(range(first, first + count))

    def swap_out_blocks(self, seq_id, first, count):
        """Evict blocks [first, first + count) of one sequence, every one of
        them on the device.  Returns (status, [(page, slot), ...])."""
        if seq_id not in self.tables and seq_id not in self.offdev:
            return UNKNOWN_SEQ, []
        blocks = self._block_range(seq_id, first, count)
        if blocks is None or any(self._split(seq_id)[0][b] is None for b in blocks):
            return INVALID, []
        if len(blocks) > len(self.slot_stack):
            return OOM, []
        return OK, self._move_out(seq_id, blocks)

    def swap_in_blocks(self, seq_id, first, count):
        """Bring back blocks [first, first + count) of one sequence, every one
        of them on the host.  Returns (status, [(slot, page), ...])."""
        if seq_id not in self.tables and seq_id not in self.offdev:
            return UNKNOWN_SEQ, []
        blocks = self._block_range(seq_id, first, count)
        if blocks is None or any(b not in self._split(seq_id)[1] for b in blocks):
            return INVALID, []
        if len(blocks) > len(self.stack):
            return OOM, []
        return OK, self._move_in(seq_id, blocks)

    # -- queries --------------------------------------------------------------
    def free_pages(self):
        return len(self.stack)

    def table(self, seq_id):
        """The sequence's block table: a page per block, None for a block on
        the host."""
        return list(self._split(seq_id)[0])

    def host_blocks(self, seq_id):
        """Block -> host slot for the sequence's blocks on the host."""
        return dict(self._split(seq_id)[1])

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
            if s in self.offdev:
                raise ValueError("a sequence with blocks on the host has no device table")
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("sequence needs more than max_blocks blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return rows, lens

    # -- invariants (checked by the tests after every op) ----------------------
    def check_invariants(self):
        holders = [0] * self.num_pages
        assert not set(self.tables) & set(self.offdev), "a sequence both resident and not"
        for s, t in list(self.tables.items()) + [(s, e[0]) for s, e in self.offdev.items()]:
            n = self.lengths[s]
            assert len(t) == blocks_for(n, self.block_size), "ceil(len/B) blocks per sequence"
            assert self.block_size * len(t) - n <= self.block_size - 1, "waste at most B-1 slots"
            dev = [p for p in t if p is not None]
            assert len(dev) == len(set(dev)), "a page twice in one table"
            for p in dev:
                holders[p] += 1
        for s, (pages, host) in self.offdev.items():
            assert host or not pages, "listed as off the device with every block on it"
            assert set(host) == {b for b, p in enumerate(pages) if p is None}, "a block in neither place"
        assert holders == self.refs, "reference counts differ from the tables holding each page"
        live = {p for p in range(self.num_pages) if holders[p] > 0}
        assert not live & set(self.stack), "a live page is also on the free list"
        assert len(self.stack) + len(live) == self.num_pages, "pages leaked or duplicated"
        assert len(set(self.stack)) == len(self.stack), "page pushed twice"
        held = [slot for _, host in self.offdev.values() for slot in host.values()]
        assert len(held) == len(set(held)), "a host slot held twice"
        assert not set(held) & set(self.slot_stack), "a held slot is also free"
        assert len(held) + len(self.slot_stack) == self.num_slots, "host slots leaked"

