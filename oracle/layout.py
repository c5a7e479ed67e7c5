"""Oracle O2/O3: the pool image, scatter of new tokens, and read-back (test infrastructure only).

What it follows:

* PageForge, "Four layers, one pointer moving through all of them": one pool
  tensor for every layer, K and V combined, whole pages of 16 tokens.
* PageFault, "The OS analogy": logical token t of a sequence lives in physical
  frame ``table[t // B]`` at slot ``t % B``; the kernels resolve every K/V
  load through that walk.
* PageForge, "Five techniques" (gather / scatter): new tokens' K/V are written
  into their physical page slots; a gather assembles a sequence's scattered
  pages into one contiguous view.

Reading where the pages disagree (their three pool layouts differ): a page is
one contiguous region holding, for each layer, for each kv head, the K block
then the V block, each ``B x D`` with the token slot outer and the dimension
inner.  So the element address of (page p, layer l, kv head h, kind c with
K=0 / V=1, slot o, dim d) is

    ((((p * L + l) * H + h) * 2 + c) * B + o) * D + d

Everything here works on raw stored bit patterns (unsigned integer arrays);
copies are exact by construction, so comparisons against the GPU are bitwise.
"""
import numpy as np

K_KIND = 0
V_KIND = 1


class Geometry:
    """Pool geometry: pages, block size, layers, kv heads, head dim, element bytes."""

    def __init__(self, num_pages, block_size, num_layers, num_kv_heads, head_dim, elem_bytes):
        self.P = int(num_pages)
        self.B = int(block_size)
        self.L = int(num_layers)
        self.H = int(num_kv_heads)
        self.D = int(head_dim)
        self.es = int(elem_bytes)

    def page_elems(self):
        return self.L * self.H * 2 * self.B * self.D

    def page_bytes(self):
        return self.page_elems() * self.es

    def pool_elems(self):
        return self.P * self.page_elems()

    def bits_dtype(self):
        return {4: np.uint32, 2: np.uint16}[self.es]


def elem_offset(g, page, layer, head, kind, slot, dim):
    """Element index of one stored value inside the flat pool."""
    return ((((page * g.L + layer) * g.H + head) * 2 + kind) * g.B + slot) * g.D + dim


def token_location(table, pos, block_size):
    """Page-table walk: (physical page, slot) of logical token ``pos``."""
    return table[pos // block_size], pos % block_size


def empty_pool(g, sentinel_bits):
    """A pool image filled with the sentinel bit pattern (a NaN for float types)."""
    return np.full(g.pool_elems(), sentinel_bits, dtype=g.bits_dtype())


def scatter(pool, g, layer, k_bits, v_bits, tok_seq, tok_pos, tables):
    """Write token t's K/V (``k_bits[t]``, ``v_bits[t]``, each ``[H][D]``) into its slot.

    ``tok_seq[t]`` is the row of ``tables`` (one block table per sequence) and
    ``tok_pos[t]`` the token's logical position.  Returns a new pool image.
    """
    out = pool.copy()
    for t in range(len(tok_seq)):
        page, slot = token_location(tables[tok_seq[t]], int(tok_pos[t]), g.B)
        for h in range(g.H):
            for kind, src in ((K_KIND, k_bits), (V_KIND, v_bits)):
                base = elem_offset(g, page, layer, h, kind, slot, 0)
                out[base:base + g.D] = src[t, h, :]
    return out


def copy_pages(pool, g, pairs):
    """Copy-on-write page copies (PagedAttention blog, "Copy-on-Write for
    Parallel Sampling": the new block gets the shared block's contents).  For
    each (source, destination) pair in order, every element of the source page
    -- all layers, heads, K and V, every slot -- is copied to the destination
    page.  Returns a new pool image."""
    out = pool.copy()
    for src, dst in pairs:
        for layer in range(g.L):
            for h in range(g.H):
                for kind in (K_KIND, V_KIND):
                    for slot in range(g.B):
                        a = elem_offset(g, src, layer, h, kind, slot, 0)
                        b = elem_offset(g, dst, layer, h, kind, slot, 0)
                        out[b:b + g.D] = out[a:a + g.D]
    return out


def swap_copy(pool, host, g, pairs, to_host):
    """Swap copies (PagedAttention blog, "Preemption and Swapping": blocks go
    to CPU memory and come back).  ``host`` is the backing store image, one
    page-sized slot after another, each slot laid out like a page.  With
    ``to_host`` each (page, slot) pair copies the whole page into the slot;
    otherwise each (slot, page) pair copies the slot into the page.  Returns
    new (pool, host) images."""
    pool, host = pool.copy(), host.copy()
    n = g.page_elems()
    for a, b in pairs:
        if to_host:
            host[b * n:(b + 1) * n] = pool[a * n:(a + 1) * n]
        else:
            pool[b * n:(b + 1) * n] = host[a * n:(a + 1) * n]
    return pool, host


def readback(pool, g, layer, table, length):
    """Gather one sequence's K and V into contiguous ``[length][H][D]`` bit arrays."""
    kc = np.empty((length, g.H, g.D), dtype=pool.dtype)
    vc = np.empty((length, g.H, g.D), dtype=pool.dtype)
    for pos in range(length):
        page, slot = token_location(table, pos, g.B)
        for h in range(g.H):
            kb = elem_offset(g, page, layer, h, K_KIND, slot, 0)
            vb = elem_offset(g, page, layer, h, V_KIND, slot, 0)
            kc[pos, h] = pool[kb:kb + g.D]
            vc[pos, h] = pool[vb:vb + g.D]
    return kc, vc
