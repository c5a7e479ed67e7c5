/*
 * pf.h -- C ABI of libpf: decode-step paged attention on MI355X (gfx950).
 *
 * Three parts, all behind plain pointers and sizes:
 *
 *  1. A host page allocator: an O(1) LIFO free list of fixed-size pages plus a
 *     block table per sequence (PageForge, "Four layers, one pointer moving
 *     through all of them" and "Five techniques": free-list allocation and
 *     page-table-style indirection; mini-infer, "Implementation Walkthrough":
 *     the free-list stack; PagedAttention blog, "Architecture": a new block is
 *     taken only when the last one is full).
 *  2. A device KV pool that the caller allocates (one allocation for every
 *     page, every layer, K and V combined: PageForge, "Four layers") and binds
 *     to the allocator handle.  Page p is one contiguous region; inside it the
 *     element (layer l, kv head h, kind c [K=0, V=1], slot o, dim d) sits at
 *         ((((p*L + l)*H + h)*2 + c)*B + o)*D + d
 *     so the K block and the V block of one (page, layer, head) are adjacent
 *     B x D tiles.
 *  3. HIP kernels: scatter of new tokens' K/V into their page slots (PageForge,
 *     "Five techniques": gather / scatter kernels), a read-back gather, and
 *     decode attention softmax(q.K^T.scale).V that walks each sequence's block
 *     table (PagedAttention blog, "The Attention Kernel"; PageFault, "The OS
 *     analogy": every K/V load goes through the table).
 *
 * Ownership: the library owns only the host handle.  Every device buffer (pool,
 * q, k, v, tables, lengths, out, workspace) belongs to the caller; streams are
 * passed as hipStream_t cast to void* (NULL = the default stream).  Kernel entry
 * points only enqueue work: device faults surface at the caller's next
 * synchronisation.  No function throws; every int result is a pf_status.
 *
 * Thread safety: allocator calls on one handle are serialised by an internal
 * mutex.  Kernel entry points read the handle's geometry, bound pointer and
 * options only; changing options or re-binding while kernels are being
 * enqueued from another thread is the caller's race.
 */
#ifndef PF_H
#define PF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the pool, q, k, v (and out unless out_dtype says PF_F32). */
typedef enum { PF_F32 = 0, PF_F16 = 1, PF_BF16 = 2 } pf_dtype;

typedef enum {
  PF_OK = 0,
  PF_ERR_INVALID = -1,      /* bad argument (range, null pointer, shape) */
  PF_ERR_OOM = -2,          /* not enough free pages; nothing was changed */
  PF_ERR_UNKNOWN_SEQ = -3,  /* sequence id not live (includes double free) */
  PF_ERR_UNBOUND = -4,      /* kernel call before pf_pool_bind */
  PF_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
  PF_ERR_HIP = -6,          /* the HIP runtime reported an error at launch */
  PF_ERR_UNSUPPORTED = -7,  /* valid but not built: block size / head dim */
  PF_ERR_SHARED = -8,       /* growth would write into a page another table shares */
  PF_ERR_SWAPPED = -9,      /* the sequence is swapped out (pf_swap_out) */
  PF_ERR_HOST_MEMORY = -10, /* host memory for the handle's own state ran out; any entry
                               point that grows the handle's state may return it (a batch
                               may then be partly applied: treat the handle as lost) */
  PF_ERR_SCRATCH = -11      /* the call needs more workspace than the library's fixed device
                               scratch holds (pf_paged_decode_attention_noalloc) */
} pf_status;

typedef struct {
  int32_t num_pages;     /* physical pages in the pool, >= 1 */
  int32_t block_size;    /* tokens per page; kernels are built for 16 */
  int32_t num_layers;    /* layers sharing the pool, >= 1 */
  int32_t num_kv_heads;  /* kv heads per layer, >= 1 */
  int32_t head_dim;      /* kernels: 16, 32, 64, 128 or 256 */
  int32_t dtype;         /* pf_dtype */
} pf_geometry;

typedef struct pf_pool pf_pool; /* opaque, host-owned */

/* ---------------------------------------------------------------- allocator */

/* Create a handle.  initial_free_order (nullable) is a permutation of
 * 0..num_pages-1 giving the order in which a fresh pool hands pages out
 * (index 0 first); NULL means 0, 1, 2, ... (mini-infer, "Implementation
 * Walkthrough": a fresh stack pops block 0 first).  A shuffled order models a
 * pool after churn (PageFault, "Four stages", stage 3: ordered and shuffled
 * frames).  *out receives the handle.  Errors: PF_ERR_INVALID. */
int pf_pool_create(const pf_geometry* geom, const int32_t* initial_free_order, pf_pool** out);

/* Destroy a handle (NULL is ignored).  Does not touch the bound device memory. */
void pf_pool_destroy(pf_pool* pool);

/* Bytes the device pool needs: num_pages * L * H * 2 * B * D * element size. */
size_t pf_pool_bytes(const pf_pool* pool);

/* Bytes of one page (all layers, heads, K and V). */
size_t pf_page_bytes(const pf_pool* pool);

/* Bind caller-owned device memory of at least pf_pool_bytes bytes, 256-byte
 * aligned: the one allocation that holds every page of the pool (PageFault,
 * "Four stages", stage 2: one device allocation for the whole pool, from which
 * a free list hands out frames; PageForge, "Four layers": K and V combined in
 * one pool).
 * Errors: PF_ERR_INVALID (null, too small, misaligned). */
int pf_pool_bind(pf_pool* pool, void* dev_ptr, size_t bytes);

/* Grow sequence seq_id to new_len tokens in total, taking
 * ceil(new_len/B) - (pages it has) pages from the top of the free stack and
 * appending them to its table in pop order.  An unknown id creates the
 * sequence.  *n_new_pages (nullable) receives the number of pages taken.
 * Errors: PF_ERR_INVALID (new_len < 0 or below the current length),
 * PF_ERR_OOM (not enough free pages: all or nothing, nothing changes; PageFault,
 * "Test": exhaustion and all-or-nothing), PF_ERR_SHARED (the growth would
 * write into the sequence's partly filled last page while another sequence
 * shares it, see pf_fork_seq; nothing changes: use pf_grow_seqs, which copies
 * it first).  Checked in the order INVALID, SHARED, OOM.  O(1) per page. */
int pf_alloc_for_seq(pf_pool* pool, uint64_t seq_id, int32_t new_len, int32_t* n_new_pages);

/* Batch form of pf_alloc_for_seq for one decode step: grow seq_ids[i] to
 * new_lens[i] for i = 0..n-1, in order, under one lock.  All or nothing over
 * the whole batch: if any entry is invalid (PF_ERR_INVALID, checked first,
 * against the lengths earlier entries would leave) or the pages do not suffice
 * (PF_ERR_OOM), nothing changes; PF_ERR_SHARED as pf_alloc_for_seq, checked
 * after INVALID and before OOM.  n_new_pages (nullable) is [n].
 * A sequence may appear more than once; later entries see earlier growth. */
int pf_alloc_for_seqs(pf_pool* pool, const uint64_t* seq_ids, const int32_t* new_lens, int32_t n,
                      int32_t* n_new_pages);

/* Copy-on-write sharing (PagedAttention blog, "Copy-on-Write for Parallel
 * Sampling": sequences sampled from one prompt hold the prompt's blocks once,
 * a reference count per block tracks the sharing, and a block is copied only
 * when a sequence writes into it).
 *
 * Fork: child gets parent's table and length; every page of it is now held by
 * one more table.  No page is taken or copied.  Errors: PF_ERR_UNKNOWN_SEQ
 * (parent not live), PF_ERR_INVALID (child already live). */
int pf_fork_seq(pf_pool* pool, uint64_t parent, uint64_t child);

/* Copy-on-write form of pf_alloc_for_seqs.  Entry i grows seq_ids[i] to
 * new_lens[i] (an unknown id creates the sequence).  If the growth writes
 * into the sequence's partly filled last page while another table holds that
 * page, a fresh page is taken first, the pair (shared page, fresh page) is
 * appended to copies, and the fresh page replaces the shared one in this
 * sequence's table only (the shared page's count drops by one); then new pages
 * are appended as usual.  At most one copy per entry, taken before that
 * entry's new pages.  The caller must run the copies (pf_copy_pages) before
 * anything writes into the fresh pages.
 *   n_new_pages  nullable [n]: pages taken by entry i, its copy included.
 *   copies       [2n] int32, filled with *n_copies (source, destination) pairs
 *                in entry order.
 * All or nothing over the batch: PF_ERR_INVALID (a length below what earlier
 * entries leave, checked first), PF_ERR_OOM (pages, copies included, do not
 * suffice); on error nothing changes and *n_copies = 0. */
int pf_grow_seqs(pf_pool* pool, const uint64_t* seq_ids, const int32_t* new_lens, int32_t n,
                 int32_t* n_new_pages, int32_t* copies, int32_t* n_copies);

/* Number of tables holding page (0 = on the free stack); -1 for a bad page id
 * or a NULL handle. */
int32_t pf_page_refcount(const pf_pool* pool, int32_t page);

/* Swapping (PagedAttention blog, "Preemption and Swapping": a sequence's blocks
 * are evicted to CPU memory and copied back when it resumes; swapping works on
 * blocks, so some blocks of a sequence may be on the GPU and others on the
 * CPU).  Whole sequences (pf_swap_out, pf_swap_in) or a block range of one
 * sequence (pf_swap_out_blocks, pf_swap_in_blocks).
 *
 * Bind a host backing store: host_ptr is caller-owned pinned memory
 * (hipHostMalloc / pin_memory), 16-byte aligned, of at least
 * num_slots * pf_page_bytes bytes; slot k is bytes [k, k+1) * pf_page_bytes,
 * laid out like a page.  Slots are handed out from a LIFO stack, slot 0 first.
 * Re-binding resets the stack and is refused (PF_ERR_INVALID) while any
 * sequence is swapped out. */
int pf_swap_bind(pf_pool* pool, void* host_ptr, size_t bytes, int32_t num_slots);

/* Free host slots (-1 for a NULL handle). */
int32_t pf_swap_free_slots(const pf_pool* pool);

/* *swapped = 1 if any block of seq_id is on the host (swapped out), else 0.
 * Errors: PF_ERR_UNKNOWN_SEQ. */
int pf_seq_swapped(const pf_pool* pool, uint64_t seq_id, int32_t* swapped);

/* Where each block of seq_id is: pages[b] = its device page, or -1 while it
 * is on the host, and slots[b] = its host slot, or -1 while it is on the
 * device, for b < *num_blocks = ceil(length / B).  pages and slots hold
 * max_blocks entries.  Errors: PF_ERR_UNKNOWN_SEQ, PF_ERR_INVALID (NULL
 * pointers, or more blocks than max_blocks: *num_blocks is still set). */
int pf_seq_blocks(const pf_pool* pool, uint64_t seq_id, int32_t max_blocks, int32_t* pages, int32_t* slots,
                  int32_t* num_blocks);

/* Swap whole sequences out: each page of each sequence's table, in order, is
 * assigned a host slot and enqueued on the stream for copying device -> host;
 * the sequence then drops its hold on those pages (pages no other table holds
 * return to the free stack, last first, as pf_free_seq would push them; pages
 * still shared stay with their other holders).  The sequence keeps its length
 * and is "swapped": growing, forking or exporting it fails with
 * PF_ERR_SWAPPED until every block is back (pf_swap_in, pf_swap_in_blocks);
 * pf_free_seq releases its slots.  A sequence of length 0 has no block to
 * move: it is marked swapped all the same, with no copy, until pf_swap_in.
 *   staging_host  caller-owned pinned memory, 8-byte aligned, of
 *                 staging_words int32 >= 2 * (pages of the sequences); receives
 *                 the (page, slot) pairs that the copy kernel reads when it
 *                 runs (keep it unchanged until the stream has passed the call).
 * The copy is enqueued before the call returns, so anything enqueued later on
 * the same stream (writes into the freed pages included) runs after it.
 * All or nothing over the batch.  Errors: PF_ERR_INVALID (a repeated id, a
 * small staging), PF_ERR_UNKNOWN_SEQ, PF_ERR_SWAPPED (some block already
 * out), PF_ERR_OOM (not enough free slots), PF_ERR_UNBOUND (no device pool or
 * no swap space), PF_ERR_HIP. */
int pf_swap_out(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t* staging_host,
                int64_t staging_words, void* hip_stream);

/* Swap sequences back in: every block of each that is on the host, in block
 * order, gets a fresh page from the free stack (pop order) and is enqueued
 * for copying host -> device; the slots return to their stack, last block
 * first.  Staging and ordering as pf_swap_out, with (slot, page) pairs.  All
 * or nothing; a swapped sequence of length 0 comes back with no copy.
 * Errors: PF_ERR_INVALID (a repeated id, a sequence that is not swapped, a
 * small staging), PF_ERR_UNKNOWN_SEQ, PF_ERR_OOM (not enough free pages),
 * PF_ERR_UNBOUND, PF_ERR_HIP. */
int pf_swap_in(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t* staging_host,
               int64_t staging_words, void* hip_stream);

/* Swap out blocks [first_block, first_block + num_blocks) of one sequence,
 * every one of them on the device: as pf_swap_out for those blocks only (a
 * slot per block in block order, (page, slot) pairs in staging_host of at
 * least 2 * num_blocks words, the pages released last block first).  The
 * sequence's other blocks stay where they are; it counts as swapped (no
 * growth, fork or export) while any block is on the host.  All or nothing.
 * Errors: PF_ERR_UNKNOWN_SEQ, PF_ERR_INVALID (num_blocks < 1, a range outside
 * the table, a block in it already on the host, a small or misaligned
 * staging), PF_ERR_OOM (not enough free slots), PF_ERR_UNBOUND, PF_ERR_HIP.
 * A null or misaligned staging is refused first (PF_ERR_INVALID); then
 * checked in the order UNBOUND, UNKNOWN_SEQ, INVALID, OOM. */
int pf_swap_out_blocks(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks,
                       int32_t* staging_host, int64_t staging_words, void* hip_stream);

/* Swap in blocks [first_block, first_block + num_blocks) of one sequence,
 * every one of them on the host (for instance fetching a swapped-out
 * sequence's blocks back one at a time): fresh pages in block order, (slot,
 * page) pairs, slots returned last block first.  When the last block on the
 * host comes back, the sequence is resident again.  All or nothing.  Errors:
 * as pf_swap_out_blocks, with PF_ERR_INVALID for a block in the range that is
 * on the device and PF_ERR_OOM for too few free pages. */
int pf_swap_in_blocks(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks,
                      int32_t* staging_host, int64_t staging_words, void* hip_stream);

/* Host halves of the swaps, with no launch: the state changes exactly as
 * pf_swap_out (to_host != 0) / pf_swap_in, resp. pf_swap_out_blocks /
 * pf_swap_in_blocks, would change it, and staging_host (any host memory)
 * receives the (page, slot) / (slot, page) pairs, *pairs of them.  The caller
 * must make those copies (a page-sized copy per pair between the bound pool
 * and the bound host store) before the pages or slots are used again.  For
 * callers that move pages themselves, and for tests.  Errors: as the calls,
 * plus PF_ERR_INVALID for a NULL pairs. */
int pf_swap_staging(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t to_host, int32_t* staging_host,
                    int64_t staging_words, int32_t* pairs);
int pf_swap_blocks_staging(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks, int32_t to_host,
                           int32_t* staging_host, int64_t staging_words, int32_t* pairs);

/* Release seq_id's hold on each of its pages and forget the sequence; pages no
 * other table holds go back on the free stack, last page first (so the
 * sequence's first page ends on top).  PageForge, "Four layers, one pointer
 * moving through all of them": free_seq returns a finished sequence's pages to
 * the free list in O(1) per page; "Does the pool actually come back to zero?":
 * a freed batch leaves the pool whole.
 * Errors: PF_ERR_UNKNOWN_SEQ (never allocated or already freed). */
int pf_free_seq(pf_pool* pool, uint64_t seq_id);

/* Pages currently on the free stack (-1 for a NULL handle).  PageForge, "Four
 * layers, one pointer moving through all of them": the allocator reports its
 * free page count (free_pages), which returns to the pool size once every
 * sequence is freed. */
int32_t pf_free_pages(const pf_pool* pool);

/* Most pages in use at once since the handle was created or the peak was last
 * reset (PageFault, "Project layout": the host free list records its peak;
 * PageForge, "Does the pool actually come back to zero?": a batch's paged peak
 * against the naive reservation).  -1 for a NULL handle. */
int32_t pf_pool_peak_pages(const pf_pool* pool);

/* Restart the peak from the pages in use now.  Errors: PF_ERR_INVALID. */
int pf_pool_reset_peak(pf_pool* pool);

/* Number of live sequences, resident or swapped out (-1 for a NULL handle). */
int32_t pf_num_seqs(const pf_pool* pool);

/* Current length of seq_id.  Errors: PF_ERR_UNKNOWN_SEQ, PF_ERR_INVALID. */
int pf_seq_len(const pf_pool* pool, uint64_t seq_id, int32_t* len);

/* Export dense host tables for n sequences: bt_host is [n][max_blocks] int32,
 * row i = the block table of seq_ids[i] padded with -1; lens_host (nullable)
 * is [n] int32 lengths (PagedAttention blog, "Architecture": a block table is
 * an int32 array of max_blocks_per_seq entries mapping logical block i to a
 * physical block; the blog zero-fills the unused entries and keeps the block
 * count beside them, here they are -1, which names no page).  Rows follow the
 * order of seq_ids (an id may repeat).  Errors: PF_ERR_UNKNOWN_SEQ, PF_ERR_INVALID (a table
 * longer than max_blocks, null pointers with n > 0), PF_ERR_SWAPPED. */
int pf_block_tables(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                    int32_t* bt_host, int32_t* lens_host);

/* ------------------------------------------------------------------ kernels */

/* The per-step host -> device table export in one call: fill staging_host
 * (caller-owned pinned memory, hipHostMalloc / pin_memory, 16-byte aligned)
 * with int32 [n][max_blocks] block tables (rows of seq_ids, padded with -1),
 * then [n] lengths, then [n] newest positions (length - 1), and enqueue on
 * the stream one kernel that copies those n*max_blocks + 2n words to meta_dev
 * (device, 16-byte aligned), reading the pinned memory directly (no DMA
 * engine round trip).  The staging buffer must not be rewritten until the
 * stream has passed this call.  With PF_OPT_EXPORT_DELTA the table part of
 * the staging may instead hold (flat index, value) pairs of the entries that
 * changed since the previous export to meta_dev, and only those entries,
 * the lengths and the newest positions are written (a decode step changes at
 * most one entry per sequence).  Errors: as pf_block_tables, plus
 * PF_ERR_INVALID for null or misaligned buffers and PF_ERR_HIP. */
int pf_export_tables(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                     int32_t* staging_host, int32_t* meta_dev, void* hip_stream);

/* Host half of pf_export_tables (step = 0) or of pf_decode_prepare's export
 * (step != 0), with no launch: fill staging_host exactly as that call would
 * for an export to meta_dev and count the export as made (the next
 * incremental one builds on it).  meta_dev only names the target for
 * PF_OPT_EXPORT_DELTA and is not accessed.  *pairs receives -1 when the
 * staging holds the whole table ([n][max_blocks] at the start), else the
 * number of (flat index, value) pairs at the start; lengths always at word
 * n*max_blocks, newest positions at n*max_blocks + n and, with step, the
 * pages of the newest tokens at n*max_blocks + 2n.  For callers that upload
 * the staging themselves, and for tests.  Errors: as pf_block_tables, plus
 * PF_ERR_INVALID for null buffers. */
int pf_export_staging(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                      const void* meta_dev, int32_t step, int32_t* staging_host, int64_t* pairs);

/* One decode step's host -> device work in one launch: pf_export_tables of
 * seq_ids into meta_dev (same staging layout, followed by [n] destination
 * pages, so staging_host needs n*max_blocks + 3n words) together with the
 * scatter of each sequence's newest token (position length - 1) for layers
 * layer0 .. layer0 + num_layers - 1, as pf_scatter_kv would do it.
 *   k, v  device [num_layers][n][H][D] in the pool dtype, 16-byte aligned.
 * Sequences of length 0 scatter nothing.  Errors: as pf_export_tables, plus
 * PF_ERR_UNBOUND and PF_ERR_INVALID for a bad layer range or pointers. */
int pf_decode_prepare(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                      int32_t* staging_host, int32_t* meta_dev, const void* k, const void* v,
                      int32_t layer0, int32_t num_layers, void* hip_stream);

/* Write num_tokens tokens' K and V into their page slots for one layer.
 *   k, v     device [num_tokens][H][D] in the pool dtype.
 *   tok_seq  device [num_tokens] int32: row of bt_dev holding the token's table.
 *   tok_pos  device [num_tokens] int32: the token's logical position.
 *   bt_dev   device [num_rows][max_blocks] int32 block tables.
 * Token t lands in page bt_dev[tok_seq[t]][tok_pos[t] / B], slot tok_pos[t] % B
 * (PageFault, "The OS analogy").  A token whose row, position or table entry is
 * out of range writes nothing (no access outside the pool).  Two tokens mapped
 * to the same slot race.  Errors: PF_ERR_INVALID, PF_ERR_UNBOUND, PF_ERR_HIP. */
int pf_scatter_kv(const pf_pool* pool, int32_t layer, const void* k, const void* v,
                  const int32_t* tok_seq, const int32_t* tok_pos, int32_t num_tokens,
                  const int32_t* bt_dev, int32_t num_rows, int32_t max_blocks, void* hip_stream);

/* Run copy-on-write copies: for j < n, page pairs[2j] is copied to page
 * pairs[2j+1] -- the whole page, every layer, head, K and V, all slots.
 *   pairs  int32 [n][2], 8-byte aligned, in device memory or in pinned host
 *          memory (read by the kernel when it runs: keep it unchanged until
 *          the stream has passed this call); as pf_grow_seqs reports them.
 * A pair with an id outside the pool copies nothing.  A destination that is
 * also another pair's source or destination races.
 * Errors: PF_ERR_INVALID, PF_ERR_UNBOUND, PF_ERR_UNSUPPORTED (page size not a
 * multiple of 16 bytes), PF_ERR_HIP. */
int pf_copy_pages(const pf_pool* pool, const int32_t* pairs, int32_t n, void* hip_stream);

/* Read back sequences' K and V through their tables into contiguous buffers
 * k_out, v_out: device [n][max_len][H][D] in the pool dtype (PageForge, "Five
 * techniques": gather_kv assembles scattered pages into a contiguous view).
 * Positions >= min(lens_dev[i], max_len) are not written.  Table entries that
 * are not valid pages leave their tokens unwritten.
 * Errors: PF_ERR_INVALID, PF_ERR_UNBOUND, PF_ERR_HIP. */
int pf_gather_kv(const pf_pool* pool, int32_t layer, const int32_t* bt_dev, const int32_t* lens_dev,
                 int32_t n, int32_t max_blocks, int32_t max_len, void* k_out, void* v_out,
                 void* hip_stream);

/* Workspace bytes pf_paged_decode_attention needs for these sizes under the
 * handle's current options (0 means none is needed). */
size_t pf_attention_workspace_bytes(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                    int32_t max_context_len);

/* Decode attention for one layer (PagedAttention blog, "The Attention Kernel";
 * PageFault, "Four stages", stage 3): for every sequence i and query head h,
 *     out[i][h] = softmax(scale * K_i q[i][h]) V_i
 * over the first ctx_dev[i] tokens of sequence i, read through row i of bt_dev,
 * with K_i, V_i of kv head h / (num_q_heads / H) (grouped-query heads are
 * consecutive).  Tokens at positions >= the length are never read.
 *   q        device [n][num_q_heads][D], pool dtype, 16-byte aligned.
 *   bt_dev   device [n][max_blocks] int32 tables (-1 padding is never read).
 *   ctx_dev  device [n] int32 lengths; each is clamped to [0, max_context_len].
 *   max_context_len  host bound on the lengths, <= max_blocks * B; sizes the grid.
 *   scale    <= 0 selects 1/sqrt(D).
 *   out      device [n][num_q_heads][D] in out_dtype (PF_F32 or the pool dtype),
 *            16-byte aligned.
 *   workspace  device, >= pf_attention_workspace_bytes(...), 256-byte aligned
 *            (nullable when that is 0); holds split-K partials.
 * Math is fp32 with an online softmax.  Work is split either into fixed token
 * ranges per (sequence, head) or, by default, into equal slices of all
 * sequences' pages (balanced schedule); partial results are merged by
 * log-sum-exp in a second kernel, in a fixed order.  The split depends only on
 * the lengths, so results depend only on logical positions (the same bits for
 * any physical page order).  A length of 0 gives a zero output.  A table entry
 * that is not a valid page contributes nothing (no access outside the pool).
 * Pools of 8-, 32- or 64-token pages and fp32 pools at head dim 256 (walked
 * in 8-token units) always use the balanced schedule and take n <= 2048.
 * Errors: PF_ERR_INVALID, PF_ERR_UNBOUND, PF_ERR_WORKSPACE, PF_ERR_UNSUPPORTED,
 * PF_ERR_HIP. */
int pf_paged_decode_attention(const pf_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                              const int32_t* bt_dev, int32_t max_blocks, const int32_t* ctx_dev,
                              int32_t n, int32_t max_context_len, float scale, void* out,
                              int32_t out_dtype, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/* pf_paged_decode_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result, with the split partials in a
 * fixed array of 16 MiB (PF_NOALLOC_SCRATCH_BYTES) of device memory inside
 * the library instead of a caller's workspace.  Each GPU the library runs on
 * holds its own copy until the process ends; the first call on a device asks
 * the runtime for the copy's address (no allocation).  Nothing is allocated
 * or freed by this call.  Every call on one GPU uses that GPU's copy, which
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls that overlap on one GPU (on different streams, or from different
 * threads before the first has run) race on it, and their results are
 * undefined.  The stream's device selects the copy (NULL: the current
 * device).  Arguments as pf_paged_decode_attention without the workspace.
 * Errors: as pf_paged_decode_attention, plus PF_ERR_SCRATCH when
 * pf_attention_workspace_bytes for these sizes exceeds the scratch (nothing
 * is enqueued), PF_ERR_HIP when the runtime gives no address. */
#define PF_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pf_paged_decode_attention_noalloc(const pf_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                                      const int32_t* bt_dev, int32_t max_blocks, const int32_t* ctx_dev, int32_t n,
                                      int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                      void* hip_stream);

/* pf_scatter_kv of each sequence's newest token fused into
 * pf_paged_decode_attention, in one launch (PageForge, "Five techniques" and its
 * roadmap: the per-step scatter launches are the cost to remove).  For every
 * sequence i with ctx_dev[i] > 0, the token at position ctx_dev[i] - 1 has K
 * and V k_new[i], v_new[i] ([H][D] each): it is written into its slot of page
 * bt_dev[i][(ctx-1)/B] for `layer`, and the attention uses it as that token.
 * The result and the pool afterwards are those of pf_scatter_kv (those tokens,
 * that layer) followed by pf_paged_decode_attention.  If the newest token's
 * table entry is not a valid page, nothing is written and that page's tokens
 * contribute nothing (as for any invalid entry).
 *   k_new, v_new  device [n][H][D], pool dtype, 16-byte aligned.
 * Other arguments as pf_paged_decode_attention.  Built for 16-token pages
 * and head dims whose rows are a multiple of 16 bytes (PF_ERR_UNSUPPORTED
 * otherwise).  Errors: as pf_paged_decode_attention. */
int pf_paged_decode_attention_append(const pf_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                                     const void* k_new, const void* v_new, const int32_t* bt_dev,
                                     int32_t max_blocks, const int32_t* ctx_dev, int32_t n,
                                     int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* The same attention over a contiguous per-sequence cache, with no table walk
 * (PageFault, "Four stages": stage 1's contiguous cache is the baseline that
 * stage 3's paged kernel is checked and timed against).  The kernels,
 * schedule, split and merge are those of pf_paged_decode_attention; only the
 * address of a 16-token block differs, so for the same K/V values, lengths and
 * handle options the two entry points return the same bits.
 *   pool     supplies the dtype, H, D and the kernel options only; it need not
 *            be bound and its memory is not read.
 *   k, v     device, pool dtype, 16-byte aligned.  Element d of kv head h of
 *            token t of sequence i is k[i*seq_stride + t*token_stride +
 *            h*head_stride + d] (strides in elements; each stride times the
 *            element size a multiple of 16 bytes).  [n][max_len][H][D] (the
 *            layout pf_gather_kv writes) and [n][H][max_len][D] are both of
 *            this form.  The kernel reads tokens t < round_up(length, B) of
 *            every sequence, all within max_len.
 *   max_len  tokens per sequence in the cache, a positive multiple of B.
 *   q, ctx_dev, n, max_context_len (<= max_len), scale, out, out_dtype,
 *   workspace (sized by pf_attention_workspace_bytes): as
 *            pf_paged_decode_attention.
 * Errors: PF_ERR_INVALID, PF_ERR_WORKSPACE, PF_ERR_UNSUPPORTED, PF_ERR_HIP. */
int pf_contiguous_decode_attention(const pf_pool* pool, const void* q, int32_t num_q_heads, const void* k,
                                   const void* v, int64_t seq_stride, int64_t token_stride, int64_t head_stride,
                                   int32_t max_len, const int32_t* ctx_dev, int32_t n, int32_t max_context_len,
                                   float scale, void* out, int32_t out_dtype, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------ options */

typedef enum {
  PF_OPT_SPLIT_TOKENS = 0, /* fixed-split schedule: tokens per split (multiple of B, <= 64 B); 0 = automatic */
  PF_OPT_GQA_MFMA = 1,     /* 1 (default): matrix-core kernel for grouped 16-bit heads; 0: vector kernel */
  PF_OPT_SCHEDULE = 2,     /* 0 (default): one split per (sequence, head) when max_context_len <= 256
                              (16-token pages, no split-tokens option set: no merge launch), else
                              balanced if n <= 2048, else fixed splits; 1: fixed splits;
                              2: balanced (n <= 2048).  Pools of other page sizes and fp32 pools
                              at head dim 256 are always balanced. */
  PF_OPT_WAVES_PER_CU = 3, /* balanced schedule: waves launched per compute unit; 0 (default) = 8,
                              or the kernel's resident capacity per CU if that is lower */
  PF_OPT_EXPORT_DELTA = 4  /* 0 (default): pf_export_tables / pf_decode_prepare upload the whole table;
                              1: they upload only the entries that differ from the previous export to
                              the same meta_dev with the same seq_ids and max_blocks (lengths and
                              newest positions always).  With 1 the caller promises that meta_dev
                              is written by nothing else between exports and still holds what the
                              previous export left there; setting the option (to either value)
                              forgets the previous export, so set it again after meta_dev is
                              reallocated or overwritten. */
} pf_option;

/* Set / read a tuning option of a handle.  Errors: PF_ERR_INVALID. */
int pf_pool_set_option(pf_pool* pool, int32_t option, int32_t value);
int pf_pool_get_option(const pf_pool* pool, int32_t option, int32_t* value);

/* Tokens per split the fixed-split schedule will use for these sizes (the
 * automatic choice or the option); 0 when the balanced schedule is chosen. */
int32_t pf_attention_split_tokens(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                  int32_t max_context_len);

/* Waves the balanced schedule will launch for these sizes; 0 when the
 * fixed-split schedule is chosen. */
int32_t pf_attention_waves(const pf_pool* pool, int32_t n, int32_t num_q_heads, int32_t max_context_len);

/* Instrumentation: when both are non-NULL, every later
 * pf_paged_decode_attention call on this handle records start_event right
 * before its partition kernel and stop_event right after it, on the call's
 * stream (hipEvent_t values cast to void*, owned by the caller).  NULL, NULL
 * turns it off.  Errors: PF_ERR_INVALID (NULL handle or only one event). */
int pf_pool_set_timing_events(pf_pool* pool, void* start_event, void* stop_event);

/* Stream markers: HIP events created without the system-scope cache
 * writeback and invalidation that default events perform when they are
 * recorded (hipEventDisableSystemFence).  On MI355X a default event placed
 * between two kernels adds about 6 us to the stream; these add none of that.
 * A marker tells the host that the work enqueued before it has run (so, for
 * instance, pinned staging read by that work may be rewritten) and, if
 * created with timing, when; it does not make device writes visible to the
 * host.  The event is returned as a hipEvent_t cast to void* and is owned by
 * the caller until pf_marker_destroy.
 *   pf_marker_create: timing != 0 keeps timestamps (for pf_marker_elapsed_ms
 *                     and pf_pool_set_timing_events).
 *   pf_marker_record: enqueue on hip_stream (NULL: the null stream).
 *   pf_marker_wait:   block the host until the marker has been reached.
 *   pf_marker_elapsed_ms: milliseconds from start to stop, both reached and
 *                     created with timing.
 * Errors: PF_ERR_INVALID (NULL event or output), PF_ERR_HIP (the runtime
 * refused, e.g. a marker never recorded). */
int pf_marker_create(int32_t timing, void** event);
int pf_marker_record(void* event, void* hip_stream);
int pf_marker_wait(void* event);
int pf_marker_elapsed_ms(void* start, void* stop, float* ms);
int pf_marker_destroy(void* event);

/* Which attention kernel a call with num_q_heads query heads would use:
 * 1 = matrix-core kernel for grouped heads, 0 = vector kernel, -1 = NULL handle
 * or bad head count. */
int32_t pf_attention_kernel(const pf_pool* pool, int32_t num_q_heads);

/* Static description of a status code. */
const char* pf_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PF_H */
