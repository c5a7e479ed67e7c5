// Host page allocator of libpf: an O(1) LIFO free list of fixed-size pages and
// one block table per sequence.
//
// Follows PageForge, "Four layers, one pointer moving through all of them"
// (a free list plus a sequence -> page-ids table behind one object whose
// alloc_for_seq / free_seq are O(1) per page), mini-infer, "Implementation
// Walkthrough" (the free list is a stack that hands out block 0 first from a
// fresh pool, and an empty pool is an error), the PagedAttention blog,
// "Architecture" (a block is taken only when the last one is full; tables only
// grow) and PageFault, "Test" (exhaustion, double free and all-or-nothing are
// checked).  Freed pages go back last-page-first so a sequence of the same shape
// allocated next gets the same pages in the same order (PageForge, "Does the
// pool actually come back to zero?": batch 2 claims batch 1's pages).
//
// Copy-on-write sharing (PagedAttention blog, "Copy-on-Write for Parallel
// Sampling"): tables may hold the same page; refs[page] counts them.  A fork
// shares the parent's whole table; a free returns only pages nobody else
// holds; a growth that would write into a shared page (only a partly filled
// last page can be written: tokens are appended) either copies it first
// (pf_grow_seqs, which reports the copy for pf_copy_pages) or is refused
// (pf_alloc_for_seq / pf_alloc_for_seqs, PF_ERR_SHARED).
//
// Swapping (PagedAttention blog, "Preemption and Swapping"): blocks move to
// page-sized slots of a caller-owned pinned host store and back -- whole
// sequences, or a block range of one sequence, so that some of its blocks are
// on the device and others on the host; the state changes here, the copies
// are enqueued by pf_swap_out / pf_swap_in / pf_swap_out_blocks /
// pf_swap_in_blocks (pf_kv.hip) in the same call.  A sequence with blocks on
// the host keeps its length and its slots; it cannot grow, fork or be
// exported until every block is back.
#include <algorithm>
#include <cstring>
#include <limits>
#include <memory>
#include <new>

#include "pf_internal.h"

size_t pf_elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PF_F32: return 4;
    case PF_F16: return 2;
    case PF_BF16: return 2;
    default: return 0;
  }
}

// True if growing e (length len) to new_len writes into its last page while
// another table holds that page too.
static bool writes_shared(const pf_pool* pool, const pf_seq_entry& e, int32_t new_len) {
  return new_len > e.len && e.len % pool->g.block_size != 0 && !e.pages.empty() &&
         pool->refs[(size_t)e.pages.back()] > 1;
}

static int32_t pop_page(pf_pool* pool) {
  const int32_t p = pool->stack.back();
  pool->stack.pop_back();
  pool->refs[(size_t)p] = 1;
  const int32_t used = pool->g.num_pages - (int32_t)pool->stack.size();
  if (used > pool->peak) pool->peak = used;
  return p;
}

static bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > std::numeric_limits<size_t>::max() / a) return false;
  *out = a * b;
  return true;
}

// Host memory for the allocator's own state (vectors and maps) can run out;
// no C++ exception may cross the C ABI, so the entry points that allocate run
// their body through guarded().
template <class F>
static int guarded(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return PF_ERR_HOST_MEMORY;
  } catch (...) {
    return PF_ERR_INVALID;
  }
}

extern "C" {

int pf_pool_create(const pf_geometry* geom, const int32_t* initial_free_order, pf_pool** out) {
  if (!geom || !out) return PF_ERR_INVALID;
  *out = nullptr;
  const pf_geometry& g = *geom;
  if (g.num_pages <= 0 || g.block_size <= 0 || g.num_layers <= 0 || g.num_kv_heads <= 0 ||
      g.head_dim <= 0 || pf_elem_bytes(g.dtype) == 0)
    return PF_ERR_INVALID;
  size_t pe = 1;
  if (!mul_ok(pe, (size_t)g.num_layers, &pe) || !mul_ok(pe, (size_t)g.num_kv_heads, &pe) ||
      !mul_ok(pe, 2, &pe) || !mul_ok(pe, (size_t)g.block_size, &pe) ||
      !mul_ok(pe, (size_t)g.head_dim, &pe))
    return PF_ERR_INVALID;
  size_t total = 0;
  if (!mul_ok(pe, (size_t)g.num_pages, &total) || !mul_ok(total, pf_elem_bytes(g.dtype), &total))
    return PF_ERR_INVALID;
  return guarded([&]() -> int {
  std::unique_ptr<pf_pool> p(new pf_pool());
  p->g = g;
  p->elem_bytes = pf_elem_bytes(g.dtype);
  p->page_elems = pe;
  p->stack.resize((size_t)g.num_pages);
  p->refs.assign((size_t)g.num_pages, 0);
  if (initial_free_order) {
    std::vector<uint8_t> seen((size_t)g.num_pages, 0);
    for (int32_t i = 0; i < g.num_pages; ++i) {
      int32_t v = initial_free_order[i];
      if (v < 0 || v >= g.num_pages || seen[(size_t)v]) return PF_ERR_INVALID;
      seen[(size_t)v] = 1;
    }
  }
  // order[0] must pop first: it goes on top, i.e. at the back.
  for (int32_t i = 0; i < g.num_pages; ++i)
    p->stack[(size_t)(g.num_pages - 1 - i)] = initial_free_order ? initial_free_order[i] : i;
  *out = p.release();
  return PF_OK;
  });
}

void pf_pool_destroy(pf_pool* pool) { delete pool; }

size_t pf_page_bytes(const pf_pool* pool) { return pool ? pool->page_elems * pool->elem_bytes : 0; }

size_t pf_pool_bytes(const pf_pool* pool) {
  return pool ? pool->page_elems * pool->elem_bytes * (size_t)pool->g.num_pages : 0;
}

int pf_pool_bind(pf_pool* pool, void* dev_ptr, size_t bytes) {
  if (!pool || !dev_ptr) return PF_ERR_INVALID;
  if (bytes < pf_pool_bytes(pool)) return PF_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(dev_ptr) % 256 != 0) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  pool->dev = dev_ptr;
  pool->dev_bytes = bytes;
  return PF_OK;
}

int pf_alloc_for_seq(pf_pool* pool, uint64_t seq_id, int32_t new_len, int32_t* n_new_pages) {
  return guarded([&]() -> int {
    if (n_new_pages) *n_new_pages = 0;
    if (!pool || new_len < 0) return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    auto it = pool->seqs.find(seq_id);
    if (it != pool->seqs.end() && it->second.swapped) return PF_ERR_SWAPPED;
    const int32_t cur_len = it == pool->seqs.end() ? 0 : it->second.len;
    const size_t have = it == pool->seqs.end() ? 0 : it->second.pages.size();
    if (new_len < cur_len) return PF_ERR_INVALID;
    if (it != pool->seqs.end() && writes_shared(pool, it->second, new_len)) return PF_ERR_SHARED;
    const int64_t B = pool->g.block_size;
    const size_t want = (size_t)(((int64_t)new_len + B - 1) / B);
    const size_t need = want - have;
    if (need > pool->stack.size()) return PF_ERR_OOM;  // all or nothing
    pf_seq_entry& e = it == pool->seqs.end() ? pool->seqs[seq_id] : it->second;
    e.pages.reserve(want);
    for (size_t i = 0; i < need; ++i) e.pages.push_back(pop_page(pool));
    if (need) e.ver = ++pool->ver_clock;
    e.len = new_len;
    if (n_new_pages) *n_new_pages = (int32_t)need;
    return PF_OK;
  });
}

// The common decode-step batch: every id names a distinct live resident
// sequence.  Resolves each entry once (no per-batch map) and applies the same
// checks, in the same order, as the general path below.  Returns -1 when the
// batch does not qualify (an unknown or repeated id): the general path then
// decides.  Caller holds the lock.
static int alloc_batch_fast(pf_pool* pool, const uint64_t* ids, const int32_t* lens, int32_t n,
                            int32_t* n_new_pages) {
  std::vector<pf_seq_entry*>& ents = pool->batch_entries;
  ents.resize((size_t)n);
  const uint64_t epoch = ++pool->batch_epoch;
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(ids[i]);
    if (it == pool->seqs.end() || it->second.batch_mark == epoch) return -1;
    it->second.batch_mark = epoch;
    ents[(size_t)i] = &it->second;
  }
  const int64_t B = pool->g.block_size;
  for (int32_t i = 0; i < n; ++i)   // negative lengths included: every length is >= 0
    if (lens[i] < ents[(size_t)i]->len) return PF_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i)
    if (ents[(size_t)i]->swapped) return PF_ERR_SWAPPED;
  size_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pf_seq_entry& e = *ents[(size_t)i];
    if (writes_shared(pool, e, lens[i])) return PF_ERR_SHARED;
    total += (size_t)(((int64_t)lens[i] + B - 1) / B) - e.pages.size();
  }
  if (total > pool->stack.size()) return PF_ERR_OOM;
  for (int32_t i = 0; i < n; ++i) {
    pf_seq_entry& e = *ents[(size_t)i];
    const size_t need = (size_t)(((int64_t)lens[i] + B - 1) / B) - e.pages.size();
    for (size_t j = 0; j < need; ++j) e.pages.push_back(pop_page(pool));
    if (need) e.ver = ++pool->ver_clock;
    e.len = lens[i];
    if (n_new_pages) n_new_pages[i] = (int32_t)need;
  }
  return PF_OK;
}

int pf_alloc_for_seqs(pf_pool* pool, const uint64_t* seq_ids, const int32_t* new_lens, int32_t n,
                      int32_t* n_new_pages) {
  return guarded([&]() -> int {
    if (!pool || n < 0 || (n > 0 && (!seq_ids || !new_lens))) return PF_ERR_INVALID;
    if (n_new_pages)
      for (int32_t i = 0; i < n; ++i) n_new_pages[i] = 0;
    std::lock_guard<std::mutex> lk(pool->mu);
    const int fast = alloc_batch_fast(pool, seq_ids, new_lens, n, n_new_pages);
    if (fast != -1) return fast;
    const int64_t B = pool->g.block_size;
    // Validation pass: lengths and page counts as the batch would leave them.
    // A sequence's last page is shared only if it is still the page it had
    // before the batch (pages taken in the batch are private).
    struct Pending {
      int32_t len;
      size_t pages;
      bool last_original;
    };
    std::unordered_map<uint64_t, Pending> pending;
    for (int32_t i = 0; i < n; ++i) {
      if (new_lens[i] < 0) return PF_ERR_INVALID;
      auto pit = pending.find(seq_ids[i]);
      int32_t cur_len = 0;
      if (pit != pending.end()) {
        cur_len = pit->second.len;
      } else {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it != pool->seqs.end()) cur_len = it->second.len;
      }
      if (new_lens[i] < cur_len) return PF_ERR_INVALID;
      pending[seq_ids[i]] = {new_lens[i], 0, true};
    }
    for (int32_t i = 0; i < n; ++i) {
      auto it = pool->seqs.find(seq_ids[i]);
      if (it != pool->seqs.end() && it->second.swapped) return PF_ERR_SWAPPED;
    }
    pending.clear();
    size_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
      auto pit = pending.find(seq_ids[i]);
      Pending cur{0, 0, false};
      auto it = pool->seqs.find(seq_ids[i]);
      if (pit != pending.end()) {
        cur = pit->second;
      } else if (it != pool->seqs.end()) {
        cur = {it->second.len, it->second.pages.size(), true};
      }
      if (cur.last_original && it != pool->seqs.end() && writes_shared(pool, it->second, new_lens[i]) &&
          cur.len == it->second.len)
        return PF_ERR_SHARED;
      const size_t want = (size_t)(((int64_t)new_lens[i] + B - 1) / B);
      total += want - cur.pages;
      pending[seq_ids[i]] = {new_lens[i], want, cur.last_original && want == cur.pages};
    }
    if (total > pool->stack.size()) return PF_ERR_OOM;
    for (int32_t i = 0; i < n; ++i) {
      pf_seq_entry& e = pool->seqs[seq_ids[i]];
      const size_t want = (size_t)(((int64_t)new_lens[i] + B - 1) / B);
      const size_t need = want - e.pages.size();
      for (size_t j = 0; j < need; ++j) e.pages.push_back(pop_page(pool));
      if (need) e.ver = ++pool->ver_clock;
      e.len = new_lens[i];
      if (n_new_pages) n_new_pages[i] = (int32_t)need;
    }
    return PF_OK;
  });
}

int pf_free_seq(pf_pool* pool, uint64_t seq_id) {
  if (!pool) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t>& slots = it->second.slots;  // blocks on the host: slots back last first
  for (size_t i = slots.size(); i-- > 0;)
    if (slots[i] >= 0) pool->slot_stack.push_back(slots[i]);
  const std::vector<int32_t>& pages = it->second.pages;
  for (size_t i = pages.size(); i-- > 0;)
    if (pages[i] >= 0 && --pool->refs[(size_t)pages[i]] == 0) pool->stack.push_back(pages[i]);
  pool->seqs.erase(it);
  return PF_OK;
}

int pf_fork_seq(pf_pool* pool, uint64_t parent, uint64_t child) {
  return guarded([&]() -> int {
    if (!pool) return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    auto it = pool->seqs.find(parent);
    if (it != pool->seqs.end() && it->second.swapped) return PF_ERR_SWAPPED;
    if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
    if (pool->seqs.count(child)) return PF_ERR_INVALID;
    pf_seq_entry copy = it->second;
    for (int32_t p : copy.pages) ++pool->refs[(size_t)p];
    copy.ver = ++pool->ver_clock;
    pool->seqs.emplace(child, std::move(copy));
    return PF_OK;
  });
}

int pf_grow_seqs(pf_pool* pool, const uint64_t* seq_ids, const int32_t* new_lens, int32_t n,
                 int32_t* n_new_pages, int32_t* copies, int32_t* n_copies) {
  return guarded([&]() -> int {
    if (n_copies) *n_copies = 0;
    if (!pool || n < 0 || (n > 0 && (!seq_ids || !new_lens || !copies || !n_copies))) return PF_ERR_INVALID;
    if (n_new_pages)
      for (int32_t i = 0; i < n; ++i) n_new_pages[i] = 0;
    std::lock_guard<std::mutex> lk(pool->mu);
    const int64_t B = pool->g.block_size;
    // Dry run over the batch: lengths (INVALID first), then the pages it takes,
    // copies included, with the reference counts as the batch changes them.
    struct Pending {
      int32_t len;
      size_t pages;
      int32_t last;  // last page id, or -1 for none / a page taken in this batch
    };
    std::unordered_map<uint64_t, int32_t> lens;
    for (int32_t i = 0; i < n; ++i) {
      if (new_lens[i] < 0) return PF_ERR_INVALID;
      auto lit = lens.find(seq_ids[i]);
      int32_t cur_len = 0;
      if (lit != lens.end()) {
        cur_len = lit->second;
      } else {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it != pool->seqs.end()) cur_len = it->second.len;
      }
      if (new_lens[i] < cur_len) return PF_ERR_INVALID;
      lens[seq_ids[i]] = new_lens[i];
    }
    for (int32_t i = 0; i < n; ++i) {
      auto it = pool->seqs.find(seq_ids[i]);
      if (it != pool->seqs.end() && it->second.swapped) return PF_ERR_SWAPPED;
    }
    std::unordered_map<uint64_t, Pending> pending;
    std::unordered_map<int32_t, int32_t> dref;  // reference count changes of the batch
    size_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
      Pending cur{0, 0, -1};
      auto pit = pending.find(seq_ids[i]);
      if (pit != pending.end()) {
        cur = pit->second;
      } else {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it != pool->seqs.end())
          cur = {it->second.len, it->second.pages.size(), it->second.pages.empty() ? -1 : it->second.pages.back()};
      }
      const bool cow = new_lens[i] > cur.len && cur.len % B != 0 && cur.last >= 0 &&
                       pool->refs[(size_t)cur.last] + dref[cur.last] > 1;
      const size_t want = (size_t)(((int64_t)new_lens[i] + B - 1) / B);
      total += want - cur.pages + (cow ? 1 : 0);
      if (cow) {
        --dref[cur.last];
        cur.last = -1;
      }
      if (want > cur.pages) cur.last = -1;
      pending[seq_ids[i]] = {new_lens[i], want, cur.last};
    }
    if (total > pool->stack.size()) return PF_ERR_OOM;
    int32_t nc = 0;
    for (int32_t i = 0; i < n; ++i) {
      pf_seq_entry& e = pool->seqs[seq_ids[i]];
      int32_t taken = 0;
      if (writes_shared(pool, e, new_lens[i])) {
        const int32_t src = e.pages.back();
        const int32_t dst = pop_page(pool);
        --pool->refs[(size_t)src];
        e.pages.back() = dst;
        copies[2 * nc] = src;
        copies[2 * nc + 1] = dst;
        ++nc;
        ++taken;
      }
      const size_t want = (size_t)(((int64_t)new_lens[i] + B - 1) / B);
      while (e.pages.size() < want) {
        e.pages.push_back(pop_page(pool));
        ++taken;
      }
      if (taken) e.ver = ++pool->ver_clock;
      e.len = new_lens[i];
      if (n_new_pages) n_new_pages[i] = taken;
    }
    *n_copies = nc;
    return PF_OK;
  });
}

int pf_swap_bind(pf_pool* pool, void* host_ptr, size_t bytes, int32_t num_slots) {
  return guarded([&]() -> int {
    if (!pool || num_slots < 0 || (num_slots > 0 && !host_ptr)) return PF_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(host_ptr) % 16 != 0) return PF_ERR_INVALID;
    size_t need = 0;
    if (!mul_ok(pool->page_elems * pool->elem_bytes, (size_t)num_slots, &need) || bytes < need)
      return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    for (const auto& kv : pool->seqs)
      if (kv.second.swapped) return PF_ERR_INVALID;  // slots in use
    pool->host = num_slots > 0 ? host_ptr : nullptr;
    pool->num_slots = num_slots;
    pool->slot_stack.resize((size_t)num_slots);
    for (int32_t i = 0; i < num_slots; ++i) pool->slot_stack[(size_t)(num_slots - 1 - i)] = i;
    return PF_OK;
  });
}

int32_t pf_swap_free_slots(const pf_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lk(pool->mu);
  return (int32_t)pool->slot_stack.size();
}

int pf_seq_swapped(const pf_pool* pool, uint64_t seq_id, int32_t* swapped) {
  if (!pool || !swapped) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
  *swapped = it->second.swapped ? 1 : 0;
  return PF_OK;
}

int pf_seq_blocks(const pf_pool* pool, uint64_t seq_id, int32_t max_blocks, int32_t* pages, int32_t* slots,
                  int32_t* num_blocks) {
  if (!pool || !num_blocks || max_blocks < 0 || (max_blocks > 0 && (!pages || !slots))) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
  const pf_seq_entry& e = it->second;
  const int32_t nb = (int32_t)e.pages.size();
  *num_blocks = nb;
  if (nb > max_blocks) return PF_ERR_INVALID;
  for (int32_t b = 0; b < nb; ++b) {
    pages[b] = e.pages[(size_t)b];
    slots[b] = e.slots.empty() ? -1 : e.slots[(size_t)b];
  }
  return PF_OK;
}

int32_t pf_page_refcount(const pf_pool* pool, int32_t page) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lk(pool->mu);
  if (page < 0 || page >= pool->g.num_pages) return -1;
  return pool->refs[(size_t)page];
}

int32_t pf_free_pages(const pf_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lk(pool->mu);
  return (int32_t)pool->stack.size();
}

int32_t pf_pool_peak_pages(const pf_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lk(pool->mu);
  return pool->peak;
}

int pf_pool_reset_peak(pf_pool* pool) {
  if (!pool) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  pool->peak = pool->g.num_pages - (int32_t)pool->stack.size();
  return PF_OK;
}

int32_t pf_num_seqs(const pf_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> lk(pool->mu);
  return (int32_t)pool->seqs.size();
}

int pf_seq_len(const pf_pool* pool, uint64_t seq_id, int32_t* len) {
  if (!pool || !len) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq_id);
  if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
  *len = it->second.len;
  return PF_OK;
}

int pf_block_tables(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                    int32_t* bt_host, int32_t* lens_host) {
  if (!pool || n < 0 || max_blocks < 0) return PF_ERR_INVALID;
  if (n > 0 && (!seq_ids || (!bt_host && max_blocks > 0))) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seq_ids[i]);
    if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
    if (it->second.swapped) return PF_ERR_SWAPPED;
    if (it->second.pages.size() > (size_t)max_blocks) return PF_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pf_seq_entry& e = pool->seqs.find(seq_ids[i])->second;
    int32_t* row = bt_host + (size_t)i * (size_t)max_blocks;
    const size_t np = e.pages.size();
    if (np) std::memcpy(row, e.pages.data(), np * sizeof(int32_t));
    for (size_t j = np; j < (size_t)max_blocks; ++j) row[j] = -1;
    if (lens_host) lens_host[i] = e.len;
  }
  return PF_OK;
}

}  // extern "C"

static void export_forget_locked(const pf_pool* pool) {
  pool->shadow.target = nullptr;
  pool->shadow.max_blocks = -1;
}

void pf_export_forget(const pf_pool* pool) {
  std::lock_guard<std::mutex> lk(pool->mu);
  export_forget_locked(pool);
}

int pf_fill_export(const pf_pool* pool, const void* target, const uint64_t* seq_ids, int32_t n,
                   int32_t max_blocks, bool step, int32_t* out, int64_t* pairs) {
  return guarded([&]() -> int {
    if (!pool || !pairs || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !out))) return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    std::vector<const pf_seq_entry*> rows((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
      auto it = pool->seqs.find(seq_ids[i]);
      if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
      if (it->second.swapped) return PF_ERR_SWAPPED;
      if (it->second.pages.size() > (size_t)max_blocks) return PF_ERR_INVALID;
      rows[(size_t)i] = &it->second;
    }
    const size_t nb = (size_t)n * (size_t)max_blocks;
    int32_t* lens = out + nb;
    int32_t* newest = lens + n;
    const int32_t B = pool->g.block_size;
    for (int32_t i = 0; i < n; ++i) {
      const pf_seq_entry& e = *rows[(size_t)i];
      lens[i] = e.len;
      newest[i] = e.len - 1;
      if (step) newest[n + i] = e.len > 0 ? e.pages[(size_t)((e.len - 1) / B)] : -1;
    }
    pf_export_shadow& sh = pool->shadow;
    bool delta = pool->export_delta && sh.target == target && target != nullptr && sh.max_blocks == max_blocks &&
                 sh.ids.size() == (size_t)n && std::equal(sh.ids.begin(), sh.ids.end(), seq_ids);
    if (delta) {
      const int64_t cap = (int64_t)nb / 2;
      int64_t k = 0;
      for (int32_t i = 0; i < n && delta; ++i) {
        const pf_seq_entry& e = *rows[(size_t)i];
        if (e.ver == sh.ver[(size_t)i]) continue;
        const int32_t np = (int32_t)e.pages.size();
        const int32_t hi = np > sh.used[(size_t)i] ? np : sh.used[(size_t)i];
        int32_t* old = sh.table.data() + (size_t)i * (size_t)max_blocks;
        for (int32_t j = 0; j < hi; ++j) {
          const int32_t cur = j < np ? e.pages[(size_t)j] : -1;
          if (cur == old[j]) continue;
          if (k == cap) {  // more changes than the staging holds as pairs: export whole
            delta = false;
            break;
          }
          out[2 * k] = i * max_blocks + j;
          out[2 * k + 1] = cur;
          old[j] = cur;
          ++k;
        }
        sh.ver[(size_t)i] = e.ver;
        sh.used[(size_t)i] = np;
      }
      if (delta) {
        *pairs = k;
        return PF_OK;
      }
    }
    for (int32_t i = 0; i < n; ++i) {
      const pf_seq_entry& e = *rows[(size_t)i];
      int32_t* row = out + (size_t)i * (size_t)max_blocks;
      const size_t np = e.pages.size();
      if (np) std::memcpy(row, e.pages.data(), np * sizeof(int32_t));
      for (size_t j = np; j < (size_t)max_blocks; ++j) row[j] = -1;
    }
    *pairs = -1;
    if (pool->export_delta && target != nullptr) {
      sh.target = target;
      sh.max_blocks = max_blocks;
      sh.ids.assign(seq_ids, seq_ids + n);
      sh.ver.resize((size_t)n);
      sh.used.resize((size_t)n);
      for (int32_t i = 0; i < n; ++i) {
        sh.ver[(size_t)i] = rows[(size_t)i]->ver;
        sh.used[(size_t)i] = (int32_t)rows[(size_t)i]->pages.size();
      }
      sh.table.assign(out, out + nb);
    } else {
      export_forget_locked(pool);
    }
    return PF_OK;
  });
}

extern "C" {

int pf_export_staging(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                      const void* meta_dev, int32_t step, int32_t* staging_host, int64_t* pairs) {
  if (!pool || !pairs || n < 0 || max_blocks < 0) return PF_ERR_INVALID;
  if (n > 0 && (!staging_host || !meta_dev)) return PF_ERR_INVALID;
  *pairs = -1;
  if (n == 0) return PF_OK;
  return pf_fill_export(pool, meta_dev, seq_ids, n, max_blocks, step != 0, staging_host, pairs);
}

int pf_pool_set_option(pf_pool* pool, int32_t option, int32_t value) {
  if (!pool) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  switch (option) {
    case PF_OPT_SPLIT_TOKENS:
      if (value < 0 || (value > 0 && (value % pool->g.block_size != 0 ||
                                      value > 64 * pool->g.block_size)))
        return PF_ERR_INVALID;
      pool->split_tokens = value;
      return PF_OK;
    case PF_OPT_GQA_MFMA:
      if (value != 0 && value != 1) return PF_ERR_INVALID;
      pool->gqa_mfma = value;
      return PF_OK;
    case PF_OPT_SCHEDULE:
      if (value < 0 || value > 2) return PF_ERR_INVALID;
      pool->schedule = value;
      return PF_OK;
    case PF_OPT_WAVES_PER_CU:
      if (value < 0 || value > 64) return PF_ERR_INVALID;
      pool->waves_per_cu = value;
      return PF_OK;
    case PF_OPT_EXPORT_DELTA:
      if (value != 0 && value != 1) return PF_ERR_INVALID;
      pool->export_delta = value;
      export_forget_locked(pool);
      return PF_OK;
    default:
      return PF_ERR_INVALID;
  }
}

int pf_pool_get_option(const pf_pool* pool, int32_t option, int32_t* value) {
  if (!pool || !value) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  switch (option) {
    case PF_OPT_SPLIT_TOKENS: *value = pool->split_tokens; return PF_OK;
    case PF_OPT_GQA_MFMA: *value = pool->gqa_mfma; return PF_OK;
    case PF_OPT_SCHEDULE: *value = pool->schedule; return PF_OK;
    case PF_OPT_WAVES_PER_CU: *value = pool->waves_per_cu; return PF_OK;
    case PF_OPT_EXPORT_DELTA: *value = pool->export_delta; return PF_OK;
    default: return PF_ERR_INVALID;
  }
}

int pf_pool_set_timing_events(pf_pool* pool, void* start_event, void* stop_event) {
  if (!pool || ((start_event == nullptr) != (stop_event == nullptr))) return PF_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  pool->ev_start = start_event;
  pool->ev_stop = stop_event;
  return PF_OK;
}

const char* pf_status_string(int status) {
  switch (status) {
    case PF_OK: return "ok";
    case PF_ERR_INVALID: return "invalid argument";
    case PF_ERR_OOM: return "out of free pages (nothing changed)";
    case PF_ERR_UNKNOWN_SEQ: return "unknown sequence id";
    case PF_ERR_UNBOUND: return "no device pool bound";
    case PF_ERR_WORKSPACE: return "workspace missing or too small";
    case PF_ERR_HIP: return "HIP runtime error";
    case PF_ERR_UNSUPPORTED: return "unsupported block size or head dim";
    case PF_ERR_SHARED: return "growth would write into a page another sequence shares (use pf_grow_seqs)";
    case PF_ERR_SWAPPED: return "sequence is swapped out";
    case PF_ERR_HOST_MEMORY: return "host memory for the handle state ran out";
    case PF_ERR_SCRATCH: return "needs more workspace than the fixed device scratch holds";
    default: return "unknown status";
  }
}

}  // extern "C"

// Swapping, under the pool lock.  Blocks move between device pages and host
// slots: out, a slot per block taken in block order, then the pages released
// last block first (a page another table holds stays with it); in, a page per
// block popped in block order, then the slots returned last block first.
// Each move writes its copy pairs ((page, slot) out, (slot, page) in) to out.

// Move blocks [first, first + count) of e (all on the device) to the host.
static void move_out(pf_pool* pool, pf_seq_entry& e, int32_t first, int32_t count, int32_t* out, int32_t* k) {
  if (e.slots.empty()) e.slots.assign(e.pages.size(), -1);
  for (int32_t b = first; b < first + count; ++b) {
    const int32_t slot = pool->slot_stack.back();
    pool->slot_stack.pop_back();
    e.slots[(size_t)b] = slot;
    out[2 * *k] = e.pages[(size_t)b];
    out[2 * *k + 1] = slot;
    ++*k;
  }
  for (int32_t b = first + count; b-- > first;) {
    const int32_t page = e.pages[(size_t)b];
    if (--pool->refs[(size_t)page] == 0) pool->stack.push_back(page);
    e.pages[(size_t)b] = -1;
  }
  e.on_host += count;
  e.swapped = true;
  e.ver = ++pool->ver_clock;
}

// Move every block of e in [first, first + count) that is on the host back
// to fresh pages.
static void move_in(pf_pool* pool, pf_seq_entry& e, int32_t first, int32_t count, int32_t* out, int32_t* k) {
  for (int32_t b = first; b < first + count; ++b) {
    if (e.pages[(size_t)b] >= 0) continue;
    const int32_t page = pop_page(pool);
    out[2 * *k] = e.slots[(size_t)b];
    out[2 * *k + 1] = page;
    ++*k;
    e.pages[(size_t)b] = page;
  }
  for (int32_t b = first + count; b-- > first;) {
    if (e.slots[(size_t)b] < 0) continue;
    pool->slot_stack.push_back(e.slots[(size_t)b]);
    e.slots[(size_t)b] = -1;
    --e.on_host;
  }
  if (e.on_host == 0) e.slots.clear();
  e.swapped = e.on_host > 0;
  e.ver = ++pool->ver_clock;
}

// Whole sequences, all or nothing: out needs every block on the device, in
// brings back every block that is on the host (and needs one to be).
int pf_swap_plan(pf_pool* pool, const uint64_t* seq_ids, int32_t n, bool to_host, int32_t* out,
                 int64_t out_words, int32_t* pairs) {
  return guarded([&]() -> int {
    *pairs = 0;
    if (!pool || n < 0 || (n > 0 && (!seq_ids || !out))) return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    if (!pool->dev || !pool->host) return PF_ERR_UNBOUND;
    std::unordered_map<uint64_t, int> seen;
    size_t total = 0;
    for (int32_t i = 0; i < n; ++i)
      if (seen[seq_ids[i]]++) return PF_ERR_INVALID;
    for (int32_t i = 0; i < n; ++i) {
      auto it = pool->seqs.find(seq_ids[i]);
      if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
      if (to_host) {
        if (it->second.swapped) return PF_ERR_SWAPPED;
        total += it->second.pages.size();
      } else {
        if (!it->second.swapped) return PF_ERR_INVALID;
        total += (size_t)it->second.on_host;
      }
    }
    if (total > (to_host ? pool->slot_stack.size() : pool->stack.size())) return PF_ERR_OOM;
    if ((int64_t)total * 2 > out_words) return PF_ERR_INVALID;
    int32_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
      pf_seq_entry& e = pool->seqs.find(seq_ids[i])->second;
      const int32_t nb = (int32_t)e.pages.size();
      if (to_host) {
        move_out(pool, e, 0, nb, out, &k);
      } else {
        move_in(pool, e, 0, nb, out, &k);
      }
    }
    *pairs = k;
    return PF_OK;
  });
}

int pf_swap_blocks_plan(pf_pool* pool, uint64_t seq_id, int32_t first, int32_t count, bool to_host, int32_t* out,
                        int64_t out_words, int32_t* pairs) {
  return guarded([&]() -> int {
    *pairs = 0;
    if (!pool || !out) return PF_ERR_INVALID;
    std::lock_guard<std::mutex> lk(pool->mu);
    if (!pool->dev || !pool->host) return PF_ERR_UNBOUND;
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end()) return PF_ERR_UNKNOWN_SEQ;
    pf_seq_entry& e = it->second;
    const int64_t nb = (int64_t)e.pages.size();
    if (count < 1 || first < 0 || (int64_t)first + count > nb) return PF_ERR_INVALID;
    for (int32_t b = first; b < first + count; ++b)
      if ((e.pages[(size_t)b] >= 0) != to_host) return PF_ERR_INVALID;  // wholly on the side it leaves
    if ((size_t)count > (to_host ? pool->slot_stack.size() : pool->stack.size())) return PF_ERR_OOM;
    if ((int64_t)count * 2 > out_words) return PF_ERR_INVALID;
    int32_t k = 0;
    if (to_host) move_out(pool, e, first, count, out, &k);
    else move_in(pool, e, first, count, out, &k);
    *pairs = k;
    return PF_OK;
  });
}

extern "C" {

int pf_swap_staging(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t to_host, int32_t* staging_host,
                    int64_t staging_words, int32_t* pairs) {
  if (!pairs) return PF_ERR_INVALID;
  return pf_swap_plan(pool, seq_ids, n, to_host != 0, staging_host, staging_words, pairs);
}

int pf_swap_blocks_staging(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks, int32_t to_host,
                           int32_t* staging_host, int64_t staging_words, int32_t* pairs) {
  if (!pairs) return PF_ERR_INVALID;
  return pf_swap_blocks_plan(pool, seq_id, first_block, num_blocks, to_host != 0, staging_host, staging_words,
                             pairs);
}

}  // extern "C"
