// Internal definition of the pf_pool handle, shared by the host allocator
// (pf_host.cpp) and the kernel entry points (pf_kernels.hip).  Not part of
// the public ABI.
#pragma once

#include <cstdint>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pf.h"

struct pf_seq_entry {
  std::vector<int32_t> pages;  // block table: logical block i -> physical page, -1 while on the host
  int32_t len = 0;             // tokens held
  int32_t on_host = 0;         // blocks swapped out to the host
  bool swapped = false;        // on_host > 0, or a length-0 sequence swapped out whole: no growth,
                               // fork or export until it is swapped in
  std::vector<int32_t> slots;  // host slot of block i while it is on the host, else -1; empty if none is
  // Version of `pages`: set from the pool's clock whenever the table changes,
  // so equal versions mean an equal table (0: never held a page).
  uint64_t ver = 0;
  uint64_t batch_mark = 0;     // last batch (pool batch_epoch) that named this sequence
};

// What the device table of the previous export holds once its upload has
// run (kept only with PF_OPT_EXPORT_DELTA): the target buffer, its rows'
// sequences, the version of each row's table and the table image.
struct pf_export_shadow {
  const void* target = nullptr;
  int32_t max_blocks = -1;
  std::vector<uint64_t> ids;
  std::vector<uint64_t> ver;
  std::vector<int32_t> used;   // entries of each row that are not -1
  std::vector<int32_t> table;  // [rows][max_blocks]
};

struct pf_pool {
  pf_geometry g{};
  size_t elem_bytes = 0;
  size_t page_elems = 0;       // L * H * 2 * B * D
  // LIFO free stack of page ids; the top is the back of the vector.
  std::vector<int32_t> stack;
  // Per page: how many block tables hold it (0 = free).
  std::vector<int32_t> refs;
  // Most pages in use at once since creation or pf_pool_reset_peak.
  int32_t peak = 0;
  std::unordered_map<uint64_t, pf_seq_entry> seqs;
  mutable std::mutex mu;
  // Caller-owned device memory bound with pf_pool_bind.
  void* dev = nullptr;
  size_t dev_bytes = 0;
  // Caller-owned pinned host swap space (pf_swap_bind): num_slots page-sized
  // slots and their LIFO free stack (top at the back).
  void* host = nullptr;
  int32_t num_slots = 0;
  std::vector<int32_t> slot_stack;
  // Tuning options (pf_pool_set_option).
  int32_t split_tokens = 0;
  int32_t gqa_mfma = 1;
  int32_t schedule = 0;       // 0 automatic, 1 fixed splits, 2 balanced
  int32_t waves_per_cu = 0;   // balanced schedule: 0 = resident capacity
  // Clock of table versions (pf_seq_entry::ver).
  uint64_t ver_clock = 0;
  // Batched growth: epoch stamped into the entries a batch names (finds
  // repeated ids without a map) and the entries it resolved.
  uint64_t batch_epoch = 0;
  std::vector<pf_seq_entry*> batch_entries;
  // Incremental table export (PF_OPT_EXPORT_DELTA) and its shadow.
  int32_t export_delta = 0;
  mutable pf_export_shadow shadow;
  // Instrumentation events around the partition kernel (hipEvent_t).
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
};

size_t pf_elem_bytes(int32_t dtype);

// Staging of one table export of seq_ids to the device buffer `target`
// (host memory `out`, under the pool lock).  Lengths go to out[n*max_blocks],
// newest positions (length - 1) to out[n*max_blocks + n] and, with step, the
// pages holding the newest tokens (-1 for length 0) to out[n*max_blocks + 2n].
// The table part: with PF_OPT_EXPORT_DELTA on and the previous export made to
// the same target with the same seq_ids and max_blocks, the entries that
// differ from it as (flat index, value) pairs at out[0 .. 2 * *pairs), if at
// most n*max_blocks/2 of them; otherwise the whole [n][max_blocks] table
// (padded with -1) at out[0..] and *pairs = -1.  Same errors as
// pf_block_tables.
int pf_fill_export(const pf_pool* pool, const void* target, const uint64_t* seq_ids, int32_t n,
                   int32_t max_blocks, bool step, int32_t* out, int64_t* pairs);

// Forget the previous export (the next one is whole); takes the pool lock.
void pf_export_forget(const pf_pool* pool);

// Host half of pf_swap_out (to_host) / pf_swap_in: validate, move the
// sequences between pages and host slots, and write the copy pairs ((page,
// slot) out, (slot, page) in) into out (out_words int32).  *pairs = pairs
// written.  Same errors as the entry points.
int pf_swap_plan(pf_pool* pool, const uint64_t* seq_ids, int32_t n, bool to_host, int32_t* out,
                 int64_t out_words, int32_t* pairs);

// The same for blocks [first, first + count) of one sequence (pf_swap_out_blocks
// / pf_swap_in_blocks).
int pf_swap_blocks_plan(pf_pool* pool, uint64_t seq_id, int32_t first, int32_t count, bool to_host, int32_t* out,
                        int64_t out_words, int32_t* pairs);
