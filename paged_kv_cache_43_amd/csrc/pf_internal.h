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
  std::vector<int32_t> pages;  // block table: logical block i -> physical page
  int32_t len = 0;             // tokens held
  bool swapped = false;        // swapped out: pages empty, slots hold the blocks
  std::vector<int32_t> slots;  // host swap slots of logical blocks 0.. (swapped only)
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
  // Instrumentation events around the partition kernel (hipEvent_t).
  void* ev_start = nullptr;
  void* ev_stop = nullptr;
};

size_t pf_elem_bytes(int32_t dtype);

// Fill [n][max_blocks] tables, [n] lengths and [n] newest positions into
// out (host memory) under the pool lock.  Same errors as pf_block_tables.
int pf_fill_meta(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks, int32_t* out);

// As pf_fill_meta, followed by [n] pages holding each sequence's newest token
// (-1 for length 0).
int pf_fill_meta_step(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks, int32_t* out);

// Host half of pf_swap_out (to_host) / pf_swap_in: validate, move the
// sequences between pages and host slots, and write the copy pairs ((page,
// slot) out, (slot, page) in) into out (out_words int32).  *pairs = pairs
// written.  Same errors as the entry points.
int pf_swap_plan(pf_pool* pool, const uint64_t* seq_ids, int32_t n, bool to_host, int32_t* out,
                 int64_t out_words, int32_t* pairs);
