// Thread-safety stress of libpf's host allocator, built with
// -fsanitize=thread against pf_host.cpp alone (no device code runs).
// Eight threads share one pool and work on disjoint sequence ids: grow,
// batch grow, fork, copy-on-write grow, swap planning out and in, free,
// table export (whole and incremental) and option changes.  Exit status 0 if every call returned an
// expected status and the pool came back whole; ThreadSanitizer reports any
// data race on stderr and makes the exit status non-zero.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <random>
#include <thread>
#include <vector>

#include "pf.h"
#include "pf_internal.h"

static std::atomic<int> failures{0};

static void expect(bool ok, const char* what, int st) {
  if (!ok) {
    std::fprintf(stderr, "unexpected status %d in %s\n", st, what);
    failures.fetch_add(1);
  }
}

static void worker(pf_pool* pool, int t) {
  std::mt19937 rng(1234 + t);
  const uint64_t base = (uint64_t)t * 100000;
  std::vector<uint64_t> live;
  std::vector<uint64_t> out;
  uint64_t next = base;
  std::vector<int32_t> staging(4096);
  std::vector<int32_t> copies(64);
  for (int it = 0; it < 3000; ++it) {
    const int r = (int)(rng() % 100);
    if (live.empty() || r < 15) {
      int32_t nn = 0;
      const int st = pf_alloc_for_seq(pool, next, (int32_t)(rng() % 80), &nn);
      expect(st == PF_OK || st == PF_ERR_OOM, "alloc", st);
      if (st == PF_OK) live.push_back(next);
      ++next;
    } else if (r < 25) {
      const int st = pf_fork_seq(pool, live[rng() % live.size()], next);
      expect(st == PF_OK, "fork", st);
      live.push_back(next++);
    } else if (r < 45) {
      uint64_t ids[4];
      int32_t lens[4], nn[4], nc = 0;
      const int k = 1 + (int)(rng() % 4);
      for (int i = 0; i < k; ++i) {
        ids[i] = live[rng() % live.size()];
        int32_t len = 0;
        pf_seq_len(pool, ids[i], &len);
        lens[i] = len + 20 * (i + 1);  // a repeated id never asks for less than an earlier entry
      }
      const int st = pf_grow_seqs(pool, ids, lens, k, nn, copies.data(), &nc);
      expect(st == PF_OK || st == PF_ERR_OOM, "grow", st);
    } else if (r < 55) {
      uint64_t id = live[rng() % live.size()];
      int32_t len = 0;
      pf_seq_len(pool, id, &len);
      const int32_t nl = len + (int32_t)(rng() % 5);
      int32_t nn = 0;
      const int st = pf_alloc_for_seqs(pool, &id, &nl, 1, &nn);
      expect(st == PF_OK || st == PF_ERR_OOM || st == PF_ERR_SHARED, "batch alloc", st);
    } else if (r < 65) {
      const size_t i = rng() % live.size();
      uint64_t id = live[i];
      int32_t pairs = 0;
      const int st = pf_swap_plan(pool, &id, 1, true, staging.data(), (int64_t)staging.size(), &pairs);
      expect(st == PF_OK || st == PF_ERR_OOM, "swap out", st);
      if (st == PF_OK) {
        out.push_back(id);
        live.erase(live.begin() + (long)i);
      }
    } else if (r < 72 && !out.empty()) {
      const size_t i = rng() % out.size();
      uint64_t id = out[i];
      int32_t pairs = 0;
      const int st = pf_swap_plan(pool, &id, 1, false, staging.data(), (int64_t)staging.size(), &pairs);
      expect(st == PF_OK || st == PF_ERR_OOM, "swap in", st);
      if (st == PF_OK) {
        live.push_back(id);
        out.erase(out.begin() + (long)i);
      }
    } else if (r < 80) {
      std::vector<int32_t> bt(64 * live.size()), lens(live.size());
      const int st = pf_block_tables(pool, live.data(), (int32_t)live.size(), 64, bt.data(), lens.data());
      expect(st == PF_OK || st == PF_ERR_INVALID, "tables", st);
      pf_free_pages(pool);
      pf_num_seqs(pool);
      pf_swap_free_slots(pool);
      pf_page_refcount(pool, (int32_t)(rng() % 400));
      int32_t v = 0;
      pf_pool_set_option(pool, PF_OPT_WAVES_PER_CU, (int32_t)(rng() % 9));
      pf_pool_get_option(pool, PF_OPT_WAVES_PER_CU, &v);
      // incremental export: the shared shadow of the previous export, two
      // fake targets per thread (never dereferenced), delta switched on and
      // off by any thread
      std::vector<int32_t> stage(67 * live.size() + 1);
      int64_t pairs = 0;
      const void* target = reinterpret_cast<const void*>((uintptr_t(t) * 2 + 1 + rng() % 2) << 12);
      const int se = pf_export_staging(pool, live.data(), (int32_t)live.size(), 64, target, (int32_t)(rng() % 2),
                                       stage.data(), &pairs);
      expect(se == PF_OK || se == PF_ERR_INVALID, "export staging", se);
      if (rng() % 16 == 0) pf_pool_set_option(pool, PF_OPT_EXPORT_DELTA, (int32_t)(rng() % 2));
    } else {
      const size_t i = rng() % live.size();
      const int st = pf_free_seq(pool, live[i]);
      expect(st == PF_OK, "free", st);
      live.erase(live.begin() + (long)i);
    }
  }
  for (uint64_t id : live) expect(pf_free_seq(pool, id) == PF_OK, "final free", -1);
  for (uint64_t id : out) expect(pf_free_seq(pool, id) == PF_OK, "final free swapped", -1);
}

int main() {
  pf_geometry g{400, 16, 1, 1, 16, PF_F16};
  pf_pool* pool = nullptr;
  if (pf_pool_create(&g, nullptr, &pool) != PF_OK) return 2;
  // fake, never dereferenced, aligned addresses: only the host bookkeeping runs
  pf_pool_bind(pool, reinterpret_cast<void*>(uintptr_t(1) << 40), pf_pool_bytes(pool));
  pf_swap_bind(pool, reinterpret_cast<void*>(uintptr_t(1) << 41), 300 * pf_page_bytes(pool), 300);
  std::vector<std::thread> th;
  for (int t = 0; t < 8; ++t) th.emplace_back(worker, pool, t);
  for (auto& x : th) x.join();
  const int whole = pf_free_pages(pool) == 400 && pf_swap_free_slots(pool) == 300 && pf_num_seqs(pool) == 0;
  for (int p = 0; p < 400; ++p)
    if (pf_page_refcount(pool, p) != 0) failures.fetch_add(1);
  pf_pool_destroy(pool);
  std::printf("failures %d, pool whole %d\n", failures.load(), whole);
  return failures.load() == 0 && whole ? 0 : 1;
}
