// Work schedules of the attention partition kernels.
//
// Grid schedule: one wave per (sequence, head, fixed context split).
//
// Balanced schedule: the context pages of every (sequence, item) -- an item is
// a query head for the vector kernel or a kv head group for the matrix-core
// kernel -- are laid end to end in (sequence, item, page) order, and each of
// W waves takes an equal slice of that stream.  A slice may start or end
// inside an item and may cover several items; each covered part of an item
// (a "piece") gives either the item's final output (the piece is the whole
// item) or a partial (max, sum, accumulator) record.  The piece of item i held
// by wave w goes to record i + w: items are contiguous in the stream, so these
// slots never collide, and there are at most items + W of them.  The wave that
// holds an item's last page also writes the item's (first record, pieces)
// pair for the merge kernel.  Slices depend only on the lengths, so the work
// split, and with it every rounding, is the same for any physical page order.
//
// On MI355X waves given equal slices finish far apart (the slowest XCD's
// about a quarter of the kernel time after the average), but handing out the
// stream at run time does not shorten the kernel: claiming finer chunks from
// counters (one global counter, one per 32-wave group, or one per workgroup in
// LDS) was measured equal or slower, since the kernel is bound by the chip's
// total HBM throughput and extra chunks add pieces and partial records.
//
// Each workgroup of four waves computes the page-count prefix of all
// sequences once, in LDS; waves then resolve their pages by binary search.
#pragma once

#include <type_traits>

#include "pf_attn.h"
#include "pf_common.h"
#include "pf_internal.h"

namespace pf {

constexpr int kSchedThreads = 256;          // four waves per workgroup
constexpr int kMaxSeqsBalanced = 2048;      // sequences the LDS prefix holds
// Contexts up to this many tokens are attended one wave per whole (sequence,
// head) with no split and no merge launch: on MI355X that beat the balanced
// schedule plus its merge on short contexts (GPT-2 shape, contexts <= 190:
// 9.7 vs 16.0 us per layer; 4 sequences of <= 64 tokens: 7.2 vs 15.2 us),
// while from a few hundred tokens on the balanced schedule is faster.
constexpr int kWholeItemTokens = 256;
constexpr int kScanPerThread = kMaxSeqsBalanced / kSchedThreads;

struct SchedLds {
  int32_t pfx[kMaxSeqsBalanced + 1];  // pfx[s]: pages of sequences before s
  int32_t ctx[kMaxSeqsBalanced];      // lengths clamped to [0, max_ctx]
  int32_t wsum[kSchedThreads / kWave];
};

__device__ inline int clamp_ctx(int c, int max_ctx) { return c < 0 ? 0 : (c > max_ctx ? max_ctx : c); }

// The lengths of the sequences this thread scans, loaded into registers
// (sched_load), then clamped and scanned (sched_scan): split so that other
// loads (a plan's first pages) can be issued while these are in flight.
struct SchedCtx {
  int c[kScanPerThread];
};

// Every load is issued, with indexes clamped into [0, n), and no branch: the
// compiler's memory-counter waits then stay exact for loads issued after
// these (a wait for a load issued in a branch waits for everything).  Values
// of sequences this thread does not scan are not used.
__device__ inline SchedCtx sched_load(const AttnArgs& a) {
  const int t = threadIdx.x;
  const int k_per = (a.n + kSchedThreads - 1) / kSchedThreads;  // <= kScanPerThread
  SchedCtx r;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) r.c[k] = a.ctx[min(t * k_per + k, a.n - 1)];
  return r;
}

// All threads of the workgroup: clamped lengths and the exclusive page-count
// prefix into LDS.  Ends with a workgroup barrier.
template <int UT = kBlock>
__device__ inline void sched_scan(const AttnArgs& a, SchedLds& L, const SchedCtx& cx) {
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int w = t / kWave;
  const int k_per = (a.n + kSchedThreads - 1) / kSchedThreads;  // <= kScanPerThread
  int incl[kScanPerThread];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    incl[k] = sum;
    if (k < k_per) {
      const int s = t * k_per + k;
      int c = 0;
      if (s < a.n) {
        c = clamp_ctx(cx.c[k], a.max_ctx);
        L.ctx[s] = c;
      }
      sum += (c + UT - 1) / UT;
      incl[k] = sum;
    }
  }
  int v = sum;  // inclusive scan across the wave
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  if (lane == kWave - 1) L.wsum[w] = v;
  __syncthreads();
  int off = v - sum;
  for (int j = 0; j < w; ++j) off += L.wsum[j];
#pragma unroll
  for (int k = 0; k < kScanPerThread; ++k) {
    const int s = t * k_per + k;
    if (k < k_per && s < a.n) L.pfx[s + 1] = off + incl[k];
  }
  if (t == 0) L.pfx[0] = 0;
  __syncthreads();
}

template <int UT = kBlock>
__device__ inline void sched_build(const AttnArgs& a, SchedLds& L) {
  sched_scan<UT>(a, L, sched_load(a));
}

// A plan of the balanced schedule, written by the host for one attention
// configuration next to the step's tables: a header {magic, items per
// sequence, waves, tokens per unit, sequences, length bound, total units
// (low, high word)} and, per wave, {page of its first unit, page of its second
// unit, key of the first, key of the second, unit index of the first, of the
// second, 0, 0}, a unit's key being item | unit-in-page << 16 | sequence << 18
// and its unit index its position in the item.  A wave reads its entry at
// launch and issues the loads of those two units and the first item's q at
// once, while the lengths are still being loaded and scanned; after the scan
// it checks both units against its own search and uses the loads only if
// they agree (the plan only moves loads earlier: results are the same bits).

struct PlanHead {
  uint4 h;     // lane 0: header words 0..3, lane 1: words 4..7 (broadcast when used)
  uint4 d, e;  // this wave's entry
};

// The header is read by lanes 0 and 1 with a per-lane load: a load of a
// uniform address would become a scalar load, whose wait (a single counter
// for every scalar load) would also hold back the length loads that follow.
__device__ inline PlanHead plan_read(const AttnArgs& a, int gw) {
  const uint4* p = reinterpret_cast<const uint4*>(a.plan);
  PlanHead r;
  r.h = p[threadIdx.x & 1];
  r.d = p[(kPlanHeaderWords + kPlanWaveWords * gw) / 4];
  r.e = p[(kPlanHeaderWords + kPlanWaveWords * gw) / 4 + 1];
  return r;
}

// The pre-issued first two units of a wave's slice.
template <class Tile>
struct PlanPre {
  Tile t[2];
  bool ok[2];
  int key[2];   // item | unit-in-page << 16 | sequence << 18, as the plan gave them
  int unit[2];  // unit index in the item, as the plan gave them
  int64_t total;
};

__device__ inline int plan_key(int s, int x, int r) { return x | (r << 16) | (s << 18); }

// Check the header against this launch, issue the loads of the wave's first
// two units (w.load(page, s, p, item, tile) with p = the unit-in-page: only
// that part of p addresses a pool page) and prefetch the first item's q.
// False (nothing issued) if the plan belongs to another configuration or the
// wave has no units.
// The loads are issued whatever the outcome, with no branch (a plan that
// does not match reads page 0 and sequence 0's q, in bounds, and is not
// used), so that the waits for the length loads issued before them stay
// exact instead of waiting for these too.
template <class Wv>
__device__ inline bool plan_start(const AttnArgs& a, const PlanHead& ph, int X, Wv& w,
                                  PlanPre<typename Wv::Tile>& pre) {
  const uint4 h0 = make_uint4(__builtin_amdgcn_readlane(ph.h.x, 0), __builtin_amdgcn_readlane(ph.h.y, 0),
                              __builtin_amdgcn_readlane(ph.h.z, 0), __builtin_amdgcn_readlane(ph.h.w, 0));
  const uint4 h1 = make_uint4(__builtin_amdgcn_readlane(ph.h.x, 1), __builtin_amdgcn_readlane(ph.h.y, 1),
                              __builtin_amdgcn_readlane(ph.h.z, 1), __builtin_amdgcn_readlane(ph.h.w, 1));
  const int k0 = (int)ph.d.z, k1 = (int)ph.d.w;
  const int s0 = (int)((unsigned)k0 >> 18), x0 = k0 & 0xffff;
  const int s1 = (int)((unsigned)k1 >> 18), x1 = k1 & 0xffff;
  // bitwise & throughout: a short-circuit chain made the compiler load the
  // header words one test at a time, a memory round trip per test
  const bool ok = ((int)h0.x == kPlanMagic) & ((int)h0.y == X) & ((int)h0.z == a.waves) &
                  ((int)h0.w == Wv::UT) & ((int)h1.x == a.n) & ((int)h1.y == a.max_ctx) &
                  ((int)ph.d.x >= 0) & (s0 < a.n) & (x0 < X) & (s1 < a.n) & (x1 < X);
  pre.total = (int64_t)h1.z | ((int64_t)h1.w << 32);
  pre.key[0] = k0;
  pre.key[1] = k1;
  pre.unit[0] = (int)ph.e.x;
  pre.unit[1] = (int)ph.e.y;
  const int ss = ok ? s0 : 0;
  pre.ok[0] = w.load(ok ? (int)ph.d.x : -1, ss, (k0 >> 16) & 3, ok ? x0 : 0, pre.t[0]);
  pre.ok[1] = w.load(ok ? (int)ph.d.y : -1, ss, (k1 >> 16) & 3, ok ? x1 : 0, pre.t[1]);
  w.prefetch(ss, ok ? x0 : 0, ok ? (int64_t)s0 * X + x0 : -1);
  return ok;
}

// Where flat page f of the stream lives: sequence s, item x, page p of the
// item, the item's page count P.  Needs 0 <= f < X * pfx[n].
struct PagePos {
  int s, x, p, P;
};

__device__ inline PagePos sched_locate(const SchedLds& L, int n, int X, int64_t f) {
  int lo = 0, hi = n;  // X*pfx[lo] <= f < X*pfx[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)X * L.pfx[mid] <= f) lo = mid;
    else hi = mid;
  }
  PagePos r;
  r.s = lo;
  r.P = L.pfx[lo + 1] - L.pfx[lo];
  const int64_t rem = f - (int64_t)X * L.pfx[lo];
  r.x = (int)(rem / r.P);
  r.p = (int)(rem - (int64_t)r.x * r.P);
  return r;
}

// The balanced schedule's driver, shared by both kernels.  Wv provides
// begin(s, x), load(page, s, p, x, tile) -> bool, page(tile, nvalid),
// finish_slot(s, x, whole, slot) and kContig (no table).
// The balanced schedule's driver, shared by both kernels: this wave's slice
// of the stream, piece by piece.  The stream is counted in units of Wv::UT
// tokens (the prefix in L must be built with the same UT); a unit is part of
// one page (Wv::kUPP units per page) or, for pages shorter than a unit, spans
// Wv::kPPU = 2 pages.  Wv provides begin(s, x), load(page, s, p, x, tile) ->
// bool (load2(page0, page1, s, x, tile) for two pages per unit),
// page(tile, nvalid), finish_slot(s, x, whole, slot) and kContig (blocks
// addressed without a table).
template <int U, int BS, class Wv>
__device__ __forceinline__ void sched_run(const AttnArgs& a, const SchedLds& L, int X, Wv& w, int lane,
                                 PlanPre<typename Wv::Tile>& pre, bool planned) {
  constexpr int UT = Wv::UT;
  using Tile = typename Wv::Tile;
  const int gw = blockIdx.x * (kSchedThreads / kWave) + threadIdx.x / kWave;
  const int64_t total = (int64_t)X * L.pfx[a.n];
  if (total == 0) return;
  planned = planned && pre.total == total;
  const int64_t chunk = (total + a.waves - 1) / a.waves;
  const int64_t wa = (int64_t)gw * chunk;
  const int64_t wb = min(wa + chunk, total);
  if (wa >= wb) return;
  int cur = -1, cs = 0, cx = 0, cP = 0, cp0 = 0, cplast = 0;
  auto close_piece = [&]() {
    const bool first = cp0 == 0, last = cplast == cP - 1;
    const int item = cs * X + cx;
    w.finish_slot(cs, cx, first && last, (int64_t)item + gw);
    if (last && lane == 0) {
      const int64_t start = (int64_t)X * L.pfx[cs] + (int64_t)cx * cP;
      const int wf = (int)(start / chunk), wl = (int)((start + cP - 1) / chunk);
      a.ws_meta[item] = make_int2(item + wf, wl - wf + 1);
    }
  };
  // One batch of up to 64 units: positions and table entries into lanes, then
  // the page pipeline.  FIRST: the wave's first batch with a plan, which
  // starts from the plan's two pre-issued units if they are the ones this
  // search found; it is peeled off the loop so that the pre-issued tiles are
  // not live in the steady state.
  auto batch = [&](int64_t base, auto first) {
    const int cnt = (int)min((int64_t)kWave, wb - base);
    int ls = 0, lx = 0, lp = 0, lP = 1, lpage = -1, lpage2 = -1, lnv = 0;
    if (lane < cnt) {
      const PagePos pp = sched_locate(L, a.n, X, base + lane);
      ls = pp.s;
      lx = pp.x;
      lp = pp.p;
      lP = pp.P;
      if constexpr (!Wv::kContig) {
        const int64_t row = (int64_t)pp.s * a.max_blocks;
        if constexpr (Wv::kPPU == 2) {
          lpage = a.bt[row + 2 * pp.p];
          if (2 * pp.p + 1 < (L.ctx[pp.s] + BS - 1) / BS) lpage2 = a.bt[row + 2 * pp.p + 1];
        } else {
          lpage = a.bt[row + pp.p / Wv::kUPP];
        }
      }
      lnv = min(UT, L.ctx[pp.s] - pp.p * UT);
    }
    auto load = [&](int i, Tile& t) {
      if constexpr (Wv::kPPU == 2)
        return w.load2(__builtin_amdgcn_readlane(lpage, i), __builtin_amdgcn_readlane(lpage2, i),
                       __builtin_amdgcn_readlane(ls, i), __builtin_amdgcn_readlane(lx, i), t);
      else
        return w.load(__builtin_amdgcn_readlane(lpage, i), __builtin_amdgcn_readlane(ls, i),
                      __builtin_amdgcn_readlane(lp, i), __builtin_amdgcn_readlane(lx, i), t);
    };
    auto proc = [&](int i, Tile& t, bool ok) {
      const int s = __builtin_amdgcn_readlane(ls, i);
      const int x = __builtin_amdgcn_readlane(lx, i);
      const int p = __builtin_amdgcn_readlane(lp, i);
      if (s * X + x != cur) {
        if (cur >= 0) close_piece();
        cur = s * X + x;
        cs = s;
        cx = x;
        cP = __builtin_amdgcn_readlane(lP, i);
        cp0 = p;
        w.begin(s, x, cur);
        // the next item of this batch, if any: load its q now
        const uint64_t nxt = __builtin_amdgcn_ballot_w64(lane > i && lane < cnt && ls * X + lx != cur);
        if (nxt) {
          const int j = __builtin_ctzll(nxt);
          const int s2 = __builtin_amdgcn_readlane(ls, j), x2 = __builtin_amdgcn_readlane(lx, j);
          w.prefetch(s2, x2, s2 * X + x2);
        }
      }
      cplast = p;
      if (p == cP - 1 && w.appends())
        w.patch_last(t, __builtin_amdgcn_readlane(lnv, i), s, x, __builtin_amdgcn_readlane(lpage, i), ok);
      if (ok) w.page(t, __builtin_amdgcn_readlane(lnv, i));
    };
    if constexpr (decltype(first)::value) {
      const int k0 = plan_key(__builtin_amdgcn_readlane(ls, 0), __builtin_amdgcn_readlane(lx, 0),
                              __builtin_amdgcn_readlane(lp, 0) % Wv::kUPP);
      const int k1 = plan_key(__builtin_amdgcn_readlane(ls, 1), __builtin_amdgcn_readlane(lx, 1),
                              __builtin_amdgcn_readlane(lp, 1) % Wv::kUPP);
      // Not the units this search found: load the right ones into the same
      // tiles (one pipeline either way: a second one beside the pre-issued
      // tiles costs registers the steady state then lacks).
      const bool same0 = k0 == pre.key[0] && __builtin_amdgcn_readlane(lp, 0) == pre.unit[0];
      const bool same1 = cnt < 2 || (k1 == pre.key[1] && __builtin_amdgcn_readlane(lp, 1) == pre.unit[1]);
      if (!(same0 && same1)) {
        pre.ok[0] = load(0, pre.t[0]);
        pre.ok[1] = load(cnt > 1 ? 1 : 0, pre.t[1]);
      }
      page_pipeline_pre<U, Tile>(cnt, pre.t, pre.ok, load, proc);
    } else {
      page_pipeline<U, Tile>(cnt, load, proc);
    }
  };
  int64_t base = wa;
  if constexpr (Wv::kPPU == 1 && U <= 2) {
    if (planned) {
      batch(base, std::true_type{});
      base += kWave;
    }
  }
  for (; base < wb; base += kWave) batch(base, std::false_type{});
  if (cur >= 0) close_piece();
}

}  // namespace pf
