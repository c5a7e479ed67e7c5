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

#include "pf_attn.h"
#include "pf_common.h"

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

// All threads of the workgroup: clamped lengths and the exclusive page-count
// prefix into LDS.  Ends with a workgroup barrier.
template <int UT = kBlock>
__device__ inline void sched_build(const AttnArgs& a, SchedLds& L) {
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
        c = clamp_ctx(a.ctx[s], a.max_ctx);
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
__device__ inline void sched_run(const AttnArgs& a, const SchedLds& L, int X, Wv& w, int lane) {
  constexpr int UT = Wv::UT;
  using Tile = typename Wv::Tile;
  const int gw = blockIdx.x * (kSchedThreads / kWave) + threadIdx.x / kWave;
  const int64_t total = (int64_t)X * L.pfx[a.n];
  if (total == 0) return;
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
  for (int64_t base = wa; base < wb; base += kWave) {
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
    page_pipeline<U, Tile>(
        cnt,
        [&](int i, Tile& t) {
          if constexpr (Wv::kPPU == 2)
            return w.load2(__builtin_amdgcn_readlane(lpage, i), __builtin_amdgcn_readlane(lpage2, i),
                           __builtin_amdgcn_readlane(ls, i), __builtin_amdgcn_readlane(lx, i), t);
          else
            return w.load(__builtin_amdgcn_readlane(lpage, i), __builtin_amdgcn_readlane(ls, i),
                          __builtin_amdgcn_readlane(lp, i), __builtin_amdgcn_readlane(lx, i), t);
        },
        [&](int i, Tile& t, bool ok) {
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
            const uint64_t nxt =
                __builtin_amdgcn_ballot_w64(lane > i && lane < cnt && ls * X + lx != cur);
            if (nxt) {
              const int j = __builtin_ctzll(nxt);
              const int s2 = __builtin_amdgcn_readlane(ls, j), x2 = __builtin_amdgcn_readlane(lx, j);
              w.prefetch(s2, x2, s2 * X + x2);
            }
          }
          cplast = p;
          if (p == cP - 1)
            w.patch_last(t, __builtin_amdgcn_readlane(lnv, i), s, x, __builtin_amdgcn_readlane(lpage, i), ok, p);
          if (ok) w.page(t, __builtin_amdgcn_readlane(lnv, i));
        });
  }
  if (cur >= 0) close_piece();
}

}  // namespace pf
