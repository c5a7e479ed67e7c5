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
// Each workgroup of four waves computes the page-count prefix of all
// sequences once, in LDS; waves then resolve their pages by binary search.
#pragma once

#include "pf_attn.h"
#include "pf_common.h"

namespace pf {

constexpr int kSchedThreads = 256;          // four waves per workgroup
constexpr int kMaxSeqsBalanced = 2048;      // sequences the LDS prefix holds
constexpr int kScanPerThread = kMaxSeqsBalanced / kSchedThreads;

struct SchedLds {
  int32_t pfx[kMaxSeqsBalanced + 1];  // pfx[s]: pages of sequences before s
  int32_t ctx[kMaxSeqsBalanced];      // lengths clamped to [0, max_ctx]
  int32_t wsum[kSchedThreads / kWave];
};

__device__ inline int clamp_ctx(int c, int max_ctx) { return c < 0 ? 0 : (c > max_ctx ? max_ctx : c); }

// All threads of the workgroup: clamped lengths and the exclusive page-count
// prefix into LDS.  Ends with a workgroup barrier.
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
      sum += (c + kBlock - 1) / kBlock;
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

}  // namespace pf
