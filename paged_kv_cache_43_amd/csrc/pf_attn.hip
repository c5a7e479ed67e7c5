// Decode attention over paged K/V: the vector partition kernel, the split
// merge kernel and the pf_paged_decode_attention entry point.
//
// What is computed (PagedAttention blog, "The Attention Kernel"; PageFault,
// "Four stages", stage 3): for sequence s and query head h,
//   out = softmax(scale * K q) V  over the first ctx[s] tokens,
// where every K/V row is found through the sequence's block table.  The blog's
// kernel keeps a running max and sum while it walks the blocks (online
// softmax) and merges partial results across thread blocks with log-sum-exp;
// both are used here, in fp32.
//
// Vector kernel (any head grouping, all dtypes), per wave:
//  * Lanes lie across the head dimension: each lane holds VEC consecutive
//    elements (a 16-byte load), D/VEC lanes cover one token, and one wave
//    instruction loads 64/(D/VEC) consecutive tokens of a page.  The K and V
//    tiles of a (page, layer, kv head) are adjacent in the pool, so a page is
//    read as 2*B*D*es contiguous bytes.
//  * Table entries are loaded once per batch of pages into lanes and broadcast
//    per page with readlane: there is no dependent load chain per page; the
//    next page's loads are issued before the current page is used.
//  * QK partial dots are summed across the D/VEC lanes of a token with DPP
//    moves; the page maximum is a wave-wide reduction; the running max is
//    therefore wave-uniform, so each lane accumulates p*v for its own tokens
//    and the per-lane accumulators are combined once per piece.
//  * Only a sequence's last page can hold tokens past the length; those get
//    score -inf and value 0 by select, never by multiplication, so sentinel
//    NaNs in the tail never reach the result.
//  * Scores are kept in log2 units: q is pre-multiplied by scale*log2(e) and
//    exponentials are exp2.
// Work is assigned by the balanced schedule (pf_sched.h) or by fixed context
// splits; both end with the same merge.
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "pf_attn.h"
#include "pf_common.h"
#include "pf_internal.h"
#include "pf_sched.h"

namespace pf {

// UT: tokens per unit of the page walk (16, or 8 for 8-token pages).
template <class T, int D, int UT = kBlock>
struct ValuShape {
  static constexpr int ES = T::es;
  static constexpr int VEC0 = 16 / ES;
  static constexpr int VEC = VEC0 < D * UT / kWave ? VEC0 : D * UT / kWave;  // elements per lane
  static constexpr int LPT = D / VEC;             // lanes per token
  static constexpr int TPI = kWave / LPT;         // tokens per wave instruction
  static constexpr int ROWS = UT / TPI;           // instructions per K (or V) unit
  static constexpr int NW = VEC * ES / 4;         // 32-bit words per lane per row
  static_assert(LPT >= 1 && LPT <= kWave && TPI <= UT && ROWS * TPI == UT, "shape");
  static_assert(NW == 1 || NW == 2 || NW == 4, "load width");
};

template <class T, int NW>
__device__ inline void widen_words(const Raw<NW>& r, float* out) {
#pragma unroll
  for (int w = 0; w < NW; ++w) T::widen(r.w[w], out + w * T::per_word);
}

template <class T, bool OUT_F32>
__device__ inline void store_out(void* out, int64_t idx, float v) {
  if constexpr (OUT_F32) {
    static_cast<float*>(out)[idx] = v;
  } else if constexpr (T::es == 4) {
    static_cast<float*>(out)[idx] = v;
  } else {
    static_cast<uint16_t*>(out)[idx] = (uint16_t)T::narrow_bits(v);
  }
}

// Zero outputs of every sequence with length 0 (balanced schedule: the
// workgroup-0 threads do it from the LDS lengths, one thread per sequence, so
// the common case costs one LDS read per thread).
template <class T, bool OUT_F32>
__device__ inline void zero_empty_rows(const AttnArgs& a, const SchedLds& L, int D) {
  if (blockIdx.x != 0) return;
  const int64_t row_elems = (int64_t)a.hq * D;
  for (int s = threadIdx.x; s < a.n; s += kSchedThreads) {  // one thread per sequence
    if (L.ctx[s] != 0) continue;
    for (int64_t e = 0; e < row_elems; ++e) store_out<T, OUT_F32>(a.out, s * row_elems + e, 0.f);
  }
}

// Per-wave state of the vector kernel: the current piece's online softmax.
// CONTIG: blocks come from a contiguous cache instead of pool pages.  BS: the
// pool's tokens per page.  UTO: unit size override (BlockUnits).
template <class T, int D, bool OUT_F32, bool CONTIG, int BS = kBlock, int UTO = 0>
struct ValuWave {
  static constexpr int UT = BlockUnits<BS, UTO>::UT;  // tokens per unit of the walk
  static constexpr int kPPU = 1;                        // pages per unit
  static constexpr int kUPP = BlockUnits<BS, UTO>::R;   // units per page
  using S = ValuShape<T, D, UT>;
  struct Tile {
    Raw<S::NW> k[S::ROWS], v[S::ROWS];
  };
  const AttnArgs& a;
  const int lane, dc, tq;
  float qf[S::VEC];
  Raw<S::NW> qnx;  // the next item's q bits, loaded ahead (prefetch)
  int64_t qn_key = -1;
  float m, l, acc[S::VEC];

  static constexpr bool kContig = CONTIG;

  __device__ ValuWave(const AttnArgs& args, int ln) : a(args), lane(ln), dc(ln % S::LPT), tq(ln / S::LPT) {}

  __device__ inline Raw<S::NW> load_q(int s, int h) const {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + ((((int64_t)s * a.hq + h) * D) + dc * S::VEC) * S::ES;
    return load_raw<S::NW>(qp);
  }

  // Issue the q load of the item that follows in this wave's stream, so that
  // its begin() does not wait behind the page loads in flight (see the
  // matrix-core kernel).  key = s * items + h.
  __device__ inline void prefetch(int s, int h, int64_t key) {
    qnx = load_q(s, h);
    qn_key = key;
  }

  // Start a piece of (sequence s, query head h), item key (or -1): q in log2
  // units, empty state.
  __device__ inline void begin(int s, int h, int64_t key = -1) {
    const Raw<S::NW> r = key >= 0 && key == qn_key ? qnx : load_q(s, h);
    widen_words<T, S::NW>(r, qf);
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) qf[i] *= a.qscale;
    // Pin q in registers here (see the matrix-core kernel's begin): it must
    // neither be re-loaded per page nor stay pending where the item-switch
    // branch rejoins the page loop.
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) asm volatile("" : "+v"(qf[i]));
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) acc[i] = 0.f;
  }

  // Issue the K and V loads of block p of sequence s (pool page `page`) for
  // query head h; false if the table entry is not a valid page (page 0 is
  // read instead, in bounds).
  __device__ inline bool load(int page, int s, int p, int h, Tile& t) const {
    const BlockAddr b = block_addr<CONTIG, D, S::ES, BS, UTO>(a, page, s, p, h / a.group);
    const int64_t lo = (int64_t)tq * b.tok + dc * S::VEC * S::ES;
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) t.k[r] = load_raw<S::NW>(b.k + lo + r * S::TPI * b.tok);
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) t.v[r] = load_raw<S::NW>(b.v + lo + r * S::TPI * b.tok);
    return b.ok;
  }

  // One unit: nvalid of its UT tokens are below the length.
  __device__ inline void page(const Tile& t, int nvalid) {
    float sc[S::ROWS];
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) {
      float kf[S::VEC];
      widen_words<T, S::NW>(t.k[r], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < S::VEC; ++e) d = fmaf(qf[e], kf[e], d);
      sc[r] = group_reduce<S::LPT, OpSum>(d);
    }
    const bool full = nvalid >= UT;
    if (!full) {
#pragma unroll
      for (int r = 0; r < S::ROWS; ++r)
        if (r * S::TPI + tq >= nvalid) sc[r] = -INFINITY;
    }
    float pm = sc[0];
#pragma unroll
    for (int r = 1; r < S::ROWS; ++r) pm = fmaxf(pm, sc[r]);
    pm = strided_reduce<S::LPT, OpMax>(pm);
    const float mn = fmaxf(m, pm);  // finite: the page holds at least one token
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < S::VEC; ++e) acc[e] *= alpha;
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) {
      const float p = fast_exp2(sc[r] - mn);
      float vf[S::VEC];
      widen_words<T, S::NW>(t.v[r], vf);
      if (!full && r * S::TPI + tq >= nvalid) {
#pragma unroll
        for (int e = 0; e < S::VEC; ++e) vf[e] = 0.f;
      }
      l += p;
#pragma unroll
      for (int e = 0; e < S::VEC; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    }
  }

  // Before page() of the sequence's last unit (unit index `unit`, row
  // nvalid-1 is its newest token), in pool page `page` (ok: a valid page).
  // With a fused append the newest token's K/V come from the input instead of
  // the pool, patched into the tile, and the first query head of each kv head
  // group writes them into the page (16-token pages only: the append entry
  // point refuses other page sizes); other waves that read the slot meanwhile
  // discard what they read.
  __device__ inline void patch_last(Tile& u, int nvalid, int s, int h, int page, bool ok, int unit = 0) {
    if constexpr (BS != kBlock) return;
    if (a.k_new == nullptr || !ok) return;
    const int tn = nvalid - 1;
    const int slot = (unit % kUPP) * UT + tn;  // the newest token's slot in its page
    const int hk = h / a.group;
    if (tq == tn % S::TPI) {
      const int64_t src = (((int64_t)s * a.hkv + hk) * D + dc * S::VEC) * S::ES;
      const Raw<S::NW> kk = load_raw<S::NW>(static_cast<const uint8_t*>(a.k_new) + src);
      const Raw<S::NW> vv = load_raw<S::NW>(static_cast<const uint8_t*>(a.v_new) + src);
#pragma unroll
      for (int r = 0; r < S::ROWS; ++r)
        if (r == tn / S::TPI) {
          u.k[r] = kk;
          u.v[r] = vv;
        }
      if (h % a.group == 0) {
        uint8_t* base = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.pool)) +
                        ((int64_t)page * a.page_elems + ((int64_t)a.layer * a.hkv + hk) * 2 * BS * D +
                         (int64_t)slot * D + dc * S::VEC) * S::ES;
        store_raw<S::NW>(base, kk);
        store_raw<S::NW>(base + (int64_t)BS * D * S::ES, vv);
      }
    }
  }

  // Balanced schedule: items are query heads, one record per slot.
  __device__ inline void finish_slot(int s, int h, bool whole, int64_t slot) { finish(s, h, whole, slot); }

  // Close the piece of row (s, h): the final output if the piece is the whole
  // context, else partial record `rec`.
  __device__ inline void finish(int s, int h, bool whole, int64_t rec) {
    l = strided_reduce<S::LPT, OpSum>(l);
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) acc[i] = strided_reduce<S::LPT, OpSum>(acc[i]);
    if (tq != 0) return;
    if (whole) {
      const int64_t row = ((int64_t)s * a.hq + h) * D;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int i = 0; i < S::VEC; ++i) store_out<T, OUT_F32>(a.out, row + dc * S::VEC + i, acc[i] * inv);
    } else {
#pragma unroll
      for (int i = 0; i < S::VEC; ++i) a.ws_acc[rec * D + dc * S::VEC + i] = acc[i];
      if (dc == 0) a.ws_ml[rec] = make_float2(m, l);
    }
  }
};

// Grid schedule: one wave per (split, query head, sequence).
template <class T, int D, int U, bool OUT_F32, bool CONTIG>
__global__ __launch_bounds__(kWave) void attn_valu_grid(AttnArgs a) {
  using Wv = ValuWave<T, D, OUT_F32, CONTIG>;
  using Tile = typename Wv::Tile;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  // The split's table entries, bounded by the table width (independent of
  // the length load).
  const int split_pages = a.split_tokens / kBlock;
  const int pg0 = split * split_pages;
  int my_page = -1;
  if constexpr (!CONTIG)
    if (lane < split_pages && pg0 + lane < a.max_blocks) my_page = a.bt[(int64_t)s * a.max_blocks + pg0 + lane];
  const int ctx = clamp_ctx(a.ctx[s], a.max_ctx);
  const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
  Wv w(a, lane);
  if (ctx == 0) {
    if (split == 0 && w.tq == 0) {
#pragma unroll
      for (int i = 0; i < Wv::S::VEC; ++i)
        store_out<T, OUT_F32>(a.out, ((int64_t)s * a.hq + h) * D + w.dc * Wv::S::VEC + i, 0.f);
    }
    return;
  }
  if (split >= nsplit) return;
  const int tok_end = min(ctx, (split + 1) * a.split_tokens);
  const int npg = (tok_end - split * a.split_tokens + kBlock - 1) / kBlock;
  w.begin(s, h);
  page_pipeline<U, Tile>(
      npg, [&](int i, Tile& t) { return w.load(__builtin_amdgcn_readlane(my_page, i), s, pg0 + i, h, t); },
      [&](int i, Tile& t, bool ok) {
        const int nv = min(kBlock, tok_end - (pg0 + i) * kBlock);
        if (pg0 + i == (ctx - 1) / kBlock) w.patch_last(t, nv, s, h, __builtin_amdgcn_readlane(my_page, i), ok);
        if (ok) w.page(t, nv);
      });
  w.finish(s, h, nsplit == 1, ((int64_t)s * a.hq + h) * a.max_splits + split);
}

// Balanced schedule (pf_sched.h): four waves per workgroup, items are query
// heads.
template <class T, int D, int U, bool OUT_F32, bool CONTIG, int BS = kBlock, int UTO = 0>
__global__ __launch_bounds__(kSchedThreads) void attn_valu_balanced(AttnArgs a) {
  using Wv = ValuWave<T, D, OUT_F32, CONTIG, BS, UTO>;
  __shared__ SchedLds L;
  sched_build<Wv::UT>(a, L);
  zero_empty_rows<T, OUT_F32>(a, L, D);
  const int lane = threadIdx.x % kWave;
  Wv w(a, lane);
  sched_run<U, BS>(a, L, a.hq, w, lane);
}

// Merge the pieces of output rows that were split (PagedAttention blog, "The
// Attention Kernel": the final reduction combines partial softmax results
// with log-sum-exp): with M = max_j m_j and w_j = 2^(m_j - M),
//   out = sum_j w_j acc_j / sum_j w_j l_j,
// sums taken in piece order.  Pieces are read in batches of kMergeBatch; a
// batch that raises M rescales what is summed so far, so with at most
// kMergeBatch pieces this is the formula above exactly as written.  Record of
// row c, piece j: rec0 + j * js + c.  Lanes lie across (row, 4-float chunk):
// D/4 lanes per row, 64/(D/4) rows per pass; a workgroup does pass `pass`.
// All loads of a batch are issued before any is used.
constexpr int kMergeBatch = 8;

template <class T, bool OUT_F32>
__device__ inline void store_out4(void* out, int64_t idx, const float* v) {
  if constexpr (OUT_F32 || T::es == 4) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = T::narrow2(v[0], v[1]);
    w.y = T::narrow2(v[2], v[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// Pieces [jb, je) of row c, chunk q of 4 floats, folded into (M, den, num)
// in piece order, kMergeBatch at a time (batch boundaries at jb + 8k).
__device__ inline void merge_span(const AttnArgs& a, int D, int64_t rec0, int64_t js, int jb, int je, int c, int q,
                                  float& M, float& den, float* num) {
  for (int j0 = jb; j0 < je; j0 += kMergeBatch) {
    float2 ml[kMergeBatch];
    float4 av[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      if (j0 + b < je) {
        const int64_t rec = rec0 + (int64_t)(j0 + b) * js + c;
        ml[b] = a.ws_ml[rec];
        av[b] = *reinterpret_cast<const float4*>(a.ws_acc + rec * D + 4 * q);
      } else {
        ml[b] = make_float2(-INFINITY, 0.f);
        av[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) Mb = fmaxf(Mb, ml[b].x);
    if (Mb != M) {  // the batch raised the max: rescale the sums so far
      const float alpha = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
      den *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] *= alpha;
      M = Mb;
    }
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const float wj = ml[b].x == -INFINITY ? 0.f : fast_exp2(ml[b].x - M);
      den += ml[b].y * wj;
      num[0] += wj * av[b].x;
      num[1] += wj * av[b].y;
      num[2] += wj * av[b].z;
      num[3] += wj * av[b].w;
    }
  }
}

template <class T, bool OUT_F32>
__device__ inline void store_merged(const AttnArgs& a, int D, int64_t out_row0, int c, int q, float den,
                                    const float* num) {
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const float o[4] = {num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
  store_out4<T, OUT_F32>(a.out, (out_row0 + c) * D + 4 * q, o);
}

// Rows of many pieces (one long sequence split over most of the grid) are
// merged by kMergeWaves waves at once: wave w folds the w-th contiguous run of
// ceil(cnt / kMergeWaves) pieces, then wave 0 folds the waves' states in wave
// order, rescaling each to the common max.  The runs depend only on the piece
// count, so the result is still the same for any physical page order.
constexpr int kMergeWaves = 8;

// One workgroup per (item or query head, pass, sequence): one wave (W = 1)
// or kMergeWaves waves (W = kMergeWaves).  Balanced schedule: the item's
// (first record, pieces) pair, records (first + j) * rows_per_item + c; grid
// schedule: query head h's splits are records row * max_splits + j.
template <class T, bool OUT_F32, bool BAL, int W>
__global__ __launch_bounds__(kWave * W) void attn_merge_kernel(AttnArgs a, int D, int items_per_seq,
                                                               int rows_per_item, int passes) {
  const int x = blockIdx.x / passes;
  const int pass = blockIdx.x % passes;
  const int s = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int ctx = clamp_ctx(a.ctx[s], a.max_ctx);
  if (ctx == 0) return;  // uniform over the workgroup, as are the returns below
  int64_t rec0, js, out_row0;
  int cnt, rows;
  if constexpr (BAL) {
    const int2 meta = a.ws_meta[(int64_t)s * items_per_seq + x];
    if (meta.y <= 1) return;
    rec0 = (int64_t)meta.x * rows_per_item;
    js = rows_per_item;
    cnt = meta.y;
    rows = rows_per_item;
    out_row0 = (int64_t)s * a.hq + (int64_t)x * rows_per_item;
  } else {
    cnt = (ctx + a.split_tokens - 1) / a.split_tokens;
    if (cnt <= 1) return;
    out_row0 = (int64_t)s * a.hq + x;
    rec0 = out_row0 * a.max_splits;
    js = 1;
    rows = 1;
  }
  const int lpr = D / 4;
  const int c = pass * (kWave / lpr) + lane / lpr;
  const int q = lane % lpr;
  float M = -INFINITY, den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (W == 1) {
    if (c >= rows) return;
    merge_span(a, D, rec0, js, 0, cnt, c, q, M, den, num);
    store_merged<T, OUT_F32>(a, D, out_row0, c, q, den, num);
  } else {
    __shared__ float sm[W][kWave], sd[W][kWave];
    __shared__ float4 sn[W][kWave];
    const int per = (cnt + W - 1) / W;
    const int jb = wave * per, je = min(cnt, jb + per);
    if (c < rows && jb < je) merge_span(a, D, rec0, js, jb, je, c, q, M, den, num);
    sm[wave][lane] = M;
    sd[wave][lane] = den;
    sn[wave][lane] = make_float4(num[0], num[1], num[2], num[3]);
    __syncthreads();
    if (wave != 0 || c >= rows) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) Mt = fmaxf(Mt, sm[w][lane]);
    float dt = 0.f, nt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm[w][lane];
      const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - Mt);
      const float4 v = sn[w][lane];
      dt += sd[w][lane] * f;
      nt[0] += f * v.x;
      nt[1] += f * v.y;
      nt[2] += f * v.z;
      nt[3] += f * v.w;
    }
    store_merged<T, OUT_F32>(a, D, out_row0, c, q, dt, nt);
  }
}

// Merge state of one 4-float chunk of a row: running max (log2 units), sum of
// weights, weighted accumulator chunk.
struct MergeState {
  float M, den, num[4];
};

// Fold two states in the order given (a first): both rescaled to the common max.
__device__ inline MergeState merge_fold(const MergeState& a, const MergeState& b) {
  MergeState r;
  r.M = fmaxf(a.M, b.M);
  const float fa = a.M == -INFINITY ? 0.f : fast_exp2(a.M - r.M);
  const float fb = b.M == -INFINITY ? 0.f : fast_exp2(b.M - r.M);
  r.den = a.den * fa + b.den * fb;
#pragma unroll
  for (int e = 0; e < 4; ++e) r.num[e] = a.num[e] * fa + b.num[e] * fb;
  return r;
}

// The states of lanes lane & ~X and lane | X (X = 16 or 32), folded lower lane
// first, in every lane (gfx950's lane swaps of each value with itself).
template <int X>
__device__ inline MergeState merge_fold_lanes(const MergeState& s) {
  MergeState lo, hi;
  auto swap = [](float v, float& l, float& h) {
    const auto r = X == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    l = __uint_as_float(r[0]);
    h = __uint_as_float(r[1]);
  };
  swap(s.M, lo.M, hi.M);
  swap(s.den, lo.den, hi.den);
#pragma unroll
  for (int e = 0; e < 4; ++e) swap(s.num[e], lo.num[e], hi.num[e]);
  return merge_fold(lo, hi);
}

// Rows of many pieces at head dim 64, 128 or 256: one workgroup of W waves per
// output row.  A wave's 64 lanes are G = 64 / (D/4) groups, each covering the
// row's D floats; piece stream t = wave * G + group folds the t-th contiguous
// run of ceil(pieces / (W * G)) pieces.  Each wave folds its groups by lane
// swaps (groups 0+1 and 2+3, then the two pairs), wave 0 folds the waves in
// order through LDS.  The runs depend only on the piece count.
template <class T, bool OUT_F32, bool BAL, int W>
__global__ __launch_bounds__(kWave * W) void attn_merge_row_kernel(AttnArgs a, int D, int items_per_seq,
                                                                   int rows_per_item) {
  const int s = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int ctx = clamp_ctx(a.ctx[s], a.max_ctx);
  if (ctx == 0) return;  // uniform over the workgroup, as are the returns below
  int64_t rec0, js, out_row0;
  int cnt, c;
  if constexpr (BAL) {
    const int x = blockIdx.x / rows_per_item;
    c = blockIdx.x % rows_per_item;
    const int2 meta = a.ws_meta[(int64_t)s * items_per_seq + x];
    if (meta.y <= 1) return;
    rec0 = (int64_t)meta.x * rows_per_item;
    js = rows_per_item;
    cnt = meta.y;
    out_row0 = (int64_t)s * a.hq + (int64_t)x * rows_per_item;
  } else {
    cnt = (ctx + a.split_tokens - 1) / a.split_tokens;
    if (cnt <= 1) return;
    out_row0 = (int64_t)s * a.hq + blockIdx.x;
    rec0 = out_row0 * a.max_splits;
    js = 1;
    c = 0;
  }
  const int lpr = D / 4;       // 16, 32 or 64 lanes per row
  const int G = kWave / lpr;   // 4, 2 or 1 streams per wave
  const int g = lane / lpr, q = lane % lpr;
  const int per = (cnt + W * G - 1) / (W * G);
  const int jb = (wave * G + g) * per, je = min(cnt, jb + per);
  MergeState st{-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
  if (jb < je) merge_span(a, D, rec0, js, jb, je, c, q, st.M, st.den, st.num);
  if (G == 4) st = merge_fold_lanes<16>(st);
  if (G >= 2) st = merge_fold_lanes<32>(st);
  __shared__ float sm[W][kWave], sd[W][kWave];
  __shared__ float4 sn[W][kWave];
  sm[wave][lane] = st.M;
  sd[wave][lane] = st.den;
  sn[wave][lane] = make_float4(st.num[0], st.num[1], st.num[2], st.num[3]);
  __syncthreads();
  if (wave != 0 || g != 0) return;
  MergeState acc{sm[0][lane], sd[0][lane], {sn[0][lane].x, sn[0][lane].y, sn[0][lane].z, sn[0][lane].w}};
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const float4 v = sn[w][lane];
    acc = merge_fold(acc, MergeState{sm[w][lane], sd[w][lane], {v.x, v.y, v.z, v.w}});
  }
  store_merged<T, OUT_F32>(a, D, out_row0, c, q, acc.den, acc.num);
}

// ---------------------------------------------------------------- launchers
// Pages per prefetch unit: two units are in flight per wave; a unit holds
// about 32 VGPRs of K/V per lane (two-page units at head dim 128, still two
// waves per SIMD, measured 1 % slower on MI355X).
template <class T, int D, int UT = kBlock>
struct ValuUnit {
  static constexpr int bytes = 2 * UT * D * T::es / kWave;  // per lane per unit
  static constexpr int U = bytes >= 128 ? 1 : (bytes >= 64 ? 2 : 4);
};

// Pools of 8, 32 or 64 tokens per page: balanced schedule, paged, 16-bit
// elements, head dim 64 or 128.
template <class T, int D, bool OUT_F32, int BS>
static void launch_valu_bs_t(const AttnArgs& a, hipStream_t st) {
  constexpr int U = ValuUnit<T, D, BlockUnits<BS>::UT>::U;
  hipLaunchKernelGGL((attn_valu_balanced<T, D, U, OUT_F32, false, BS>), dim3(a.waves / (kSchedThreads / kWave)),
                     dim3(kSchedThreads), 0, st, a);
}

template <class T, int D, bool OUT_F32>
static int launch_valu_bs_d(const AttnArgs& a, int bs, hipStream_t st) {
  switch (bs) {
    case 8: launch_valu_bs_t<T, D, OUT_F32, 8>(a, st); return PF_OK;
    case 32: launch_valu_bs_t<T, D, OUT_F32, 32>(a, st); return PF_OK;
    case 64: launch_valu_bs_t<T, D, OUT_F32, 64>(a, st); return PF_OK;
    default: return PF_ERR_UNSUPPORTED;
  }
}

template <class T>
static int launch_valu_bs(const AttnArgs& a, int D, int bs, hipStream_t st) {
  if (D == 64) return a.out_f32 ? launch_valu_bs_d<T, 64, true>(a, bs, st) : launch_valu_bs_d<T, 64, false>(a, bs, st);
  if (D == 128)
    return a.out_f32 ? launch_valu_bs_d<T, 128, true>(a, bs, st) : launch_valu_bs_d<T, 128, false>(a, bs, st);
  return PF_ERR_UNSUPPORTED;
}

// fp32 K/V at head dim 256: 16-token pages walked in 8-token units (a 16-token
// unit is 128 VGPRs of K/V per lane, too many for two in flight); balanced
// schedule, paged pool.
constexpr int kHalfUnit = 8;

static bool half_units(const pf_geometry& g) {
  return g.dtype == PF_F32 && g.head_dim == 256 && g.block_size == kBlock;
}

// (fp32 output is the pool dtype, so there is no separate fp32-out form.)
template <bool CONTIG>
static void launch_valu_half(const AttnArgs& a, hipStream_t st) {
  constexpr int U = ValuUnit<ElF32, 256, kHalfUnit>::U;
  hipLaunchKernelGGL((attn_valu_balanced<ElF32, 256, U, false, CONTIG, kBlock, kHalfUnit>),
                     dim3(a.waves / (kSchedThreads / kWave)), dim3(kSchedThreads), 0, st, a);
}

static const void* valu_half_ptr() {
  constexpr int U = ValuUnit<ElF32, 256, kHalfUnit>::U;
  return reinterpret_cast<const void*>(&attn_valu_balanced<ElF32, 256, U, false, false, kBlock, kHalfUnit>);
}

// Block sizes other than 16 are built for 16-bit elements at head dim 64 or
// 128, balanced schedule, paged pool.
static bool block_size_supported(int bs, int dtype, int D) {
  if (bs == kBlock) return true;
  return (bs == 8 || bs == 32 || bs == 64) && dtype != PF_F32 && (D == 64 || D == 128);
}

template <class T, int D, bool OUT_F32>
static const void* valu_kernel_ptr(bool balanced) {
  constexpr int U = ValuUnit<T, D>::U;
  return balanced ? reinterpret_cast<const void*>(&attn_valu_balanced<T, D, U, OUT_F32, false>)
                  : reinterpret_cast<const void*>(&attn_valu_grid<T, D, U, OUT_F32, false>);
}

template <class T, int D, bool OUT_F32, bool CONTIG>
static void launch_valu(const AttnArgs& a, bool balanced, hipStream_t st) {
  constexpr int U = ValuUnit<T, D>::U;
  if (balanced)
    hipLaunchKernelGGL((attn_valu_balanced<T, D, U, OUT_F32, CONTIG>), dim3(a.waves / (kSchedThreads / kWave)),
                       dim3(kSchedThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_valu_grid<T, D, U, OUT_F32, CONTIG>), dim3(a.max_splits, a.hq, a.n), dim3(kWave),
                       0, st, a);
}

template <class T, bool OUT_F32, bool CONTIG>
static int dispatch_valu_d(const AttnArgs& a, int D, bool balanced, hipStream_t st) {
  switch (D) {
    case 16: launch_valu<T, 16, OUT_F32, CONTIG>(a, balanced, st); return PF_OK;
    case 32: launch_valu<T, 32, OUT_F32, CONTIG>(a, balanced, st); return PF_OK;
    case 64: launch_valu<T, 64, OUT_F32, CONTIG>(a, balanced, st); return PF_OK;
    case 128: launch_valu<T, 128, OUT_F32, CONTIG>(a, balanced, st); return PF_OK;
    case 256:
      if constexpr (T::es == 2) {
        launch_valu<T, 256, OUT_F32, CONTIG>(a, balanced, st);
        return PF_OK;
      }
      return PF_ERR_UNSUPPORTED;
    default: return PF_ERR_UNSUPPORTED;
  }
}

template <class T>
static int dispatch_valu(const AttnArgs& a, int D, bool balanced, bool contig, hipStream_t st) {
  if (contig)
    return a.out_f32 ? dispatch_valu_d<T, true, true>(a, D, balanced, st)
                     : dispatch_valu_d<T, false, true>(a, D, balanced, st);
  return a.out_f32 ? dispatch_valu_d<T, true, false>(a, D, balanced, st)
                   : dispatch_valu_d<T, false, false>(a, D, balanced, st);
}

template <class T>
static const void* valu_ptr_dtype(int D) {
  switch (D) {
    case 16: return valu_kernel_ptr<T, 16, false>(true);
    case 32: return valu_kernel_ptr<T, 32, false>(true);
    case 64: return valu_kernel_ptr<T, 64, false>(true);
    case 128: return valu_kernel_ptr<T, 128, false>(true);
    case 256:
      if constexpr (T::es == 2) return valu_kernel_ptr<T, 256, false>(true);
      return nullptr;
    default: return nullptr;
  }
}

template <class T, bool BAL>
static void launch_merge_row(const AttnArgs& a, int D, int items_per_seq, int rows_per_item, hipStream_t st) {
  const dim3 grid(BAL ? items_per_seq * rows_per_item : a.hq, a.n);
  if (a.out_f32)
    hipLaunchKernelGGL((attn_merge_row_kernel<T, true, BAL, kMergeWaves>), grid, dim3(kWave * kMergeWaves), 0, st,
                       a, D, items_per_seq, rows_per_item);
  else
    hipLaunchKernelGGL((attn_merge_row_kernel<T, false, BAL, kMergeWaves>), grid, dim3(kWave * kMergeWaves), 0,
                       st, a, D, items_per_seq, rows_per_item);
}

template <class T, bool BAL, int W>
static void launch_merge_w(const AttnArgs& a, dim3 grid, int D, int items_per_seq, int rows_per_item, int passes,
                           hipStream_t st) {
  if (a.out_f32)
    hipLaunchKernelGGL((attn_merge_kernel<T, true, BAL, W>), grid, dim3(kWave * W), 0, st, a, D, items_per_seq,
                       rows_per_item, passes);
  else
    hipLaunchKernelGGL((attn_merge_kernel<T, false, BAL, W>), grid, dim3(kWave * W), 0, st, a, D, items_per_seq,
                       rows_per_item, passes);
}

// Rows expected to hold many pieces -- the balanced schedule's waves spread
// over few items (16 or more waves per item), or 16 or more fixed splits --
// are merged kMergeWaves waves per row group; the choice depends only on the
// call's sizes.  Measured on MI355X, one sequence of 2^20 tokens (GQA shape,
// ~1000 pieces per row): one wave per row group took ~88 us, about as long as
// the partition kernel; eight waves take ~15 us, and sixteen are no faster
// (the few workgroups of such a call are then bound by their CUs' bandwidth).
template <class T>
static void launch_merge(const AttnArgs& a, int D, bool balanced, int items_per_seq, int rows_per_item,
                         hipStream_t st) {
  const int rows = balanced ? rows_per_item : 1;
  const int rpp = kWave / (D / 4);  // rows per pass of the merge
  const int passes = (rows + rpp - 1) / rpp;
  const dim3 grid((balanced ? items_per_seq : a.hq) * passes, a.n);
  const int64_t items = (int64_t)a.n * (balanced ? items_per_seq : a.hq);
  const bool wide = balanced ? (int64_t)a.waves >= 16 * items : a.max_splits >= 16;
  // few rows in all (one long sequence): one workgroup per row, so the reading
  // spreads over as many CUs as there are rows
  const bool per_row = wide && D >= 64 && items * rows <= 256;
  if (balanced) {
    if (per_row) launch_merge_row<T, true>(a, D, items_per_seq, rows_per_item, st);
    else if (wide) launch_merge_w<T, true, kMergeWaves>(a, grid, D, items_per_seq, rows_per_item, passes, st);
    else launch_merge_w<T, true, 1>(a, grid, D, items_per_seq, rows_per_item, passes, st);
  } else {
    if (per_row) launch_merge_row<T, false>(a, D, items_per_seq, rows_per_item, st);
    else if (wide) launch_merge_w<T, false, kMergeWaves>(a, grid, D, items_per_seq, rows_per_item, passes, st);
    else launch_merge_w<T, false, 1>(a, grid, D, items_per_seq, rows_per_item, passes, st);
  }
}

static bool valu_supports(int dtype, int D) {
  (void)dtype;
  switch (D) {
    case 16: case 32: case 64: case 128: case 256: return true;  // fp32 at 256: half units
    default: return false;
  }
}

// Compute units of the current device (256 on MI355X if the query fails),
// asked once per device; the cache may be filled by several threads at once.
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Resident waves per CU of a balanced kernel (16 if the query fails), asked
// of the runtime once per kernel and device: the answer depends only on the
// kernel's resources, and the query would otherwise run on every call.
static int occupancy_waves(const void* kernel, size_t lds) {
  struct Entry {
    const void* kernel;
    int dev, waves;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    dev = -1;
  }
  {
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry& e : cache)
      if (e.kernel == kernel && e.dev == dev) return e.waves;
  }
  int blocks = 0;
  int waves = 16;
  if (!kernel || hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kSchedThreads, lds) != hipSuccess ||
      blocks <= 0) {
    (void)hipGetLastError();
  } else {
    waves = blocks * (kSchedThreads / kWave);
  }
  std::lock_guard<std::mutex> lk(mu);
  cache.push_back({kernel, dev, waves});
  return waves;
}

}  // namespace pf

using namespace pf;

namespace {

struct Plan {
  bool mfma;
  bool balanced;
  int32_t split;     // grid schedule: tokens per split
  int64_t splits;    // grid schedule: splits of the longest context
  int32_t waves;     // balanced schedule: waves in the grid
  int64_t records;   // partial records
  int64_t items;     // balanced schedule: items (for the meta array)
  int32_t items_per_seq, rows_per_item;
};

bool use_mfma(const pf_pool* pool, int32_t num_q_heads) {
  const pf_geometry& g = pool->g;
  if (!pool->gqa_mfma || g.dtype == PF_F32) return false;
  const int group = num_q_heads / g.num_kv_heads;
  return group > 1 && group <= 16 && mfma_supports(g.head_dim) && (g.block_size == 8 || g.block_size % kBlock == 0);
}

// Grid schedule split: the largest split (64 pages) unless that leaves fewer
// work items than about two per SIMD, then halve down to 4 pages.  Measured on
// the 13B-style and GQA workloads: fewer, longer splits win, since each work
// item pays a prologue and a partial write.
int32_t grid_split(const pf_pool* pool, bool mfma, int32_t n, int32_t num_q_heads, int32_t max_ctx) {
  if (pool->split_tokens > 0) return pool->split_tokens;
  const int64_t heads = mfma ? pool->g.num_kv_heads : num_q_heads;
  const int64_t want = 2 * 4 * 256;
  int32_t st = 64 * kBlock;
  while (st > 4 * kBlock && (int64_t)n * heads * ((max_ctx + st - 1) / st) < want) st /= 2;
  return st;
}

Plan make_plan(const pf_pool* pool, int32_t n, int32_t num_q_heads, int32_t max_ctx) {
  Plan p{};
  const pf_geometry& g = pool->g;
  p.mfma = use_mfma(pool, num_q_heads);
  p.items_per_seq = p.mfma ? g.num_kv_heads : num_q_heads;
  p.rows_per_item = p.mfma ? num_q_heads / g.num_kv_heads : 1;
  const int sched = pool->schedule;
  const bool half = half_units(g);
  p.balanced = sched == 2 || (sched == 0 && n <= kMaxSeqsBalanced) || g.block_size != kBlock || half;
  if (n > kMaxSeqsBalanced) p.balanced = false;
  // short contexts: every (sequence, head) whole in one wave, nothing to merge
  const bool whole = sched == 0 && g.block_size == kBlock && !half && pool->split_tokens == 0 &&
                     max_ctx <= kWholeItemTokens;
  if (whole) p.balanced = false;
  // tokens per unit of the walk
  const int ut = half ? kHalfUnit : (g.block_size < kBlock ? g.block_size : kBlock);
  if (p.balanced) {
    // Waves: 8 per CU (two per SIMD), or fewer if the kernel's occupancy is
    // lower, and no more than one wave per 4 pages of the longest possible
    // stream; whole workgroups.  Measured on the 13B-style and GQA workloads:
    // 8 per CU is as fast as the full resident capacity for the first and
    // clearly faster for the second (fewer pieces, fewer partial records).
    int per_cu = pool->waves_per_cu;
    if (per_cu <= 0) {
      const void* k = p.mfma ? mfma_balanced_kernel(g.dtype, g.head_dim)
                      : half ? valu_half_ptr()
                      : g.dtype == PF_F32 ? valu_ptr_dtype<ElF32>(g.head_dim)
                      : (g.dtype == PF_F16 ? valu_ptr_dtype<ElF16>(g.head_dim) : valu_ptr_dtype<ElBF16>(g.head_dim));
      const int occ = occupancy_waves(k, 0);
      per_cu = occ > 0 && occ < 8 ? occ : 8;
    }
    const int64_t wpg = kSchedThreads / kWave;
    const int64_t upper = (int64_t)n * p.items_per_seq * ((max_ctx + ut - 1) / ut);
    int64_t waves = (int64_t)device_cus() * per_cu;
    const int64_t cap = (upper + 3) / 4;
    if (waves > cap) waves = cap;
    waves = ((waves + wpg - 1) / wpg) * wpg;
    if (waves < wpg) waves = wpg;
    p.waves = (int32_t)waves;
    p.items = (int64_t)n * p.items_per_seq;
    p.records = (p.items + waves) * p.rows_per_item;
  } else {
    p.split = whole ? (max_ctx <= kBlock ? kBlock : (max_ctx + kBlock - 1) / kBlock * kBlock)
                    : grid_split(pool, p.mfma, n, num_q_heads, max_ctx);
    p.splits = max_ctx <= 0 ? 1 : (max_ctx + p.split - 1) / p.split;
    p.records = p.splits > 1 ? (int64_t)n * num_q_heads * p.splits : 0;
  }
  return p;
}

// Workspace: fp32 accumulators [records][D], (max, sum) pairs [records], and
// for the balanced schedule the per-item (first record, pieces) pairs.
size_t plan_workspace(const Plan& p, int head_dim) {
  if (p.records == 0) return 0;
  size_t bytes = (size_t)p.records * head_dim * 4 + (size_t)p.records * 8;
  if (p.balanced) bytes += (size_t)p.items * 8;
  return bytes;
}

}  // namespace

extern "C" int32_t pf_attention_kernel(const pf_pool* pool, int32_t num_q_heads) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->g.num_kv_heads != 0) return -1;
  return use_mfma(pool, num_q_heads) ? 1 : 0;
}

extern "C" int32_t pf_attention_split_tokens(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                             int32_t max_context_len) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->g.num_kv_heads != 0) return 0;
  const Plan p = make_plan(pool, n, num_q_heads, max_context_len);
  return p.balanced ? 0 : p.split;
}

extern "C" int32_t pf_attention_waves(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                      int32_t max_context_len) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->g.num_kv_heads != 0) return 0;
  const Plan p = make_plan(pool, n, num_q_heads, max_context_len);
  return p.balanced ? p.waves : 0;
}

extern "C" size_t pf_attention_workspace_bytes(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                               int32_t max_context_len) {
  if (!pool || n <= 0 || num_q_heads <= 0 || max_context_len <= 0 || num_q_heads % pool->g.num_kv_heads != 0)
    return 0;
  return plan_workspace(make_plan(pool, n, num_q_heads, max_context_len), pool->g.head_dim);
}

namespace {

// Checks shared by both entry points, then plan, workspace and launches.  The
// caller has filled the block source of `a` (pool and table, or contiguous
// cache) and validated it.
int attend(const pf_pool* pool, AttnArgs& a, bool contig, const void* q, int32_t num_q_heads,
           const int32_t* ctx_dev, int32_t n, int32_t max_context_len, float scale, void* out, int32_t out_dtype,
           void* workspace, size_t workspace_bytes, void* hip_stream) {
  const pf_geometry& g = pool->g;
  if (n < 0 || num_q_heads <= 0 || num_q_heads % g.num_kv_heads != 0 || max_context_len < 0)
    return PF_ERR_INVALID;
  if (out_dtype != PF_F32 && out_dtype != g.dtype) return PF_ERR_INVALID;
  // the contiguous twin walks 16-token blocks whatever the pool's page size
  const int bs = contig ? kBlock : g.block_size;
  if (!valu_supports(g.dtype, g.head_dim) || !block_size_supported(bs, g.dtype, g.head_dim))
    return PF_ERR_UNSUPPORTED;
  if (bs != kBlock && n > kMaxSeqsBalanced) return PF_ERR_UNSUPPORTED;
  const bool half = half_units(g);  // the contiguous twin walks 16-token blocks, so this holds for it too
  if (half && n > kMaxSeqsBalanced) return PF_ERR_UNSUPPORTED;
  if (n == 0) return PF_OK;
  if (n > 65535 || num_q_heads > 65535) return PF_ERR_INVALID;
  if (!q || !ctx_dev || !out) return PF_ERR_INVALID;
  const size_t qa = (size_t)g.head_dim * pool->elem_bytes >= 16 ? 16 : 8;
  if (reinterpret_cast<uintptr_t>(q) % qa != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return PF_ERR_INVALID;

  const Plan p = make_plan(pool, n, num_q_heads, max_context_len);
  if (!p.balanced && p.splits > 65535) return PF_ERR_INVALID;
  a.q = q;
  a.out = out;
  a.ctx = ctx_dev;
  a.hkv = g.num_kv_heads;
  a.hq = num_q_heads;
  a.group = num_q_heads / g.num_kv_heads;
  a.max_ctx = max_context_len;
  a.n = n;
  a.split_tokens = p.balanced ? kBlock : p.split;
  a.max_splits = p.balanced ? 1 : (int32_t)p.splits;
  a.waves = p.waves;
  const float sc = scale > 0.f ? scale : 1.f / std::sqrt((float)g.head_dim);
  a.qscale = sc * kLog2e;
  a.out_f32 = out_dtype == PF_F32 && g.dtype != PF_F32 ? 1 : 0;

  const size_t need = plan_workspace(p, g.head_dim);
  if (need > 0) {
    if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return PF_ERR_WORKSPACE;
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(w);
    a.ws_ml = reinterpret_cast<float2*>(w + p.records * g.head_dim * 4);
    a.ws_meta = reinterpret_cast<int2*>(w + p.records * g.head_dim * 4 + p.records * 8);
  }
  if (p.balanced && need == 0) return PF_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)hip_stream;
  if (pool->ev_start) (void)hipEventRecord((hipEvent_t)pool->ev_start, st);
  int rc;
  if (half) {
    if (contig) launch_valu_half<true>(a, st);
    else launch_valu_half<false>(a, st);
    rc = PF_OK;
  } else if (bs != kBlock) {
    if (p.mfma) rc = launch_mfma_bs(a, g.dtype, g.head_dim, bs, st);
    else if (g.dtype == PF_F16) rc = launch_valu_bs<ElF16>(a, g.head_dim, bs, st);
    else rc = launch_valu_bs<ElBF16>(a, g.head_dim, bs, st);
  } else if (p.mfma) {
    rc = launch_mfma(a, g.dtype, g.head_dim, p.balanced, contig, st);
  } else {
    switch (g.dtype) {
      case PF_F32: rc = dispatch_valu<ElF32>(a, g.head_dim, p.balanced, contig, st); break;
      case PF_F16: rc = dispatch_valu<ElF16>(a, g.head_dim, p.balanced, contig, st); break;
      default: rc = dispatch_valu<ElBF16>(a, g.head_dim, p.balanced, contig, st); break;
    }
  }
  if (rc != PF_OK) return rc;
  if (hipGetLastError() != hipSuccess) return PF_ERR_HIP;
  if (pool->ev_stop) (void)hipEventRecord((hipEvent_t)pool->ev_stop, st);
  if (p.records > 0) {
    switch (g.dtype) {
      case PF_F32: launch_merge<ElF32>(a, g.head_dim, p.balanced, p.items_per_seq, p.rows_per_item, st); break;
      case PF_F16: launch_merge<ElF16>(a, g.head_dim, p.balanced, p.items_per_seq, p.rows_per_item, st); break;
      default: launch_merge<ElBF16>(a, g.head_dim, p.balanced, p.items_per_seq, p.rows_per_item, st); break;
    }
    if (hipGetLastError() != hipSuccess) return PF_ERR_HIP;
  }
  return PF_OK;
}

}  // namespace

static int paged_attention(const pf_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                           const void* k_new, const void* v_new, const int32_t* bt_dev, int32_t max_blocks,
                           const int32_t* ctx_dev, int32_t n, int32_t max_context_len, float scale, void* out,
                           int32_t out_dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  const pf_geometry& g = pool->g;
  if (layer < 0 || layer >= g.num_layers || max_blocks <= 0 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks * g.block_size)
    return PF_ERR_INVALID;
  if (n > 0 && !bt_dev) return PF_ERR_INVALID;
  AttnArgs a{};
  a.pool = pool->dev;
  a.bt = bt_dev;
  a.page_elems = (int64_t)pool->page_elems;
  a.layer = layer;
  a.num_pages = g.num_pages;
  a.max_blocks = max_blocks;
  a.k_new = k_new;
  a.v_new = v_new;
  return attend(pool, a, false, q, num_q_heads, ctx_dev, n, max_context_len, scale, out, out_dtype, workspace,
                workspace_bytes, hip_stream);
}

extern "C" int pf_paged_decode_attention(const pf_pool* pool, int32_t layer, const void* q,
                                         int32_t num_q_heads, const int32_t* bt_dev,
                                         int32_t max_blocks, const int32_t* ctx_dev, int32_t n,
                                         int32_t max_context_len, float scale, void* out,
                                         int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                         void* hip_stream) {
  return paged_attention(pool, layer, q, num_q_heads, nullptr, nullptr, bt_dev, max_blocks, ctx_dev, n,
                         max_context_len, scale, out, out_dtype, workspace, workspace_bytes, hip_stream);
}

// ------------------------------------------------- the no-allocation variant
// The workspace of pf_paged_decode_attention_noalloc: a fixed device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is asked of the runtime once per device, with that
// device current, and that address is what the kernels receive.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of `scratch` on device dev, or null if the runtime
// cannot give it.  Thread-safe; the answer is kept per device.
static void* scratch_on(int dev) {
  static std::mutex mu;
  static void* addr[64];
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

extern "C" int pf_paged_decode_attention_noalloc(const pf_pool* pool, int32_t layer, const void* q,
                                                 int32_t num_q_heads, const int32_t* bt_dev, int32_t max_blocks,
                                                 const int32_t* ctx_dev, int32_t n, int32_t max_context_len,
                                                 float scale, void* out, int32_t out_dtype, void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  const size_t need = pf_attention_workspace_bytes(pool, n, num_q_heads, max_context_len);
  if (need > kScratchBytes) return PF_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipStream_t st = (hipStream_t)hip_stream;
    if ((st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess) {
      (void)hipGetLastError();
      return PF_ERR_HIP;
    }
    ws = scratch_on(dev);
    if (ws == nullptr) return PF_ERR_HIP;
  }
  return paged_attention(pool, layer, q, num_q_heads, nullptr, nullptr, bt_dev, max_blocks, ctx_dev, n,
                         max_context_len, scale, out, out_dtype, ws, ws ? kScratchBytes : 0, hip_stream);
}

extern "C" int pf_paged_decode_attention_append(const pf_pool* pool, int32_t layer, const void* q,
                                                int32_t num_q_heads, const void* k_new, const void* v_new,
                                                const int32_t* bt_dev, int32_t max_blocks, const int32_t* ctx_dev,
                                                int32_t n, int32_t max_context_len, float scale, void* out,
                                                int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                                void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (pool->g.block_size != kBlock) return PF_ERR_UNSUPPORTED;
  if (n > 0 && (!k_new || !v_new || reinterpret_cast<uintptr_t>(k_new) % 16 != 0 ||
                reinterpret_cast<uintptr_t>(v_new) % 16 != 0))
    return PF_ERR_INVALID;
  if ((size_t)pool->g.head_dim * pool->elem_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  return paged_attention(pool, layer, q, num_q_heads, k_new, v_new, bt_dev, max_blocks, ctx_dev, n,
                         max_context_len, scale, out, out_dtype, workspace, workspace_bytes, hip_stream);
}

extern "C" int pf_contiguous_decode_attention(const pf_pool* pool, const void* q, int32_t num_q_heads,
                                              const void* k, const void* v, int64_t seq_stride,
                                              int64_t token_stride, int64_t head_stride, int32_t max_len,
                                              const int32_t* ctx_dev, int32_t n, int32_t max_context_len,
                                              float scale, void* out, int32_t out_dtype, void* workspace,
                                              size_t workspace_bytes, void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (max_len <= 0 || max_len % kBlock != 0 || max_context_len < 0 || max_context_len > max_len)
    return PF_ERR_INVALID;
  const int64_t es = (int64_t)pool->elem_bytes;
  if (seq_stride <= 0 || token_stride <= 0 || head_stride <= 0 || (seq_stride * es) % 16 != 0 ||
      (token_stride * es) % 16 != 0 || (head_stride * es) % 16 != 0)
    return PF_ERR_INVALID;
  if (n > 0 && (!k || !v || reinterpret_cast<uintptr_t>(k) % 16 != 0 || reinterpret_cast<uintptr_t>(v) % 16 != 0))
    return PF_ERR_INVALID;
  AttnArgs a{};
  a.kc = k;
  a.vc = v;
  a.c_seq = seq_stride;
  a.c_tok = token_stride;
  a.c_head = head_stride;
  a.max_blocks = max_len / kBlock;
  return attend(pool, a, true, q, num_q_heads, ctx_dev, n, max_context_len, scale, out, out_dtype, workspace,
                workspace_bytes, hip_stream);
}
