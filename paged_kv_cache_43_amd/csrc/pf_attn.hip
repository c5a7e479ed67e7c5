// Decode attention over paged K/V: split partition kernel, split-K merge
// kernel and the pf_paged_decode_attention entry point.
//
// What is computed (PagedAttention blog, "The Attention Kernel"; PageFault,
// "Four stages", stage 3): for sequence s and query head h,
//   out = softmax(scale * K q) V  over the first ctx[s] tokens,
// where every K/V row is found through the sequence's block table.  The blog's
// kernel keeps a running max and sum while it walks the blocks (online
// softmax) and merges partial results across thread blocks with log-sum-exp;
// both are used here, in fp32.
//
// Work decomposition (gfx950, wave64):
//  * One wave per work item (sequence, head, context split).  A split is a
//    fixed range of split_tokens logical tokens (a multiple of the page size),
//    so split boundaries and the merge order depend only on logical positions:
//    ordered and shuffled page orders give the same bits.
//  * The split's block-table entries are loaded once into lanes and broadcast
//    per page with readlane: there is no dependent load chain per page.
//  * Lanes lie across the head dimension: each lane holds VEC consecutive
//    elements (a 16-byte load), D/VEC lanes cover one token, and one wave
//    instruction loads 64/(D/VEC) consecutive tokens of a page.  The K and V
//    tiles of a (page, layer, kv head) are adjacent in the pool, so a page is
//    read as 2*B*D*es contiguous bytes.
//  * The next page's K/V loads are issued before the current page is used.
//  * QK partial dots are summed across the D/VEC lanes of a token with DPP
//    moves; the page maximum is a wave-wide reduction; the running max is
//    therefore wave-uniform, so each lane can accumulate p*v for its own
//    tokens and the per-lane accumulators are combined once per split.
//  * Only the sequence's last page can hold tokens past the length; it takes
//    a masked path that replaces their scores by -inf and their values by 0
//    (selects, never multiplications, so sentinel NaNs in the tail never reach
//    the result).
//  * Scores are kept in log2 units: q is pre-multiplied by scale*log2(e) and
//    exponentials are exp2.
#include <cmath>

#include "pf_attn.h"
#include "pf_common.h"
#include "pf_internal.h"

namespace pf {

template <class T, int D>
struct ValuShape {
  static constexpr int ES = T::es;
  static constexpr int VEC0 = 16 / ES;
  static constexpr int VEC = VEC0 < D * kBlock / kWave ? VEC0 : D * kBlock / kWave;  // elements per lane
  static constexpr int LPT = D / VEC;             // lanes per token
  static constexpr int TPI = kWave / LPT;         // tokens per wave instruction
  static constexpr int ROWS = kBlock / TPI;       // instructions per K (or V) tile
  static constexpr int NW = VEC * ES / 4;         // 32-bit words per lane per row
  static_assert(LPT >= 1 && LPT <= kWave && TPI <= kBlock && ROWS * TPI == kBlock, "shape");
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

template <class T, int D, bool OUT_F32>
__global__ __launch_bounds__(kWave) void attn_valu_kernel(AttnArgs a) {
  using S = ValuShape<T, D>;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int dc = lane % S::LPT;   // which VEC-chunk of the head dimension
  const int tq = lane / S::LPT;   // which token of a wave instruction

  int ctx = a.ctx[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
  const int64_t out_row = ((int64_t)s * a.hq + h) * D;
  if (ctx == 0) {
    if (split == 0 && tq == 0) {
#pragma unroll
      for (int i = 0; i < S::VEC; ++i) store_out<T, OUT_F32>(a.out, out_row + dc * S::VEC + i, 0.f);
    }
    return;
  }
  if (split >= nsplit) return;

  // q, pre-scaled into log2 units
  float qf[S::VEC];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (out_row + dc * S::VEC) * S::ES;
    Raw<S::NW> r = load_raw<S::NW>(qp);
    widen_words<T, S::NW>(r, qf);
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) qf[i] *= a.qscale;
  }

  const int tok0 = split * a.split_tokens;
  const int tok_end = min(ctx, tok0 + a.split_tokens);
  const int pg0 = tok0 / kBlock;
  const int npg = (tok_end - tok0 + kBlock - 1) / kBlock;
  // this split's table entries, one per lane
  const int my_page = lane < npg ? a.bt[(int64_t)s * a.max_blocks + pg0 + lane] : -1;

  const int hk = h / a.group;
  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const int64_t head_off = ((int64_t)a.layer * a.hkv + hk) * 2 * kBlock * D;  // elements
  const int64_t lane_off = (int64_t)(tq * D + dc * S::VEC);                   // elements

  float m = -INFINITY;
  float l = 0.f;
  float acc[S::VEC];
#pragma unroll
  for (int i = 0; i < S::VEC; ++i) acc[i] = 0.f;

  Raw<S::NW> ka[S::ROWS], va[S::ROWS], kb[S::ROWS], vb[S::ROWS];

  // Page i's address; an entry that is not a valid page reads page 0 instead
  // (in bounds) and is then skipped, so every path issues the same loads and
  // the wait counts stay exact.
  auto page_ptr = [&](int i, bool* ok) -> const uint8_t* {
    const int page = __builtin_amdgcn_readlane(my_page, i);
    *ok = (unsigned)page < (unsigned)a.num_pages;
    const int64_t el = (int64_t)(*ok ? page : 0) * a.page_elems + head_off + lane_off;
    return pool + el * S::ES;
  };
  auto load_tile = [&](const uint8_t* p, Raw<S::NW>* kt, Raw<S::NW>* vt) {
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) kt[r] = load_raw<S::NW>(p + (int64_t)r * S::TPI * D * S::ES);
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r)
      vt[r] = load_raw<S::NW>(p + ((int64_t)kBlock * D + r * S::TPI * D) * S::ES);
  };
  auto process = [&](const Raw<S::NW>* kt, const Raw<S::NW>* vt, int nvalid) {
    // nvalid: tokens of this page below the length (1..B)
    float sc[S::ROWS];
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) {
      float kf[S::VEC];
      widen_words<T, S::NW>(kt[r], kf);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < S::VEC; ++i) d = fmaf(qf[i], kf[i], d);
      sc[r] = group_reduce<S::LPT, OpSum>(d);
    }
    const bool full = nvalid >= kBlock;
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
    for (int i = 0; i < S::VEC; ++i) acc[i] *= alpha;
#pragma unroll
    for (int r = 0; r < S::ROWS; ++r) {
      const float p = fast_exp2(sc[r] - mn);
      float vf[S::VEC];
      widen_words<T, S::NW>(vt[r], vf);
      if (!full && r * S::TPI + tq >= nvalid) {
#pragma unroll
        for (int i = 0; i < S::VEC; ++i) vf[i] = 0.f;
      }
      l += p;
#pragma unroll
      for (int i = 0; i < S::VEC; ++i) acc[i] = fmaf(p, vf[i], acc[i]);
    }
  };
  auto nvalid_of = [&](int i) { return min(kBlock, tok_end - (pg0 + i) * kBlock); };

  // Two register tiles: the next page's loads are in flight while the current
  // page is used.  The steady-state loop issues its prefetch unconditionally;
  // the last one or two pages are peeled off after it.
  bool ok_a, ok_b;
  load_tile(page_ptr(0, &ok_a), ka, va);
  int i = 0;
  for (; i + 2 < npg; i += 2) {
    load_tile(page_ptr(i + 1, &ok_b), kb, vb);
    if (ok_a) process(ka, va, kBlock);
    load_tile(page_ptr(i + 2, &ok_a), ka, va);
    if (ok_b) process(kb, vb, kBlock);
  }
  if (i + 1 < npg) {
    load_tile(page_ptr(i + 1, &ok_b), kb, vb);
    if (ok_a) process(ka, va, kBlock);
    if (ok_b) process(kb, vb, nvalid_of(i + 1));
  } else {
    if (ok_a) process(ka, va, nvalid_of(i));
  }

  // combine the per-lane accumulators of the TPI token slots
  l = strided_reduce<S::LPT, OpSum>(l);
#pragma unroll
  for (int i = 0; i < S::VEC; ++i) acc[i] = strided_reduce<S::LPT, OpSum>(acc[i]);

  if (tq != 0) return;
  if (nsplit == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) store_out<T, OUT_F32>(a.out, out_row + dc * S::VEC + i, acc[i] * inv);
  } else {
    const int64_t rec = ((int64_t)s * a.hq + h) * a.max_splits + split;
#pragma unroll
    for (int i = 0; i < S::VEC; ++i) a.ws_acc[rec * D + dc * S::VEC + i] = acc[i];
    if (dc == 0) a.ws_ml[rec] = make_float2(m, l);
  }
}

// Merge the splits of every (sequence, query head) with more than one split:
// M = max m_j, out = sum_j 2^(m_j - M) acc_j / sum_j 2^(m_j - M) l_j, summed in
// split order (PagedAttention blog, "The Attention Kernel": the final
// reduction combines partial softmax results with log-sum-exp).
template <class T, bool OUT_F32>
__global__ __launch_bounds__(kWave) void attn_merge_kernel(AttnArgs a, int D) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = a.ctx[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
  if (nsplit <= 1) return;
  const int64_t rec0 = ((int64_t)s * a.hq + h) * a.max_splits;
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j) M = fmaxf(M, a.ws_ml[rec0 + j].x);
  float den = 0.f;
  for (int j = 0; j < nsplit; ++j) {
    const float2 ml = a.ws_ml[rec0 + j];
    den += ml.x == -INFINITY ? 0.f : ml.y * fast_exp2(ml.x - M);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t out_row = ((int64_t)s * a.hq + h) * D;
  for (int d = threadIdx.x; d < D; d += kWave) {
    float num = 0.f;
    for (int j = 0; j < nsplit; ++j) {
      const float mj = a.ws_ml[rec0 + j].x;
      if (mj != -INFINITY) num += a.ws_acc[(rec0 + j) * D + d] * fast_exp2(mj - M);
    }
    store_out<T, OUT_F32>(a.out, out_row + d, num * inv);
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int D, bool OUT_F32>
static void launch_valu(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_valu_kernel<T, D, OUT_F32>), dim3(a.max_splits, a.hq, a.n), dim3(kWave),
                     0, st, a);
}

template <class T, bool OUT_F32>
static int dispatch_valu_d(const AttnArgs& a, int D, hipStream_t st) {
  switch (D) {
    case 16: launch_valu<T, 16, OUT_F32>(a, st); return PF_OK;
    case 32: launch_valu<T, 32, OUT_F32>(a, st); return PF_OK;
    case 64: launch_valu<T, 64, OUT_F32>(a, st); return PF_OK;
    case 128: launch_valu<T, 128, OUT_F32>(a, st); return PF_OK;
    case 256:
      if constexpr (T::es == 2) {
        launch_valu<T, 256, OUT_F32>(a, st);
        return PF_OK;
      }
      return PF_ERR_UNSUPPORTED;
    default: return PF_ERR_UNSUPPORTED;
  }
}

template <class T>
static int dispatch_valu(const AttnArgs& a, int D, hipStream_t st) {
  return a.out_f32 ? dispatch_valu_d<T, true>(a, D, st) : dispatch_valu_d<T, false>(a, D, st);
}

template <class T>
static void launch_merge(const AttnArgs& a, int D, hipStream_t st) {
  if (a.out_f32)
    hipLaunchKernelGGL((attn_merge_kernel<T, true>), dim3(a.hq, a.n), dim3(kWave), 0, st, a, D);
  else
    hipLaunchKernelGGL((attn_merge_kernel<T, false>), dim3(a.hq, a.n), dim3(kWave), 0, st, a, D);
}

static bool valu_supports(int dtype, int D) {
  switch (D) {
    case 16: case 32: case 64: case 128: return true;
    case 256: return dtype != PF_F32;
    default: return false;
  }
}

}  // namespace pf

using namespace pf;

static int32_t split_tokens_for(const pf_pool* pool, bool mfma, int32_t max_ctx) {
  int32_t st = pool->split_tokens;
  if (st <= 0) st = mfma ? 512 : 256;
  (void)max_ctx;
  return st;
}

static bool use_mfma(const pf_pool* pool, int32_t num_q_heads) {
  const pf_geometry& g = pool->g;
  if (!pool->gqa_mfma || g.dtype == PF_F32) return false;
  const int group = num_q_heads / g.num_kv_heads;
  return group > 1 && group <= 16 && mfma_supports(g.head_dim);
}

extern "C" int32_t pf_attention_kernel(const pf_pool* pool, int32_t num_q_heads) {
  if (!pool || num_q_heads <= 0 || num_q_heads % pool->g.num_kv_heads != 0) return -1;
  return use_mfma(pool, num_q_heads) ? 1 : 0;
}

extern "C" int32_t pf_attention_split_tokens(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                             int32_t max_context_len) {
  (void)n;
  if (!pool || num_q_heads <= 0) return 0;
  return split_tokens_for(pool, use_mfma(pool, num_q_heads), max_context_len);
}

static int64_t max_splits_for(int32_t max_ctx, int32_t split) {
  return max_ctx <= 0 ? 1 : (max_ctx + split - 1) / split;
}

extern "C" size_t pf_attention_workspace_bytes(const pf_pool* pool, int32_t n, int32_t num_q_heads,
                                               int32_t max_context_len) {
  if (!pool || n <= 0 || num_q_heads <= 0 || max_context_len <= 0) return 0;
  const int32_t split = split_tokens_for(pool, use_mfma(pool, num_q_heads), max_context_len);
  const int64_t S = max_splits_for(max_context_len, split);
  if (S <= 1) return 0;
  const int64_t recs = (int64_t)n * num_q_heads * S;
  return (size_t)(recs * pool->g.head_dim * 4 + recs * 8);
}

extern "C" int pf_paged_decode_attention(const pf_pool* pool, int32_t layer, const void* q,
                                         int32_t num_q_heads, const int32_t* bt_dev,
                                         int32_t max_blocks, const int32_t* ctx_dev, int32_t n,
                                         int32_t max_context_len, float scale, void* out,
                                         int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                         void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  const pf_geometry& g = pool->g;
  if (layer < 0 || layer >= g.num_layers || n < 0 || num_q_heads <= 0 ||
      num_q_heads % g.num_kv_heads != 0 || max_blocks <= 0 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks * g.block_size)
    return PF_ERR_INVALID;
  if (out_dtype != PF_F32 && out_dtype != g.dtype) return PF_ERR_INVALID;
  if (g.block_size != kBlock || !valu_supports(g.dtype, g.head_dim)) return PF_ERR_UNSUPPORTED;
  if (n == 0) return PF_OK;
  if (n > 65535 || num_q_heads > 65535) return PF_ERR_INVALID;
  if (!q || !bt_dev || !ctx_dev || !out) return PF_ERR_INVALID;
  const size_t qa = (size_t)g.head_dim * pool->elem_bytes >= 16 ? 16 : 8;
  if (reinterpret_cast<uintptr_t>(q) % qa != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return PF_ERR_INVALID;

  const bool mfma = use_mfma(pool, num_q_heads);
  AttnArgs a{};
  a.pool = pool->dev;
  a.q = q;
  a.out = out;
  a.bt = bt_dev;
  a.ctx = ctx_dev;
  a.page_elems = (int64_t)pool->page_elems;
  a.layer = layer;
  a.hkv = g.num_kv_heads;
  a.hq = num_q_heads;
  a.group = num_q_heads / g.num_kv_heads;
  a.num_pages = g.num_pages;
  a.max_blocks = max_blocks;
  a.max_ctx = max_context_len;
  a.n = n;
  a.split_tokens = split_tokens_for(pool, mfma, max_context_len);
  const int64_t S = max_splits_for(max_context_len, a.split_tokens);
  if (S > 65535) return PF_ERR_INVALID;
  a.max_splits = (int32_t)S;
  const float sc = scale > 0.f ? scale : 1.f / std::sqrt((float)g.head_dim);
  a.qscale = sc * kLog2e;
  a.out_f32 = out_dtype == PF_F32 && g.dtype != PF_F32 ? 1 : 0;

  const size_t need = pf_attention_workspace_bytes(pool, n, num_q_heads, max_context_len);
  if (need > 0) {
    if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
      return PF_ERR_WORKSPACE;
    const int64_t recs = (int64_t)n * num_q_heads * S;
    a.ws_acc = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float2*>(static_cast<uint8_t*>(workspace) + recs * g.head_dim * 4);
  }

  hipStream_t st = (hipStream_t)hip_stream;
  if (pool->ev_start) hipEventRecord((hipEvent_t)pool->ev_start, st);
  int rc;
  if (mfma) {
    rc = g.dtype == PF_F16 ? launch_mfma_f16(a, g.head_dim, st) : launch_mfma_bf16(a, g.head_dim, st);
  } else {
    switch (g.dtype) {
      case PF_F32: rc = dispatch_valu<ElF32>(a, g.head_dim, st); break;
      case PF_F16: rc = dispatch_valu<ElF16>(a, g.head_dim, st); break;
      default: rc = dispatch_valu<ElBF16>(a, g.head_dim, st); break;
    }
  }
  if (rc != PF_OK) return rc;
  if (hipGetLastError() != hipSuccess) return PF_ERR_HIP;
  if (pool->ev_stop) hipEventRecord((hipEvent_t)pool->ev_stop, st);
  if (S > 1) {
    switch (g.dtype) {
      case PF_F32: launch_merge<ElF32>(a, g.head_dim, st); break;
      case PF_F16: launch_merge<ElF16>(a, g.head_dim, st); break;
      default: launch_merge<ElBF16>(a, g.head_dim, st); break;
    }
    if (hipGetLastError() != hipSuccess) return PF_ERR_HIP;
  }
  return PF_OK;
}
