// Internal interface between the attention entry point (pf_attn.hip) and the
// matrix-core kernel for grouped query heads (pf_attn_mfma.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pf_common.h"

namespace pf {

struct AttnArgs {
  const void* pool;        // bound device pool
  const void* q;           // [n][hq][D]
  void* out;               // [n][hq][D]
  float* ws_acc;           // partial accumulators, D floats per record
  float2* ws_ml;           // partial (running max in log2 units, sum) per record
  int2* ws_meta;           // balanced schedule: per item (first record, pieces)
  const int32_t* bt;       // [n][max_blocks]
  const int32_t* ctx;      // [n]
  int64_t page_elems;      // elements per page
  int32_t layer, hkv, hq, group, num_pages, max_blocks, max_ctx, n;
  int32_t split_tokens, max_splits, out_f32;
  int32_t waves;           // balanced schedule: waves in the grid
  float qscale;            // scale * log2(e)
  // Contiguous cache (no table): element (s, t, h, d) of K is
  // kc[s*c_seq + t*c_tok + h*c_head + d], of V likewise in vc.
  const void* kc;
  const void* vc;
  int64_t c_seq, c_tok, c_head;
  // Fused append (pf_paged_decode_attention_append): [n][hkv][D] K/V of each
  // sequence's newest token, written into its slot and used from registers;
  // null otherwise.
  const void* k_new;
  const void* v_new;
};

template <int NW>
__device__ inline void store_raw(void* p, const Raw<NW>& r) {
  if constexpr (NW == 4) *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
  else if constexpr (NW == 2) *reinterpret_cast<uint2*>(p) = make_uint2(r.w[0], r.w[1]);
  else *reinterpret_cast<uint32_t*>(p) = r.w[0];
}

// Where the 16 tokens of block p of sequence s live for kv head hk: byte
// addresses of the K and V rows of the block's first token and the byte step
// from one token to the next.  Paged: the block is pool page `page` (the
// table entry), whose K and V tiles are adjacent 16 x D runs; an entry that is
// not a valid page addresses page 0 instead (in bounds) and reports ok =
// false.  Contiguous: the block sits in the caller's per-sequence cache.
struct BlockAddr {
  const uint8_t* k;
  const uint8_t* v;
  int64_t tok;
  bool ok;
};

// p is the unit index inside the sequence (units of BlockUnits<BS, UTO>::UT
// tokens); page is the table entry of the page holding it.
template <bool CONTIG, int D, int ES, int BS = kBlock, int UTO = 0>
__device__ inline BlockAddr block_addr(const AttnArgs& a, int page, int s, int p, int hk) {
  using BU = BlockUnits<BS, UTO>;
  if constexpr (CONTIG) {
    const int64_t off = ((int64_t)s * a.c_seq + (int64_t)p * BU::UT * a.c_tok + (int64_t)hk * a.c_head) * ES;
    return {static_cast<const uint8_t*>(a.kc) + off, static_cast<const uint8_t*>(a.vc) + off, a.c_tok * ES, true};
  } else {
    const bool ok = (unsigned)page < (unsigned)a.num_pages;
    const int64_t off =
        ((int64_t)(ok ? page : 0) * a.page_elems + ((int64_t)a.layer * a.hkv + hk) * 2 * BS * D) * ES +
        (int64_t)(p % BU::R) * BU::UT * D * ES;
    const uint8_t* k = static_cast<const uint8_t*>(a.pool) + off;
    return {k, k + BS * D * ES, (int64_t)D * ES, ok};
  }
}

bool mfma_supports(int head_dim);
// Launch the matrix-core partition kernel (balanced or grid schedule) over
// the paged pool or, with contig, over a contiguous cache.
int launch_mfma(const AttnArgs& a, int dtype, int head_dim, bool balanced, bool contig, hipStream_t st);
// The same for a pool of block_size 32 or 64 (balanced schedule, paged).
int launch_mfma_bs(const AttnArgs& a, int dtype, int head_dim, int block_size, hipStream_t st);
// The balanced matrix-core kernel of the default page size (for occupancy
// queries), or null.
const void* mfma_balanced_kernel(int dtype, int head_dim);

}  // namespace pf
