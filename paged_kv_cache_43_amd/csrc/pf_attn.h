// Internal interface between the attention entry point (pf_attn.hip) and the
// matrix-core kernel for grouped query heads (pf_attn_mfma.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pf {

struct AttnArgs {
  const void* pool;        // bound device pool
  const void* q;           // [n][hq][D]
  void* out;               // [n][hq][D]
  float* ws_acc;           // [n][hq][max_splits][D] split partial accumulators
  float2* ws_ml;           // [n][hq][max_splits] (running max in log2 units, sum)
  const int32_t* bt;       // [n][max_blocks]
  const int32_t* ctx;      // [n]
  int64_t page_elems;      // elements per page
  int32_t layer, hkv, hq, group, num_pages, max_blocks, max_ctx, n;
  int32_t split_tokens, max_splits, out_f32;
  float qscale;            // scale * log2(e)
};

bool mfma_supports(int head_dim);
int launch_mfma_f16(const AttnArgs& a, int head_dim, hipStream_t st);
int launch_mfma_bf16(const AttnArgs& a, int head_dim, hipStream_t st);

}  // namespace pf
