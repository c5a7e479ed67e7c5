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
};

bool mfma_supports(int head_dim);
// Launch the matrix-core partition kernel (balanced or grid schedule).
int launch_mfma(const AttnArgs& a, int dtype, int head_dim, bool balanced, hipStream_t st);
// Resident waves per CU of the balanced matrix-core kernel (0 if unknown).
int mfma_balanced_waves_per_cu(int dtype, int head_dim);

}  // namespace pf
