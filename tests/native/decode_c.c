/* One decode-attention pass driven from plain C through libpf and the HIP
 * runtime, with no Python and no torch: create a pool handle, allocate device
 * memory for the pool, bind it, grow every sequence, export the block tables
 * through pinned staging, scatter every context token's K/V of every layer,
 * then run pf_paged_decode_attention per layer with fp32 output.
 *
 * usage: decode_c <input.bin> <output.bin>
 * input (little-endian): int32 n, layers, hq, hkv, d, dtype, num_pages, block;
 *   int32 free_order[num_pages]; int32 lens[n];
 *   K bits [layers][tokens][hkv][d], V bits likewise (tokens in (sequence,
 *   position) order, element size of dtype); q bits [layers][n][hq][d].
 * output: float32 [layers][n][hq][d].
 * Exit status 0 on success; any failing call prints its name and status. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pf.h"

#define HIP(x)                                                                   \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define PF(x)                                                                    \
  do {                                                                           \
    int s_ = (x);                                                                \
    if (s_ != PF_OK) {                                                           \
      fprintf(stderr, "%s returned %d\n", #x, s_);                              \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static void* read_all(const char* path, size_t* size) {
  FILE* f = fopen(path, "rb");
  void* p = NULL;
  long sz;
  if (!f) return NULL;
  if (fseek(f, 0, SEEK_END) == 0 && (sz = ftell(f)) > 0 && fseek(f, 0, SEEK_SET) == 0) {
    p = malloc((size_t)sz);
    if (p && fread(p, 1, (size_t)sz, f) != (size_t)sz) {
      free(p);
      p = NULL;
    }
    *size = (size_t)sz;
  }
  fclose(f);
  return p;
}

int main(int argc, char** argv) {
  size_t size = 0, es, tokens = 0, kv_layer_bytes, q_layer_bytes, need, ws_bytes;
  const int32_t *hdr, *free_order, *lens;
  const uint8_t *kbits, *vbits, *qbits;
  int32_t n, layers, hq, hkv, d, dtype, num_pages, block, max_len = 0, max_blocks, i, p, layer;
  int32_t *tok_seq, *tok_pos, *staging, *d_meta, *d_tok_seq, *d_tok_pos;
  uint64_t* ids;
  pf_geometry g;
  pf_pool* pool = NULL;
  void *d_pool, *d_k, *d_v, *d_q, *d_out, *d_ws = NULL;
  float* out;
  FILE* fo;
  uint8_t* buf;

  if (argc != 3) {
    fprintf(stderr, "usage: decode_c <input.bin> <output.bin>\n");
    return 2;
  }
  buf = (uint8_t*)read_all(argv[1], &size);
  if (!buf || size < 32) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  hdr = (const int32_t*)buf;
  n = hdr[0]; layers = hdr[1]; hq = hdr[2]; hkv = hdr[3]; d = hdr[4]; dtype = hdr[5];
  num_pages = hdr[6]; block = hdr[7];
  if (n <= 0 || layers <= 0 || hkv <= 0 || hq <= 0 || d <= 0 || num_pages <= 0 || block <= 0) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  es = dtype == PF_F32 ? 4 : 2;
  free_order = hdr + 8;
  lens = free_order + num_pages;
  for (i = 0; i < n; ++i) {
    tokens += (size_t)lens[i];
    if (lens[i] > max_len) max_len = lens[i];
  }
  kv_layer_bytes = tokens * (size_t)hkv * (size_t)d * es;
  q_layer_bytes = (size_t)n * (size_t)hq * (size_t)d * es;
  need = 4 * (8 + (size_t)num_pages + (size_t)n) + 2 * (size_t)layers * kv_layer_bytes + (size_t)layers * q_layer_bytes;
  if (size != need) {
    fprintf(stderr, "input holds %zu bytes, expected %zu\n", size, need);
    return 1;
  }
  kbits = (const uint8_t*)(lens + n);
  vbits = kbits + (size_t)layers * kv_layer_bytes;
  qbits = vbits + (size_t)layers * kv_layer_bytes;
  max_blocks = max_len > 0 ? (max_len + block - 1) / block : 1;

  /* host allocator: every sequence grown to its length */
  g.num_pages = num_pages; g.block_size = block; g.num_layers = layers;
  g.num_kv_heads = hkv; g.head_dim = d; g.dtype = dtype;
  PF(pf_pool_create(&g, free_order, &pool));
  ids = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)n);
  tok_seq = (int32_t*)malloc(sizeof(int32_t) * (tokens ? tokens : 1));
  tok_pos = (int32_t*)malloc(sizeof(int32_t) * (tokens ? tokens : 1));
  out = (float*)malloc(sizeof(float) * (size_t)layers * (size_t)n * (size_t)hq * (size_t)d);
  if (!ids || !tok_seq || !tok_pos || !out) return 1;
  for (i = 0, tokens = 0; i < n; ++i) {
    ids[i] = (uint64_t)i;
    for (p = 0; p < lens[i]; ++p, ++tokens) {
      tok_seq[tokens] = i;
      tok_pos[tokens] = p;
    }
  }
  PF(pf_alloc_for_seqs(pool, ids, lens, n, NULL));

  /* device memory: the pool, the tables (n*max_blocks entries, then lengths
     and newest positions), pinned staging for their upload */
  HIP(hipMalloc(&d_pool, pf_pool_bytes(pool)));
  PF(pf_pool_bind(pool, d_pool, pf_pool_bytes(pool)));
  HIP(hipMalloc((void**)&d_meta, sizeof(int32_t) * ((size_t)n * max_blocks + 2 * (size_t)n)));
  HIP(hipHostMalloc((void**)&staging, sizeof(int32_t) * ((size_t)n * max_blocks + 3 * (size_t)n), 0));
  PF(pf_export_tables(pool, ids, n, max_blocks, staging, d_meta, NULL));

  /* scatter every context token of every layer */
  HIP(hipMalloc((void**)&d_tok_seq, sizeof(int32_t) * (tokens ? tokens : 1)));
  HIP(hipMalloc((void**)&d_tok_pos, sizeof(int32_t) * (tokens ? tokens : 1)));
  HIP(hipMalloc(&d_k, kv_layer_bytes ? kv_layer_bytes : 16));
  HIP(hipMalloc(&d_v, kv_layer_bytes ? kv_layer_bytes : 16));
  HIP(hipMemcpy(d_tok_seq, tok_seq, sizeof(int32_t) * tokens, hipMemcpyHostToDevice));
  HIP(hipMemcpy(d_tok_pos, tok_pos, sizeof(int32_t) * tokens, hipMemcpyHostToDevice));
  for (layer = 0; layer < layers; ++layer) {
    HIP(hipMemcpy(d_k, kbits + (size_t)layer * kv_layer_bytes, kv_layer_bytes, hipMemcpyHostToDevice));
    HIP(hipMemcpy(d_v, vbits + (size_t)layer * kv_layer_bytes, kv_layer_bytes, hipMemcpyHostToDevice));
    PF(pf_scatter_kv(pool, layer, d_k, d_v, d_tok_seq, d_tok_pos, (int32_t)tokens, d_meta, n, max_blocks, NULL));
    HIP(hipDeviceSynchronize());   /* d_k / d_v are reused by the next layer */
  }

  /* attention, layer by layer, fp32 output */
  ws_bytes = pf_attention_workspace_bytes(pool, n, hq, max_len);
  if (ws_bytes) HIP(hipMalloc(&d_ws, ws_bytes));
  HIP(hipMalloc(&d_q, q_layer_bytes));
  HIP(hipMalloc(&d_out, sizeof(float) * (size_t)n * hq * d));
  for (layer = 0; layer < layers; ++layer) {
    HIP(hipMemcpy(d_q, qbits + (size_t)layer * q_layer_bytes, q_layer_bytes, hipMemcpyHostToDevice));
    PF(pf_paged_decode_attention(pool, layer, d_q, hq, d_meta, max_blocks, d_meta + (size_t)n * max_blocks, n,
                                 max_len, 0.0f, d_out, PF_F32, d_ws, ws_bytes, NULL));
    HIP(hipMemcpy(out + (size_t)layer * n * hq * d, d_out, sizeof(float) * (size_t)n * hq * d,
                  hipMemcpyDeviceToHost));
  }
  HIP(hipDeviceSynchronize());

  fo = fopen(argv[2], "wb");
  if (!fo || fwrite(out, sizeof(float), (size_t)layers * n * hq * d, fo) != (size_t)layers * n * hq * d) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(fo);

  for (i = 0; i < n; ++i) PF(pf_free_seq(pool, (uint64_t)i));
  if (pf_free_pages(pool) != num_pages) {
    fprintf(stderr, "pool did not come back whole\n");
    return 1;
  }
  pf_pool_destroy(pool);
  HIP(hipFree(d_pool)); HIP(hipFree(d_meta)); HIP(hipHostFree(staging)); HIP(hipFree(d_tok_seq));
  HIP(hipFree(d_tok_pos)); HIP(hipFree(d_k)); HIP(hipFree(d_v)); HIP(hipFree(d_q)); HIP(hipFree(d_out));
  if (d_ws) HIP(hipFree(d_ws));
  free(ids); free(tok_seq); free(tok_pos); free(out); free(buf);
  printf("decode_c ok: %d sequences, %d layers, %zu tokens\n", n, layers, tokens);
  return 0;
}
