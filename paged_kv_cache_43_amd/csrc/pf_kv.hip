// scatter_kv and gather_kv: moving tokens' K/V into and out of their pages.
//
// PageForge, "Five techniques" (gather / scatter kernels): new tokens' K/V are
// written into their physical pages, and a gather assembles a sequence's
// scattered pages into one contiguous view.  Here the gather is only a
// read-back for verification; attention reads the pages in place.
//
// Pool layout (see include/pf.h): page p, layer l, kv head h, kind c (K=0,
// V=1), slot o, dim d at ((((p*L + l)*H + h)*2 + c)*B + o)*D + d.  Both kernels
// move 16-byte chunks: one thread per (token, head, kind, 16-byte column), so
// a token's D-vector is written by D*es/16 adjacent threads into one
// contiguous row of its page.
#include "pf_common.h"
#include "pf_internal.h"

namespace pf {

struct KvArgs {
  uint8_t* pool;
  const uint8_t* k;        // scatter: source [T][H][D]
  const uint8_t* v;
  uint8_t* k_out;          // gather: destination [n][max_len][H][D]
  uint8_t* v_out;
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  const int32_t* bt;
  const int32_t* lens;
  int64_t total;           // threads of work
  int64_t page_elems;
  int32_t layer, L, H, D, B, es, num_pages, rows, max_blocks, max_len;
};

__global__ __launch_bounds__(256) void scatter_kv_kernel(KvArgs a) {
  const int cols = a.D * a.es / 16;  // 16-byte columns per token row
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)(i % cols);
    int64_t r = i / cols;
    const int kind = (int)(r % 2);
    r /= 2;
    const int h = (int)(r % a.H);
    const int64_t t = r / a.H;
    const int32_t seq = a.tok_seq[t];
    const int32_t pos = a.tok_pos[t];
    if (seq < 0 || seq >= a.rows || pos < 0 || (int64_t)pos >= (int64_t)a.max_blocks * a.B) continue;
    const int32_t page = a.bt[(int64_t)seq * a.max_blocks + pos / a.B];
    if (page < 0 || page >= a.num_pages) continue;
    const int64_t dst_el = (int64_t)page * a.page_elems +
                           ((((int64_t)a.layer * a.H + h) * 2 + kind) * a.B + pos % a.B) * a.D;
    const int64_t src_el = (t * a.H + h) * (int64_t)a.D;
    const uint8_t* src = (kind ? a.v : a.k) + src_el * a.es + col * 16;
    uint8_t* dst = a.pool + dst_el * a.es + col * 16;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

__global__ __launch_bounds__(256) void gather_kv_kernel(KvArgs a) {
  const int cols = a.D * a.es / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)(i % cols);
    int64_t r = i / cols;
    const int kind = (int)(r % 2);
    r /= 2;
    const int h = (int)(r % a.H);
    r /= a.H;
    const int pos = (int)(r % a.max_len);
    const int64_t s = r / a.max_len;
    int32_t len = a.lens[s];
    if (len > a.max_len) len = a.max_len;
    if (pos >= len || (int64_t)pos >= (int64_t)a.max_blocks * a.B) continue;
    const int32_t page = a.bt[s * a.max_blocks + pos / a.B];
    if (page < 0 || page >= a.num_pages) continue;
    const int64_t src_el = (int64_t)page * a.page_elems +
                           ((((int64_t)a.layer * a.H + h) * 2 + kind) * a.B + pos % a.B) * a.D;
    const int64_t dst_el = ((s * a.max_len + pos) * a.H + h) * (int64_t)a.D;
    uint8_t* dst = (kind ? a.v_out : a.k_out) + dst_el * a.es + col * 16;
    *reinterpret_cast<uint4*>(dst) =
        *reinterpret_cast<const uint4*>(a.pool + src_el * a.es + col * 16);
  }
}


// Copy-on-write page copies (PagedAttention blog, "Copy-on-Write for Parallel
// Sampling": the new block receives the shared block's contents): pair j
// copies page pairs[2j] to page pairs[2j+1], all layers, heads, K and V.  A
// page is one contiguous run of page_bytes, so the copy is a flat 16-byte
// stream; consecutive threads take consecutive chunks of one pair (reads and
// writes both coalesced).  Pairs with an id outside the pool copy nothing.
__global__ __launch_bounds__(256) void copy_pages_kernel(uint8_t* pool, const int32_t* pairs, int64_t chunks,
                                                         int64_t total, int32_t num_pages) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / chunks;
    const int64_t c = i - j * chunks;
    const int32_t src = pairs[2 * j], dst = pairs[2 * j + 1];
    if (src < 0 || src >= num_pages || dst < 0 || dst >= num_pages) continue;
    reinterpret_cast<uint4*>(pool + (int64_t)dst * chunks * 16)[c] =
        reinterpret_cast<const uint4*>(pool + (int64_t)src * chunks * 16)[c];
  }
}

// Swap copies (PagedAttention blog, "Preemption and Swapping": blocks move to
// CPU memory and back): pair j moves one whole page between the device pool
// and a page-sized slot of the pinned host store -- (page, slot) pairs when
// to_host, (slot, page) otherwise.  The kernel reads and writes host memory
// directly over the host link.  Work unit: one 16 KiB span of one page per
// workgroup, the span's pair read once, then kSwapPer independent 16-byte
// loads per thread before any store.  (One chunk per thread, pair read and
// data read back to back, cost about 50 us more per host-to-device launch on
// MI355X at any size: two dependent host reads per wave.)  The grid holds at
// most kSwapGrid workgroups (two per CU), which take the units grid-stride:
// with every unit's workgroup resident at once, a host-to-device call of
// 12-20 MB put all its host reads in flight together and ran 11-18 % slower
// than the other direction; capped, host to device runs at the DMA engine's
// rate (57 GB/s on MI355X) and device to host within a few percent of it.
// Out-of-range ids copy nothing.
constexpr int kSwapPer = 4;
constexpr int kSwapSpan = 256 * kSwapPer;  // 16-byte chunks per unit
constexpr int kSwapGrid = 512;

__global__ __launch_bounds__(256) void swap_copy_kernel(uint8_t* pool, uint8_t* host, const int32_t* pairs,
                                                        int64_t chunks, int64_t spans, int64_t units,
                                                        int32_t num_pages, int32_t num_slots, int32_t to_host) {
  for (int64_t w = blockIdx.x; w < units; w += gridDim.x) {
    const int64_t j = w / spans;
    const int64_t c0 = (w - j * spans) * kSwapSpan + threadIdx.x;
    const int32_t a = pairs[2 * j], b = pairs[2 * j + 1];
    const int32_t page = to_host ? a : b, slot = to_host ? b : a;
    if (page < 0 || page >= num_pages || slot < 0 || slot >= num_slots) continue;
    uint4* dp = reinterpret_cast<uint4*>(pool + (int64_t)page * chunks * 16);
    uint4* hp = reinterpret_cast<uint4*>(host + (int64_t)slot * chunks * 16);
    const uint4* src = to_host ? dp : hp;
    uint4* dst = to_host ? hp : dp;
    uint4 r[kSwapPer];
#pragma unroll
    for (int u = 0; u < kSwapPer; ++u)
      if (c0 + 256 * u < chunks) r[u] = src[c0 + 256 * u];
#pragma unroll
    for (int u = 0; u < kSwapPer; ++u)
      if (c0 + 256 * u < chunks) dst[c0 + 256 * u] = r[u];
  }
}

// Table upload and the scatter of each sequence's newest token for a range of
// layers, in one launch.  Threads [0, up_threads) upload: a whole export
// copies 16-byte words of the staging (host memory, read over the bus, no DMA
// engine round trip) into the device table, lengths and newest positions; an
// incremental one writes (flat index, value) pairs into the table and copies
// the lengths and newest positions.  The rest each move one 16-byte column of
// one (layer, sequence, head, K|V) row, with the destination page read from
// the staging rather than the device table, so the two halves do not depend
// on each other.
struct PrepArgs {
  const uint4* src;          // whole export: n16 16-byte words
  uint4* dst;
  int64_t n16;
  const int2* pairs;         // incremental export: npairs (flat index, value)
  int32_t* table;            // n * max_blocks entries
  int64_t npairs, table_words;
  const int32_t* tail_src;   // words after the n16 (whole) or lengths + newest (incremental)
  int32_t* tail_dst;
  int64_t tail;
  int64_t up_threads;
  uint8_t* pool;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* lens_host;  // staging: lengths
  const int32_t* page_host;  // staging: newest token's page
  int64_t page_elems;
  int64_t sc_threads;
  int32_t n, layer0, H, D, B, es, num_pages;
};

__global__ __launch_bounds__(256) void prepare_kernel(PrepArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.up_threads) {
    if (i < a.n16) a.dst[i] = a.src[i];
    if (i < a.npairs) {
      const int2 pr = a.pairs[i];
      if (pr.x >= 0 && pr.x < a.table_words) a.table[pr.x] = pr.y;  // staging rewritten too early: no stray write
    }
    if (i < a.tail) a.tail_dst[i] = a.tail_src[i];
    return;
  }
  int64_t r = i - a.up_threads;
  if (r >= a.sc_threads) return;
  const int cols = a.D * a.es / 16;
  const int col = (int)(r % cols);
  r /= cols;
  const int kind = (int)(r % 2);
  r /= 2;
  const int h = (int)(r % a.H);
  r /= a.H;
  const int s = (int)(r % a.n);
  const int l = (int)(r / a.n);
  const int32_t len = a.lens_host[s];
  const int32_t page = a.page_host[s];
  if (len <= 0 || page < 0 || page >= a.num_pages) return;
  const int pos = len - 1;
  const int64_t dst_el = (int64_t)page * a.page_elems +
                         ((((int64_t)(a.layer0 + l) * a.H + h) * 2 + kind) * a.B + pos % a.B) * a.D;
  const int64_t src_el = (((int64_t)l * a.n + s) * a.H + h) * (int64_t)a.D;
  *reinterpret_cast<uint4*>(a.pool + dst_el * a.es + col * 16) =
      *reinterpret_cast<const uint4*>((kind ? a.v : a.k) + src_el * a.es + col * 16);
}

static inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static int launch_grid(int64_t total, int* blocks) {
  int64_t b = (total + 255) / 256;
  if (b > 65536) b = 65536;  // grid-stride beyond this
  if (b < 1) b = 1;
  *blocks = (int)b;
  return 0;
}

}  // namespace pf

extern "C" int pf_scatter_kv(const pf_pool* pool, int32_t layer, const void* k, const void* v,
                             const int32_t* tok_seq, const int32_t* tok_pos, int32_t num_tokens,
                             const int32_t* bt_dev, int32_t num_rows, int32_t max_blocks,
                             void* hip_stream) {
  using namespace pf;
  if (!pool) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  const pf_geometry& g = pool->g;
  if (layer < 0 || layer >= g.num_layers || num_tokens < 0 || num_rows < 0 || max_blocks < 0)
    return PF_ERR_INVALID;
  if ((size_t)g.head_dim * pool->elem_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PF_OK;
  if (!k || !v || !tok_seq || !tok_pos || !bt_dev || !aligned16(k) || !aligned16(v))
    return PF_ERR_INVALID;
  KvArgs a{};
  a.pool = static_cast<uint8_t*>(pool->dev);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.tok_seq = tok_seq;
  a.tok_pos = tok_pos;
  a.bt = bt_dev;
  a.page_elems = (int64_t)pool->page_elems;
  a.layer = layer;
  a.L = g.num_layers;
  a.H = g.num_kv_heads;
  a.D = g.head_dim;
  a.B = g.block_size;
  a.es = (int32_t)pool->elem_bytes;
  a.num_pages = g.num_pages;
  a.rows = num_rows;
  a.max_blocks = max_blocks;
  a.total = (int64_t)num_tokens * g.num_kv_heads * 2 * (g.head_dim * a.es / 16);
  int blocks;
  launch_grid(a.total, &blocks);
  hipLaunchKernelGGL(scatter_kv_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream, a);
  return hipGetLastError() == hipSuccess ? PF_OK : PF_ERR_HIP;
}

extern "C" int pf_gather_kv(const pf_pool* pool, int32_t layer, const int32_t* bt_dev,
                            const int32_t* lens_dev, int32_t n, int32_t max_blocks, int32_t max_len,
                            void* k_out, void* v_out, void* hip_stream) {
  using namespace pf;
  if (!pool) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  const pf_geometry& g = pool->g;
  if (layer < 0 || layer >= g.num_layers || n < 0 || max_blocks < 0 || max_len < 0)
    return PF_ERR_INVALID;
  if ((size_t)g.head_dim * pool->elem_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  if (n == 0 || max_len == 0) return PF_OK;
  if (!bt_dev || !lens_dev || !k_out || !v_out || !aligned16(k_out) || !aligned16(v_out))
    return PF_ERR_INVALID;
  KvArgs a{};
  a.pool = static_cast<uint8_t*>(pool->dev);
  a.k_out = static_cast<uint8_t*>(k_out);
  a.v_out = static_cast<uint8_t*>(v_out);
  a.bt = bt_dev;
  a.lens = lens_dev;
  a.page_elems = (int64_t)pool->page_elems;
  a.layer = layer;
  a.L = g.num_layers;
  a.H = g.num_kv_heads;
  a.D = g.head_dim;
  a.B = g.block_size;
  a.es = (int32_t)pool->elem_bytes;
  a.num_pages = g.num_pages;
  a.max_blocks = max_blocks;
  a.max_len = max_len;
  a.total = (int64_t)n * max_len * g.num_kv_heads * 2 * (g.head_dim * a.es / 16);
  int blocks;
  launch_grid(a.total, &blocks);
  hipLaunchKernelGGL(gather_kv_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream, a);
  return hipGetLastError() == hipSuccess ? PF_OK : PF_ERR_HIP;
}

// Fill the staging for an export of seq_ids to meta_dev and set the upload
// half of a: whole (16-byte words) or incremental (pairs).
static int stage_export(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks, bool step,
                        int32_t* staging_host, int32_t* meta_dev, pf::PrepArgs& a) {
  int64_t pairs = -1;
  const int st = pf_fill_export(pool, meta_dev, seq_ids, n, max_blocks, step, staging_host, &pairs);
  if (st != PF_OK) return st;
  const int64_t nb = (int64_t)n * max_blocks;
  if (pairs < 0) {
    const int64_t words = nb + 2 * (int64_t)n;
    a.n16 = words / 4;
    a.src = reinterpret_cast<const uint4*>(staging_host);
    a.dst = reinterpret_cast<uint4*>(meta_dev);
    a.tail = words - a.n16 * 4;
    a.tail_src = staging_host + a.n16 * 4;
    a.tail_dst = meta_dev + a.n16 * 4;
  } else {
    a.npairs = pairs;
    a.pairs = reinterpret_cast<const int2*>(staging_host);
    a.table = meta_dev;
    a.table_words = nb;
    a.tail = 2 * (int64_t)n;
    a.tail_src = staging_host + nb;
    a.tail_dst = meta_dev + nb;
  }
  int64_t up = a.n16 > a.npairs ? a.n16 : a.npairs;
  if (a.tail > up) up = a.tail;
  a.up_threads = up;
  return PF_OK;
}

extern "C" int pf_export_tables(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                                int32_t* staging_host, int32_t* meta_dev, void* hip_stream) {
  using namespace pf;
  if (!pool || n < 0 || max_blocks < 0) return PF_ERR_INVALID;
  if (n == 0) return PF_OK;
  if (!staging_host || !meta_dev || !aligned16(staging_host) || !aligned16(meta_dev)) return PF_ERR_INVALID;
  PrepArgs a{};
  const int st = stage_export(pool, seq_ids, n, max_blocks, false, staging_host, meta_dev, a);
  if (st != PF_OK) return st;
  const int64_t blocks = (a.up_threads + 255) / 256;
  if (blocks > 0x7fffffff) {
    pf_export_forget(pool);
    return PF_ERR_INVALID;
  }
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, a);
  if (hipGetLastError() != hipSuccess) {
    pf_export_forget(pool);
    return PF_ERR_HIP;
  }
  return PF_OK;
}

extern "C" int pf_decode_prepare(const pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t max_blocks,
                                 int32_t* staging_host, int32_t* meta_dev, const void* k, const void* v,
                                 int32_t layer0, int32_t num_layers, void* hip_stream) {
  using namespace pf;
  if (!pool || n < 0 || max_blocks < 0 || num_layers < 0) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  const pf_geometry& g = pool->g;
  if (layer0 < 0 || layer0 + num_layers > g.num_layers) return PF_ERR_INVALID;
  if ((size_t)g.head_dim * pool->elem_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  if (n == 0) return PF_OK;
  if (!staging_host || !meta_dev || !aligned16(staging_host) || !aligned16(meta_dev)) return PF_ERR_INVALID;
  if (num_layers > 0 && (!k || !v || !aligned16(k) || !aligned16(v))) return PF_ERR_INVALID;
  PrepArgs a{};
  const int st = stage_export(pool, seq_ids, n, max_blocks, true, staging_host, meta_dev, a);
  if (st != PF_OK) return st;
  a.pool = static_cast<uint8_t*>(pool->dev);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.lens_host = staging_host + (int64_t)n * max_blocks;
  a.page_host = staging_host + (int64_t)n * max_blocks + 2 * (int64_t)n;
  a.page_elems = (int64_t)pool->page_elems;
  a.n = n;
  a.layer0 = layer0;
  a.H = g.num_kv_heads;
  a.D = g.head_dim;
  a.B = g.block_size;
  a.es = (int32_t)pool->elem_bytes;
  a.num_pages = g.num_pages;
  a.sc_threads = (int64_t)num_layers * n * g.num_kv_heads * 2 * (g.head_dim * a.es / 16);
  const int64_t blocks = (a.up_threads + a.sc_threads + 255) / 256;
  if (blocks > 0x7fffffff) {
    pf_export_forget(pool);
    return PF_ERR_INVALID;
  }
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, a);
  if (hipGetLastError() != hipSuccess) {
    pf_export_forget(pool);
    return PF_ERR_HIP;
  }
  return PF_OK;
}

extern "C" int pf_copy_pages(const pf_pool* pool, const int32_t* pairs, int32_t n, void* hip_stream) {
  if (!pool || n < 0) return PF_ERR_INVALID;
  if (!pool->dev) return PF_ERR_UNBOUND;
  if (n == 0) return PF_OK;
  if (!pairs || (reinterpret_cast<uintptr_t>(pairs) & 7) != 0) return PF_ERR_INVALID;
  const size_t page_bytes = pool->page_elems * pool->elem_bytes;
  if (page_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  const int64_t chunks = (int64_t)(page_bytes / 16);
  const int64_t total = chunks * n;
  int blocks = 0;
  if (pf::launch_grid(total, &blocks) != PF_OK) return PF_ERR_INVALID;
  hipLaunchKernelGGL(pf::copy_pages_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream,
                     static_cast<uint8_t*>(pool->dev), pairs, chunks, total, pool->g.num_pages);
  return hipGetLastError() == hipSuccess ? PF_OK : PF_ERR_HIP;
}

// Enqueue the copies of `pairs` (page, slot) / (slot, page) pairs in staging_host.
static int swap_launch(pf_pool* pool, int32_t* staging_host, int32_t pairs, bool to_host, void* hip_stream) {
  const size_t page_bytes = pool->page_elems * pool->elem_bytes;
  const int64_t chunks = (int64_t)(page_bytes / 16);
  const int64_t spans = (chunks + pf::kSwapSpan - 1) / pf::kSwapSpan;
  const int64_t units = spans * pairs;
  const int64_t blocks = units < pf::kSwapGrid ? units : pf::kSwapGrid;
  hipLaunchKernelGGL(pf::swap_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream,
                     static_cast<uint8_t*>(pool->dev), static_cast<uint8_t*>(pool->host), staging_host, chunks,
                     spans, units, pool->g.num_pages, pool->num_slots, to_host ? 1 : 0);
  return hipGetLastError() == hipSuccess ? PF_OK : PF_ERR_HIP;
}

static int swap_call(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t* staging_host,
                     int64_t staging_words, bool to_host, void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (n > 0 && (!staging_host || (reinterpret_cast<uintptr_t>(staging_host) & 7) != 0)) return PF_ERR_INVALID;
  const size_t page_bytes = pool->page_elems * pool->elem_bytes;
  if (page_bytes % 16 != 0) return PF_ERR_UNSUPPORTED;
  int32_t pairs = 0;
  const int st = pf_swap_plan(pool, seq_ids, n, to_host, staging_host, staging_words, &pairs);
  if (st != PF_OK || pairs == 0) return st;
  return swap_launch(pool, staging_host, pairs, to_host, hip_stream);
}

static int swap_blocks_call(pf_pool* pool, uint64_t seq_id, int32_t first, int32_t count, int32_t* staging_host,
                            int64_t staging_words, bool to_host, void* hip_stream) {
  if (!pool) return PF_ERR_INVALID;
  if (!staging_host || (reinterpret_cast<uintptr_t>(staging_host) & 7) != 0) return PF_ERR_INVALID;
  if ((pool->page_elems * pool->elem_bytes) % 16 != 0) return PF_ERR_UNSUPPORTED;
  int32_t pairs = 0;
  const int st = pf_swap_blocks_plan(pool, seq_id, first, count, to_host, staging_host, staging_words, &pairs);
  if (st != PF_OK || pairs == 0) return st;
  return swap_launch(pool, staging_host, pairs, to_host, hip_stream);
}

extern "C" int pf_swap_out_blocks(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks,
                                  int32_t* staging_host, int64_t staging_words, void* hip_stream) {
  return swap_blocks_call(pool, seq_id, first_block, num_blocks, staging_host, staging_words, true, hip_stream);
}

extern "C" int pf_swap_in_blocks(pf_pool* pool, uint64_t seq_id, int32_t first_block, int32_t num_blocks,
                                 int32_t* staging_host, int64_t staging_words, void* hip_stream) {
  return swap_blocks_call(pool, seq_id, first_block, num_blocks, staging_host, staging_words, false, hip_stream);
}

extern "C" int pf_swap_out(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t* staging_host,
                           int64_t staging_words, void* hip_stream) {
  return swap_call(pool, seq_ids, n, staging_host, staging_words, true, hip_stream);
}

extern "C" int pf_swap_in(pf_pool* pool, const uint64_t* seq_ids, int32_t n, int32_t* staging_host,
                          int64_t staging_words, void* hip_stream) {
  return swap_call(pool, seq_ids, n, staging_host, staging_words, false, hip_stream);
}

// ------------------------------------------------------------ stream markers
// Events without the system-scope fence: recording one adds no cache
// writeback / invalidation to the stream (a default event did, about 6 us
// between two kernels on MI355X).
extern "C" int pf_marker_create(int32_t timing, void** event) {
  if (!event) return PF_ERR_INVALID;
  *event = nullptr;
  unsigned flags = hipEventDisableSystemFence;
  if (!timing) flags |= hipEventDisableTiming;
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, flags) != hipSuccess) {
    (void)hipGetLastError();
    return PF_ERR_HIP;
  }
  *event = e;
  return PF_OK;
}

extern "C" int pf_marker_record(void* event, void* hip_stream) {
  if (!event) return PF_ERR_INVALID;
  if (hipEventRecord((hipEvent_t)event, (hipStream_t)hip_stream) != hipSuccess) {
    (void)hipGetLastError();
    return PF_ERR_HIP;
  }
  return PF_OK;
}

extern "C" int pf_marker_wait(void* event) {
  if (!event) return PF_ERR_INVALID;
  if (hipEventSynchronize((hipEvent_t)event) != hipSuccess) {
    (void)hipGetLastError();
    return PF_ERR_HIP;
  }
  return PF_OK;
}

extern "C" int pf_marker_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return PF_ERR_INVALID;
  if (hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)stop) != hipSuccess) {
    (void)hipGetLastError();
    return PF_ERR_HIP;
  }
  return PF_OK;
}

extern "C" int pf_marker_destroy(void* event) {
  if (!event) return PF_ERR_INVALID;
  if (hipEventDestroy((hipEvent_t)event) != hipSuccess) {
    (void)hipGetLastError();
    return PF_ERR_HIP;
  }
  return PF_OK;
}
