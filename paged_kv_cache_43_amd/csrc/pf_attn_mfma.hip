// Matrix-core decode attention for grouped query heads (16-bit K/V, head dim
// 64 or 128, 2..16 query heads per kv head).
//
// With g query heads sharing one kv head, a page's scores for the whole group
// are a small dense product, S^T[16 tokens x 16 heads] = K[16 x D] Q^T[D x 16],
// and the value update is O^T[D x 16] += V^T[D x 16 tokens] P^T[16 x 16].
// Both run on MFMA: K and V are read from HBM once per kv head instead of once
// per query head (the vector kernel's cost), and the group's rows beyond g are
// zero padding.  The softmax is the same online, log2-unit, fp32 recurrence as
// the vector kernel (PagedAttention blog, "The Attention Kernel").
//
// One wave per (sequence, kv head, context split).  Per page:
//  * K: each lane loads 16 contiguous bytes (token lane%16, dims 8*(lane/16)+
//    32c..) -- exactly the A operand of v_mfma_f32_16x16x32 -- straight from
//    HBM into registers.
//  * V: loaded with 16-byte coalesced loads and staged through LDS (a padded
//    row-major tile, one per wave); one transposing LDS read (ds_read_b64_tr_b16)
//    per 16-dim block gives each lane the four tokens x one dim that the A
//    operand of v_mfma_f32_16x16x16 wants (V^T).  Tokens past the length are
//    written to LDS as zeros (their K rows are masked to -inf).
//  * The score accumulator puts tokens 4*(lane/16)+r of head lane%16 in each
//    lane, which is exactly the B operand layout (P^T) of the value product,
//    so probabilities never leave registers.  They are split into a 16-bit
//    high part and a 16-bit remainder and both are multiplied, which keeps the
//    probabilities to about 16 significant bits instead of 8.
//  * The next page's K and V loads are issued before the current page is used.
#include <cmath>

#include "pf_attn.h"
#include "pf_common.h"
#include "pf_internal.h"
#include "pf_sched.h"

namespace pf {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

template <class T>
struct Mfma;

template <>
struct Mfma<ElBF16> {
  __device__ static inline f4 qk(const uint4& a, const uint4& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c,
                                                   0, 0, 0);
  }
  __device__ static inline f4 pv(const uint2& a, const uint2& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c,
                                                     0, 0, 0);
  }
};

template <>
struct Mfma<ElF16> {
  __device__ static inline f4 qk(const uint4& a, const uint4& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0,
                                                  0, 0);
  }
  __device__ static inline f4 pv(const uint2& a, const uint2& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), c, 0,
                                                 0, 0);
  }
};

// fp32 -> (high, remainder) 16-bit patterns of type T, packed two per word.
template <class T>
__device__ inline void split_pack(const float* p, uint2* hi, uint2* lo) {
  hi->x = T::narrow2(p[0], p[1]);
  hi->y = T::narrow2(p[2], p[3]);
  float b[4];
  T::widen(hi->x, b);
  T::widen(hi->y, b + 2);
  lo->x = T::narrow2(p[0] - b[0], p[1] - b[1]);
  lo->y = T::narrow2(p[2] - b[2], p[3] - b[3]);
}

template <class T, bool OUT_F32>
__device__ inline void store_vec4(void* out, int64_t idx, const float* v) {
  if constexpr (OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = T::narrow2(v[0], v[1]);
    w.y = T::narrow2(v[2], v[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// Per-wave state of the matrix-core kernel: the current piece's online
// softmax for the 16 score columns (query heads of one kv head, padded).
// CONTIG: blocks come from a contiguous cache instead of pool pages.  BS: the
// pool's tokens per page.  The walk is in 16-token tiles: a 32- or 64-token
// page is two or four tiles, and a tile of 8-token pages spans two pages
// (rows 0..7 from the first, 8..15 from the second).
template <class T, int D, bool OUT_F32, bool CONTIG, int BS = kBlock>
struct MfmaWave {
  static_assert(BS == 8 || BS % kBlock == 0, "block size");
  static constexpr int UT = kBlock;                 // tokens per unit of the walk
  static constexpr int kPPU = BS < kBlock ? kBlock / BS : 1;  // pages per unit
  static constexpr int kUPP = BS < kBlock ? 1 : BS / kBlock;  // units per page
  static_assert(kPPU == 1 || kPPU == 2, "pages per tile");
  static constexpr int ES = 2;
  static constexpr int KC = D / 32;                // 32-dim chunks of the score product
  static constexpr int DB = D / 16;                // 16-dim blocks of the value product
  static constexpr int VCH = D * ES / 16;          // 16-byte chunks per token row
  static constexpr int VL = kBlock * VCH / kWave;  // 16-byte V loads per lane per page
  // LDS row pitch in bytes: 16-byte aligned rows, and a pitch of 8 (mod 32)
  // dwords so the transposed reads of one 16-lane group hit 32 distinct banks.
  static constexpr int PITCH = D * ES + 32;
  static constexpr int TILE_BYTES = kBlock * PITCH;
  struct Tile {
    uint4 k[KC];
    uint4 v[VL];
    uint32_t okm;  // two pages per tile: bit 0 first page valid, bit 1 second
  };
  const AttnArgs& a;
  uint8_t* vt;  // this wave's V staging tile in LDS
  const int lane, col, grp;
  const bool head_ok;
  uint4 qop[KC];
  uint4 qnx[KC];  // the next item's Q^T operand, loaded ahead (prefetch)
  int64_t qn_key = -1;
  float m, l;  // running max (log2 units) of head col; this lane's share of the sum
  f4 acc[DB];

  __device__ MfmaWave(const AttnArgs& args, uint8_t* stage, int ln)
      : a(args), vt(stage), lane(ln), col(ln % 16), grp(ln / 16), head_ok(ln % 16 < args.group) {}

  static constexpr bool kContig = CONTIG;

  // The Q^T operand of (sequence s, kv head hk): head col, dims 32c + 8*grp
  // .. +8; zero rows past the group.
  __device__ inline void load_q(int s, int hk, uint4* dst) const {
    const int head = hk * a.group + col;
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (((int64_t)s * a.hq + (head_ok ? head : 0)) * D) * ES;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + (32 * c + 8 * grp) * ES);
      dst[c] = head_ok ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // Issue the loads of the item that follows in this wave's stream, so that
  // its begin() finds q in registers: a begin() that loads q waits behind
  // every page load in flight and drains the page pipeline (measured: waves
  // that switch item mid-slice finished 2.3 us later).  key = s * items + hk.
  __device__ inline void prefetch(int s, int hk, int64_t key) {
    load_q(s, hk, qnx);
    qn_key = key;
  }

  // Start a piece of (sequence s, kv head hk), item key (or -1): q and an
  // empty state.
  __device__ inline void begin(int s, int hk, int64_t key = -1) {
    if (key >= 0 && key == qn_key) {
#pragma unroll
      for (int c = 0; c < KC; ++c) qop[c] = qnx[c];
    } else {
      load_q(s, hk, qop);
    }
    // Pin q in registers, complete, here: begin() runs on a rarely taken
    // branch inside the page loop.  Left alone, the compiler re-loads q at
    // every page (or leaves the load pending where the branch rejoins), and
    // each page then waits for all outstanding loads, prefetch included.
#pragma unroll
    for (int c = 0; c < KC; ++c)
      asm volatile("" : "+v"(qop[c].x), "+v"(qop[c].y), "+v"(qop[c].z), "+v"(qop[c].w));
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // Issue the loads of block p of sequence s (pool page `page`) for kv head
  // hk: K as score-product operands, V as 16-byte coalesced chunks.  False if
  // the table entry is not a valid page (page 0 is read instead, in bounds).
  __device__ inline bool load(int page, int s, int p, int hk, Tile& t) const {
    const BlockAddr b = block_addr<CONTIG, D, ES, BS>(a, page, s, p, hk);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      t.k[c] = load16_stream(b.k + col * b.tok + (32 * c + 8 * grp) * ES);
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int f = r * kWave + lane;  // token f / VCH, 16-byte chunk f % VCH
      t.v[r] = load16_stream(b.v + (f / VCH) * b.tok + (f % VCH) * 16);
    }
    return b.ok;
  }

  // The same for a tile of two 8-token pages (first, second; an entry that is
  // not a valid page reads page 0, in bounds, and its rows are masked).
  __device__ inline bool load2(int page0, int page1, int s, int hk, Tile& t) const {
    const BlockAddr b0 = block_addr<CONTIG, D, ES, BS>(a, page0, s, 0, hk);
    const BlockAddr b1 = block_addr<CONTIG, D, ES, BS>(a, page1, s, 0, hk);
    const uint8_t* kb = (col < BS ? b0.k : b1.k) + (col % BS) * b0.tok;
#pragma unroll
    for (int c = 0; c < KC; ++c) t.k[c] = load16_stream(kb + (32 * c + 8 * grp) * ES);
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int f = r * kWave + lane;
      const int tok = f / VCH;
      t.v[r] = load16_stream((tok < BS ? b0.v : b1.v) + (tok % BS) * b0.tok + (f % VCH) * 16);
    }
    t.okm = (b0.ok ? 1u : 0u) | (b1.ok ? 2u : 0u);
    return b0.ok || b1.ok;
  }

  // One tile: nvalid of its 16 tokens are below the length (and, for two
  // pages per tile, in a valid page).
  __device__ inline void page(const Tile& t, int nvalid) {
    bool lo_ok = true, hi_ok = true;
    if constexpr (kPPU == 2) {
      lo_ok = (t.okm & 1u) != 0;
      hi_ok = (t.okm & 2u) != 0;
      if (!((lo_ok && nvalid > 0) || (hi_ok && nvalid > BS))) return;  // nothing valid
    }
    const bool full = nvalid >= kBlock && lo_ok && hi_ok;
    auto tok_ok = [&](int tok) { return tok < nvalid && (tok < BS ? lo_ok : hi_ok); };
    // stage V (row-major, padded rows; tokens past the length as zeros)
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int f = r * kWave + lane;
      const int tok = f / VCH;
      const int ch = f % VCH;
      uint4 v = t.v[r];
      if (!full && !tok_ok(tok)) v = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(vt + tok * PITCH + ch * 16) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // scores S^T: token 4*grp + r, head col
    f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sc = Mfma<T>::qk(t.k[c], qop[c], sc);
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = sc[r] * a.qscale;
      if (!full && !tok_ok(4 * grp + r)) z[r] = -INFINITY;
    }
    // The reference max m moves only when some score exceeds it by more than
    // 8 (log2 units): probabilities then stay below 2^8, and the cross-group
    // max and the rescale are skipped for most pages.
    const float lim = m + 8.f;
    const bool over = (z[0] > lim) | (z[1] > lim) | (z[2] > lim) | (z[3] > lim);
    if (__builtin_amdgcn_ballot_w64(over)) {
      float pm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      pm = xor16<OpMax>(pm);
      pm = xor32<OpMax>(pm);
      const float mn = fmaxf(m, pm);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[r] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    uint2 phi, plo;
    split_pack<T>(p, &phi, &plo);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // V^T operands with transposed LDS reads: in each 16-lane group, lane i
    // receives element i%4 of the 8-byte chunk addressed by lane 4k + i/4
    // (k = 0..3), so lane 4k + m points at row 4*grp + k, dims 16b + 4m.., and
    // lane col ends up with dim 16b + col of tokens 4*grp .. 4*grp + 3.
    const uint8_t* tsrc = vt + (4 * grp + col / 4) * PITCH + (4 * (col % 4)) * ES;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const s4 vv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(tsrc + 16 * b * ES));
      const uint2 vop = __builtin_bit_cast(uint2, vv);
      acc[b] = Mfma<T>::pv(vop, phi, acc[b]);
      acc[b] = Mfma<T>::pv(vop, plo, acc[b]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }

  // Before page() of the sequence's last tile (row nvalid-1 is its newest
  // token), in pool page `page` (ok: a valid page).  With a fused append the
  // newest token's K/V come from the input instead of the pool, patched into
  // the tile, and this wave (the only one for this kv head) writes them into
  // the page (16-token pages only).
  __device__ inline void patch_last(Tile& u, int nvalid, int s, int hk, int page, bool ok, int unit = 0) {
    (void)unit;  // 16-token units: the newest token's row is its slot
    if (a.k_new == nullptr || !ok) return;
    const int tn = nvalid - 1;
    const int64_t row = ((int64_t)s * a.hkv + hk) * D * ES;
    uint8_t* pbase = const_cast<uint8_t*>(static_cast<const uint8_t*>(a.pool)) +
                     ((int64_t)page * a.page_elems + ((int64_t)a.layer * a.hkv + hk) * 2 * BS * D +
                      (int64_t)tn * D) * ES;
    if (col == tn) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int64_t off = (32 * c + 8 * grp) * ES;
        u.k[c] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.k_new) + row + off);
        *reinterpret_cast<uint4*>(pbase + off) = u.k[c];
      }
    }
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int f = r * kWave + lane;
      if (f / VCH == tn) {
        const int64_t off = (f % VCH) * 16;
        u.v[r] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.v_new) + row + off);
        *reinterpret_cast<uint4*>(pbase + (int64_t)BS * D * ES + off) = u.v[r];
      }
    }
  }

  // Balanced schedule: items are kv heads; slot k holds the group's records
  // k * group .. k * group + group - 1.
  __device__ inline void finish_slot(int s, int hk, bool whole, int64_t slot) {
    finish(s, hk, whole, slot * a.group, 1);
  }

  // Close the piece of (sequence s, kv head hk): the group's final outputs if
  // the piece is the whole context, else the partial record rec_base +
  // col * rec_mul of each query head.
  __device__ inline void finish(int s, int hk, bool whole, int64_t rec_base, int64_t rec_mul) {
    // the four k-groups hold disjoint tokens of the same heads: add their sums
    l = xor16<OpSum>(l);
    l = xor32<OpSum>(l);
    if (!head_ok) return;
    const int64_t row = (int64_t)s * a.hq + hk * a.group + col;
    if (whole) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const float o[4] = {acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv, acc[b][3] * inv};
        store_vec4<T, OUT_F32>(a.out, row * D + 16 * b + 4 * grp, o);
      }
    } else {
      const int64_t rec = rec_base + col * rec_mul;
#pragma unroll
      for (int b = 0; b < DB; ++b)
        *reinterpret_cast<float4*>(a.ws_acc + rec * D + 16 * b + 4 * grp) =
            make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
      if (grp == 0) a.ws_ml[rec] = make_float2(m, l);
    }
  }
};

// Grid schedule: one wave per (split, kv head, sequence).
template <class T, int D, int U, bool OUT_F32, bool CONTIG>
__global__ __launch_bounds__(kWave) void attn_mfma_grid(AttnArgs a) {
  using Wv = MfmaWave<T, D, OUT_F32, CONTIG>;
  using Tile = typename Wv::Tile;
  __shared__ __attribute__((aligned(16))) uint8_t vt[Wv::TILE_BYTES];
  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int split_pages = a.split_tokens / kBlock;
  const int pg0 = split * split_pages;
  int my_page = -1;
  if constexpr (!CONTIG)
    if (lane < split_pages && pg0 + lane < a.max_blocks) my_page = a.bt[(int64_t)s * a.max_blocks + pg0 + lane];
  const int ctx = clamp_ctx(a.ctx[s], a.max_ctx);
  const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
  Wv w(a, vt, lane);
  if (ctx == 0) {
    if (split == 0 && w.head_ok) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < Wv::DB; ++b)
        store_vec4<T, OUT_F32>(a.out, ((int64_t)s * a.hq + hk * a.group + w.col) * D + 16 * b + 4 * w.grp, z);
    }
    return;
  }
  if (split >= nsplit) return;
  const int tok_end = min(ctx, (split + 1) * a.split_tokens);
  const int npg = (tok_end - split * a.split_tokens + kBlock - 1) / kBlock;
  w.begin(s, hk);
  page_pipeline<U, Tile>(
      npg, [&](int i, Tile& t) { return w.load(__builtin_amdgcn_readlane(my_page, i), s, pg0 + i, hk, t); },
      [&](int i, Tile& t, bool ok) {
        const int nv = min(kBlock, tok_end - (pg0 + i) * kBlock);
        if (pg0 + i == (ctx - 1) / kBlock) w.patch_last(t, nv, s, hk, __builtin_amdgcn_readlane(my_page, i), ok);
        if (ok) w.page(t, nv);
      });
  w.finish(s, hk, nsplit == 1, ((int64_t)s * a.hq + hk * a.group) * a.max_splits + split, a.max_splits);
}

// Balanced schedule (pf_sched.h): four waves per workgroup, items are kv
// heads (each covering its group of query heads).
template <class T, int D, int U, bool OUT_F32, bool CONTIG, int BS = kBlock>
__global__ __launch_bounds__(kSchedThreads) void attn_mfma_balanced(AttnArgs a) {
  using Wv = MfmaWave<T, D, OUT_F32, CONTIG, BS>;
  __shared__ SchedLds L;
  __shared__ __attribute__((aligned(16))) uint8_t vt[kSchedThreads / kWave][Wv::TILE_BYTES];
  sched_build<Wv::UT>(a, L);
  if (blockIdx.x == 0) {  // zero rows of empty sequences: one thread per sequence
    const int64_t row_elems = (int64_t)a.hq * D;
    for (int s0 = threadIdx.x; s0 < a.n; s0 += kSchedThreads) {
      if (L.ctx[s0] != 0) continue;
      for (int64_t e = 0; e < row_elems; ++e) {
        if constexpr (OUT_F32) static_cast<float*>(a.out)[s0 * row_elems + e] = 0.f;
        else static_cast<uint16_t*>(a.out)[s0 * row_elems + e] = 0;
      }
    }
  }
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  Wv w(a, vt[wave], lane);
  sched_run<U, BS>(a, L, a.hkv, w, lane);
}

bool mfma_supports(int head_dim) { return head_dim == 64 || head_dim == 128; }

// One page per prefetch unit (two pages in flight per wave): measured at least
// as fast as two- or three-page units and as a ring of three one-page tiles on
// MI355X, all at the same two waves per SIMD.
template <class T, int D, bool OUT_F32, bool CONTIG>
static void launch_d(const AttnArgs& a, bool balanced, hipStream_t st) {
  if (balanced)
    hipLaunchKernelGGL((attn_mfma_balanced<T, D, 1, OUT_F32, CONTIG>), dim3(a.waves / (kSchedThreads / kWave)),
                       dim3(kSchedThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_grid<T, D, 1, OUT_F32, CONTIG>), dim3(a.max_splits, a.hkv, a.n), dim3(kWave), 0,
                       st, a);
}

template <class T, int D, bool CONTIG>
static void launch_o(const AttnArgs& a, bool balanced, hipStream_t st) {
  if (a.out_f32) launch_d<T, D, true, CONTIG>(a, balanced, st);
  else launch_d<T, D, false, CONTIG>(a, balanced, st);
}

template <class T>
static int launch_t(const AttnArgs& a, int D, bool balanced, bool contig, hipStream_t st) {
  if (D == 64) {
    if (contig) launch_o<T, 64, true>(a, balanced, st);
    else launch_o<T, 64, false>(a, balanced, st);
    return PF_OK;
  }
  if (D == 128) {
    if (contig) launch_o<T, 128, true>(a, balanced, st);
    else launch_o<T, 128, false>(a, balanced, st);
    return PF_OK;
  }
  return PF_ERR_UNSUPPORTED;
}

int launch_mfma(const AttnArgs& a, int dtype, int head_dim, bool balanced, bool contig, hipStream_t st) {
  return dtype == PF_F16 ? launch_t<ElF16>(a, head_dim, balanced, contig, st)
                         : launch_t<ElBF16>(a, head_dim, balanced, contig, st);
}

template <class T, int D, bool OUT_F32>
static int launch_bs_d(const AttnArgs& a, int bs, hipStream_t st) {
  const dim3 grid(a.waves / (kSchedThreads / kWave));
  switch (bs) {
    case 8: hipLaunchKernelGGL((attn_mfma_balanced<T, D, 1, OUT_F32, false, 8>), grid, dim3(kSchedThreads), 0, st, a); return PF_OK;
    case 32: hipLaunchKernelGGL((attn_mfma_balanced<T, D, 1, OUT_F32, false, 32>), grid, dim3(kSchedThreads), 0, st, a); return PF_OK;
    case 64: hipLaunchKernelGGL((attn_mfma_balanced<T, D, 1, OUT_F32, false, 64>), grid, dim3(kSchedThreads), 0, st, a); return PF_OK;
    default: return PF_ERR_UNSUPPORTED;
  }
}

template <class T>
static int launch_bs_t(const AttnArgs& a, int D, int bs, hipStream_t st) {
  if (D == 64) return a.out_f32 ? launch_bs_d<T, 64, true>(a, bs, st) : launch_bs_d<T, 64, false>(a, bs, st);
  if (D == 128) return a.out_f32 ? launch_bs_d<T, 128, true>(a, bs, st) : launch_bs_d<T, 128, false>(a, bs, st);
  return PF_ERR_UNSUPPORTED;
}

int launch_mfma_bs(const AttnArgs& a, int dtype, int head_dim, int block_size, hipStream_t st) {
  return dtype == PF_F16 ? launch_bs_t<ElF16>(a, head_dim, block_size, st)
                         : launch_bs_t<ElBF16>(a, head_dim, block_size, st);
}

const void* mfma_balanced_kernel(int dtype, int head_dim) {
  if (head_dim == 64)
    return dtype == PF_F16 ? reinterpret_cast<const void*>(&attn_mfma_balanced<ElF16, 64, 1, false, false>)
                           : reinterpret_cast<const void*>(&attn_mfma_balanced<ElBF16, 64, 1, false, false>);
  if (head_dim == 128)
    return dtype == PF_F16 ? reinterpret_cast<const void*>(&attn_mfma_balanced<ElF16, 128, 1, false, false>)
                           : reinterpret_cast<const void*>(&attn_mfma_balanced<ElBF16, 128, 1, false, false>);
  return nullptr;
}

}  // namespace pf
