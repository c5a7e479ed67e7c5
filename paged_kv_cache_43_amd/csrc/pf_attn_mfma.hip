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
//    row-major tile, one per wave) so each lane can pick the four tokens x one
//    dim that the A operand of v_mfma_f32_16x16x16 wants (V^T).  Tokens past
//    the length are written to LDS as zeros (their K rows are masked to -inf).
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
  uint32_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = T::narrow_bits(p[i]);
    float back[2];
    T::widen(h[i], back);  // low half of the word holds the value
    r[i] = T::narrow_bits(p[i] - back[0]);
  }
  hi->x = h[0] | (h[1] << 16);
  hi->y = h[2] | (h[3] << 16);
  lo->x = r[0] | (r[1] << 16);
  lo->y = r[2] | (r[3] << 16);
}

template <class T, bool OUT_F32>
__device__ inline void store_vec4(void* out, int64_t idx, const float* v) {
  if constexpr (OUT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = T::narrow_bits(v[0]) | (T::narrow_bits(v[1]) << 16);
    w.y = T::narrow_bits(v[2]) | (T::narrow_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

template <class T, int D, bool OUT_F32>
__global__ __launch_bounds__(kWave) void attn_mfma_kernel(AttnArgs a) {
  constexpr int ES = 2;
  constexpr int KC = D / 32;              // 32-dim chunks of the score product
  constexpr int DB = D / 16;              // 16-dim blocks of the value product
  constexpr int VCH = D * ES / 16;        // 16-byte chunks per token row
  constexpr int VL = kBlock * VCH / kWave;  // 16-byte V loads per lane per page
  constexpr int PITCH = D * ES + 8;       // LDS row pitch in bytes (bank spread)
  __shared__ __attribute__((aligned(16))) uint8_t vt[kBlock * PITCH];

  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane % 16;   // token (K operand) / head (score columns)
  const int grp = lane / 16;   // k-group
  const int g = a.group;
  const int head = hk * g + col;  // query head of this lane's score column
  const bool head_ok = col < g;

  int ctx = a.ctx[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
  if (ctx == 0) {
    if (split == 0 && head_ok) {
      const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < DB; ++b)
        store_vec4<T, OUT_F32>(a.out, ((int64_t)s * a.hq + head) * D + 16 * b + 4 * grp, z);
    }
    return;
  }
  if (split >= nsplit) return;

  // Q^T operand: head col, dims 32c + 8*grp .. +8 (zero rows past the group)
  uint4 qop[KC];
  {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (((int64_t)s * a.hq + (head_ok ? head : 0)) * D) * ES;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + (32 * c + 8 * grp) * ES);
      qop[c] = head_ok ? v : make_uint4(0, 0, 0, 0);
    }
  }

  const int tok0 = split * a.split_tokens;
  const int tok_end = min(ctx, tok0 + a.split_tokens);
  const int pg0 = tok0 / kBlock;
  const int npg = (tok_end - tok0 + kBlock - 1) / kBlock;
  const int my_page = lane < npg ? a.bt[(int64_t)s * a.max_blocks + pg0 + lane] : -1;

  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  const int64_t head_off = ((int64_t)a.layer * a.hkv + hk) * 2 * kBlock * D;  // elements
  const float c2 = a.qscale;  // scale * log2(e)

  float m = -INFINITY;  // running max (log2 units) of head col
  float l = 0.f;        // this lane's share of the running sum
  f4 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f4{0.f, 0.f, 0.f, 0.f};

  uint4 ka[KC], va[VL], kb[KC], vb[VL];

  auto page_base = [&](int i, bool* ok) -> const uint8_t* {
    const int page = __builtin_amdgcn_readlane(my_page, i);
    *ok = (unsigned)page < (unsigned)a.num_pages;
    return pool + ((int64_t)(*ok ? page : 0) * a.page_elems + head_off) * ES;
  };
  auto load_tile = [&](const uint8_t* p, uint4* kt, uint4* vr) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      kt[c] = *reinterpret_cast<const uint4*>(p + (col * D + 32 * c + 8 * grp) * ES);
#pragma unroll
    for (int r = 0; r < VL; ++r)
      vr[r] = *reinterpret_cast<const uint4*>(p + kBlock * D * ES + (r * kWave + lane) * 16);
  };
  auto process = [&](const uint4* kt, const uint4* vr, int nvalid) {
    const bool full = nvalid >= kBlock;
    // stage V (row-major, padded rows; tokens past the length as zeros)
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int f = r * kWave + lane;
      const int tok = f / VCH;
      const int ch = f % VCH;
      uint4 v = vr[r];
      if (!full && tok >= nvalid) v = make_uint4(0, 0, 0, 0);
      uint8_t* dst = vt + tok * PITCH + ch * 16;
      *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(v.z, v.w);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // scores S^T: token 4*grp + r, head col
    f4 sc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sc = Mfma<T>::qk(kt[c], qop[c], sc);
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = sc[r] * c2;
      if (!full && 4 * grp + r >= nvalid) z[r] = -INFINITY;
    }
    float pm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    pm = fmaxf(pm, shfl_xor(pm, 16));
    pm = fmaxf(pm, shfl_xor(pm, 32));
    const float mn = fmaxf(m, pm);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[r] - mn);
    l = l * alpha + (p[0] + p[1]) + (p[2] + p[3]);
    uint2 phi, plo;
    split_pack<T>(p, &phi, &plo);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      // V^T operand: dim 16b + col, tokens 4*grp + j
      const uint8_t* src = vt + (4 * grp) * PITCH + (16 * b + col) * ES;
      const uint32_t v0 = *reinterpret_cast<const uint16_t*>(src);
      const uint32_t v1 = *reinterpret_cast<const uint16_t*>(src + PITCH);
      const uint32_t v2 = *reinterpret_cast<const uint16_t*>(src + 2 * PITCH);
      const uint32_t v3 = *reinterpret_cast<const uint16_t*>(src + 3 * PITCH);
      const uint2 vop = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
      acc[b] *= alpha;
      acc[b] = Mfma<T>::pv(vop, phi, acc[b]);
      acc[b] = Mfma<T>::pv(vop, plo, acc[b]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };
  auto nvalid_of = [&](int i) { return min(kBlock, tok_end - (pg0 + i) * kBlock); };

  bool ok_a, ok_b;
  load_tile(page_base(0, &ok_a), ka, va);
  int i = 0;
  for (; i + 2 < npg; i += 2) {
    load_tile(page_base(i + 1, &ok_b), kb, vb);
    if (ok_a) process(ka, va, kBlock);
    load_tile(page_base(i + 2, &ok_a), ka, va);
    if (ok_b) process(kb, vb, kBlock);
  }
  if (i + 1 < npg) {
    load_tile(page_base(i + 1, &ok_b), kb, vb);
    if (ok_a) process(ka, va, kBlock);
    if (ok_b) process(kb, vb, nvalid_of(i + 1));
  } else {
    if (ok_a) process(ka, va, nvalid_of(i));
  }

  // the four k-groups hold disjoint tokens of the same heads: add their sums
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (!head_ok) return;
  const int64_t row = (int64_t)s * a.hq + head;
  if (nsplit == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const float o[4] = {acc[b][0] * inv, acc[b][1] * inv, acc[b][2] * inv, acc[b][3] * inv};
      store_vec4<T, OUT_F32>(a.out, row * D + 16 * b + 4 * grp, o);
    }
  } else {
    const int64_t rec = row * a.max_splits + split;
#pragma unroll
    for (int b = 0; b < DB; ++b)
      *reinterpret_cast<float4*>(a.ws_acc + rec * D + 16 * b + 4 * grp) =
          make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    if (grp == 0) a.ws_ml[rec] = make_float2(m, l);
  }
}

bool mfma_supports(int head_dim) { return head_dim == 64 || head_dim == 128; }

template <class T>
static int launch(const AttnArgs& a, int D, hipStream_t st) {
  const dim3 grid(a.max_splits, a.hkv, a.n);
  if (D == 64) {
    if (a.out_f32) hipLaunchKernelGGL((attn_mfma_kernel<T, 64, true>), grid, dim3(kWave), 0, st, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<T, 64, false>), grid, dim3(kWave), 0, st, a);
    return PF_OK;
  }
  if (D == 128) {
    if (a.out_f32) hipLaunchKernelGGL((attn_mfma_kernel<T, 128, true>), grid, dim3(kWave), 0, st, a);
    else hipLaunchKernelGGL((attn_mfma_kernel<T, 128, false>), grid, dim3(kWave), 0, st, a);
    return PF_OK;
  }
  return PF_ERR_UNSUPPORTED;
}

int launch_mfma_f16(const AttnArgs& a, int D, hipStream_t st) { return launch<ElF16>(a, D, st); }
int launch_mfma_bf16(const AttnArgs& a, int D, hipStream_t st) { return launch<ElBF16>(a, D, st); }

}  // namespace pf
