// Device helpers shared by the libpf kernels: element types, raw vector loads,
// wave64 cross-lane reductions.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pf {

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per page of the default build (grid schedule, contiguous twin)

// The attention kernels walk a sequence in units of at most 16 tokens: a
// 16-token page is one unit, a 32- or 64-token page two or four (one table
// entry, rows offset inside the page), an 8-token page one 8-token unit.
// UTO > 0 sets the unit size instead (fp32 K/V at head dim 256 walks 16-token
// pages in 8-token units: a 16-token unit is 128 VGPRs of K/V per lane there,
// too many for two in flight).
template <int BS, int UTO = 0>
struct BlockUnits {
  static constexpr int UT = UTO > 0 ? UTO : (BS < 16 ? BS : 16);  // tokens per unit
  static constexpr int R = BS / UT;                                // units per page
  static_assert(UT * R == BS && (BS == 8 || BS % 16 == 0), "block size");
};
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- elements
// Stored element types.  Values are handled as raw bit patterns in 32-bit
// words and widened to fp32 for arithmetic.
struct ElF32 {
  static constexpr int es = 4;
  static constexpr int per_word = 1;
  __device__ static inline void widen(uint32_t w, float* o) { o[0] = __uint_as_float(w); }
  __device__ static inline uint32_t narrow_bits(float f) { return __float_as_uint(f); }
};

struct ElF16 {
  static constexpr int es = 2;
  static constexpr int per_word = 2;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  __device__ static inline void widen(uint32_t w, float* o) {
    f2 f = __builtin_convertvector(__builtin_bit_cast(h2, w), f2);
    o[0] = f.x;
    o[1] = f.y;
  }
  __device__ static inline uint32_t narrow_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
  __device__ static inline uint32_t narrow2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
  }
};

struct ElBF16 {
  static constexpr int es = 2;
  static constexpr int per_word = 2;
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  __device__ static inline void widen(uint32_t w, float* o) {
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xffff0000u);
  }
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  __device__ static inline uint32_t narrow_bits(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }
  __device__ static inline uint32_t narrow2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, b2));
  }
};

// ------------------------------------------------------------------ loads
template <int NW>
struct Raw {
  uint32_t w[NW];
};

// Loads of K/V that is read once per launch carry the non-temporal hint: on
// MI355X streaming the pool this way ran the attention kernels 11 % faster
// (13B-style: 261 -> 235 us; GQA: 70 -> 63 us, cache flushed) than plain
// loads, which keep the lines in L2 and the MALL for no reuse.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int NW>
__device__ inline Raw<NW> load_raw(const void* p) {
  Raw<NW> r;
  if constexpr (NW == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (NW == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    static_assert(NW == 1, "load width");
    r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  return r;
}

// ------------------------------------------------------- cross-lane moves
// DPP controls (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor = 0x120;     // + amount (1..15)

template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// v op v[lane ^ 16] and v op v[lane ^ 32] with gfx950's lane swaps:
// v_permlane16_swap / v_permlane32_swap of v with itself leave the pair
// {v[lane & ~16], v[lane | 16]} (resp. 32) in every lane, a VALU operation,
// where a shuffle across 16-lane rows is a ds_bpermute round trip through the
// LDS crossbar.  + and max are commutative, so the result is the shuffle's
// bit for bit (checked on the hardware: lane layout as stated).
template <class Op>
__device__ inline float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class Op>
__device__ inline float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct OpSum {
  __device__ static inline float f(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ static inline float f(float a, float b) { return fmaxf(a, b); }
};

// All-reduce over aligned groups of G consecutive lanes (G a power of two <= 64).
template <int G, class Op>
__device__ inline float group_reduce(float v) {
  if constexpr (G >= 2) v = Op::f(v, dpp<kDppXor1>(v));
  if constexpr (G >= 4) v = Op::f(v, dpp<kDppXor2>(v));
  if constexpr (G >= 8) v = Op::f(v, dpp<kDppRowHalfMirror>(v));
  if constexpr (G >= 16) v = Op::f(v, dpp<kDppRowMirror>(v));
  if constexpr (G >= 32) v = xor16<Op>(v);
  if constexpr (G >= 64) v = xor32<Op>(v);
  return v;
}

// All-reduce over the lanes that share (lane % G): strides G, 2G, ..., 32.
template <int G, class Op>
__device__ inline float strided_reduce(float v) {
  if constexpr (G <= 1) v = Op::f(v, dpp<kDppRowRor + 1>(v));
  if constexpr (G <= 2) v = Op::f(v, dpp<kDppRowRor + 2>(v));
  if constexpr (G <= 4) v = Op::f(v, dpp<kDppRowRor + 4>(v));
  if constexpr (G <= 8) v = Op::f(v, dpp<kDppRowRor + 8>(v));
  if constexpr (G <= 16) v = xor16<Op>(v);
  if constexpr (G <= 32) v = xor32<Op>(v);
  return v;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Streams npg pages through registers, U pages per unit, two units in flight:
// the next unit's loads are issued before the current unit is used.  The
// steady-state loop issues its prefetch unconditionally (so the compiler's
// memory-counter waits only cover the unit being used); the last one or two
// units are peeled.  load(i, tile) issues the loads of page i and returns
// whether page i's table entry is a valid page; pages past npg load page
// npg-1 again and are not used.  proc(i, tile, ok) is called for every page
// in order and may modify the tile (it is not used afterwards).
template <int U, class Tile, class LoadF, class ProcF>
__device__ inline void page_pipeline(int npg, LoadF&& load, ProcF&& proc) {
  Tile ta[U], tb[U];
  bool oka[U], okb[U];
  auto load_unit = [&](int j, Tile* t, bool* ok) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = j * U + u;
      ok[u] = load(i < npg ? i : npg - 1, t[u]);
    }
  };
  auto proc_unit = [&](int j, Tile* t, const bool* ok) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j * U + u < npg) proc(j * U + u, t[u], ok[u]);
  };
  const int nu = (npg + U - 1) / U;
  load_unit(0, ta, oka);
  int j = 0;
  for (; j + 2 < nu; j += 2) {
    load_unit(j + 1, tb, okb);
    proc_unit(j, ta, oka);
    load_unit(j + 2, ta, oka);
    proc_unit(j + 1, tb, okb);
  }
  if (j + 1 < nu) {
    load_unit(j + 1, tb, okb);
    proc_unit(j, ta, oka);
    proc_unit(j + 1, tb, okb);
  } else {
    proc_unit(j, ta, oka);
  }
}

}  // namespace pf
