// Decoding packed codes straight into matrix-core operands (gfx950,
// v_mfma_f32_16x16x32_f16).
//
// For v_mfma_f32_16x16x32_f16 lane l holds A[l % 16][8 (l / 16) + j] and
// B[8 (l / 16) + j][l % 16] (j < 8) and gets D[4 (l / 16) + r][l % 16] (r < 4). Here the
// B columns are 16 output rows of a weight and the A rows are 16 inputs. The order of the
// 32 K positions inside one instruction is free as long as A and B agree, so each lane
// group g = l / 16 takes a contiguous "span" of its row: SPAN elements that it feeds to
// MF consecutive instructions, 8 elements at a time. A span is a few whole code words, so
// a lane loads and decodes its own words:
//
//   4 bits   span 32 = 4 words     fragment f = word f (4 pair lookups)
//   3 bits   span 32 = 3 words     fragment f = bits 24f .. 24f+23 (4 six-bit pair indices)
//   2 bits   span 32 = 2 words     fragment f = bytes 2f, 2f+1 (2 lookups of 4 codes)
//   trits    span 40 = 2 words     fragment f = base-81 digits 2f, 2f+1 of the span (2
//                                  lookups of 4 trits)
//
// Every fragment lies inside one scale group (groups are 16 or more elements and fragments
// start at multiples of 8), and its pairs are multiplied by that group's fp16 scale before
// the matrix multiply.
#pragma once

#include "qmv_decode.hpp"

namespace tq {


template <int L>
struct Span;
template <>
struct Span<16> { static constexpr int words = 4, elems = 32, mf = 4; };
template <>
struct Span<8> { static constexpr int words = 3, elems = 32, mf = 4; };
template <>
struct Span<4> { static constexpr int words = 2, elems = 32, mf = 4; };
template <>
struct Span<3> { static constexpr int words = 2, elems = 40, mf = 5; };

// Index of the first code word of a span starting at element e0 (a multiple of the span).
template <int L>
__device__ __forceinline__ int span_first_word(int e0) {
  if constexpr (L == 3) return e0 / 20;
  else return (e0 * (L == 16 ? 4 : L == 8 ? 3 : 2)) >> 5;
}

// Lookup tables of the matrix-core path: the qmv tables for the bit formats; for trits one
// entry per base-81 digit (4 trits, two pairs, 8 bytes), 32 copies.
template <int L>
struct MLut { static constexpr int entries = Lut<L>::entries, eb = Lut<L>::eb; };
template <>
struct MLut<3> { static constexpr int entries = 81, eb = 8; };

template <int L>
constexpr int mlut_bytes() {
  return MLut<L>::entries * 256;
}

template <int L>
__device__ __forceinline__ uint32_t mlut_slot(int lane) {
  return MLut<L>::eb == 4 ? static_cast<uint32_t>(lane & 63) * 4u
                          : static_cast<uint32_t>(lane & 31) * 8u;
}

// 32-bit word i of the table, from the fp16 centroids h.
template <int L>
__device__ __forceinline__ uint32_t mlut_word(int i, const uint16_t* h) {
  if constexpr (L != 3) {
    return lut_word<L>(i, h);
  } else {
    // entry e = t0 + 3 t1 + 9 t2 + 27 t3; word d of the entry holds trits 2d, 2d + 1
    const int e = i >> 6, d = i & 1;
    const int t01 = d ? (e / 9) % 9 : e % 9;
    const int a = t01 % 3, b = t01 / 3;
    return static_cast<uint32_t>(h[a]) | (static_cast<uint32_t>(h[b]) << 16);
  }
}

template <int L, int NT>
__device__ __forceinline__ void build_mlut(uint32_t* lut, const uint16_t* h) {
  constexpr int quads = MLut<L>::entries * 64 / 4;
#pragma unroll
  for (int k = 0; k < (quads + NT - 1) / NT; ++k) {
    const int qi = threadIdx.x + k * NT;
    if (qi < quads) {
      const uint32_t v0 = mlut_word<L>(4 * qi, h), v1 = mlut_word<L>(4 * qi + 1, h);
      reinterpret_cast<uint4*>(lut)[qi] = make_uint4(v0, v1, v0, v1);
    }
  }
}

// The five base-81 digits of a trit word v < 3^20 (each digit = 4 trits, least significant
// first), without a divide instruction: v / 6561 by a 32-bit multiply-high
// (floor(v * 2681326939 / 2^44), exact for all 32-bit v), the rest by 24-bit multiplies
// (x / 81 = (x * 6473) >> 19 for x < 6561; x / 6561 = high half of x * 654621 for
// x < 3^12), all checked exhaustively over their ranges.
__device__ __forceinline__ void trit_digits81(uint32_t v, uint32_t (&q)[5]) {
  const uint32_t hi = __umulhi(v, 2681326939u) >> 12;     // v / 6561  (< 3^12)
  const uint32_t lo = v - hi * 6561u;                      // < 6561
  const uint32_t q1 = __umul24(lo, 6473u) >> 19;           // lo / 81
  q[0] = lo - q1 * 81u;
  q[1] = q1;
  // hi / 6561 (< 81): bits 32.. of a 24 x 24-bit product (v_mul_hi_u32_u24)
  const uint32_t q4 =
      static_cast<uint32_t>((static_cast<uint64_t>(hi & 0xffffffu) * 654621ull) >> 32);
  const uint32_t r = hi - q4 * 6561u;                      // < 6561
  const uint32_t q3 = __umul24(r, 6473u) >> 19;
  q[2] = r - q3 * 81u;
  q[3] = q3;
  q[4] = q4;
}

__device__ __forceinline__ uint32_t pk_mul_h(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}

// Table indices of one span: the code words themselves for the bit formats, the ten base-81
// digits for trits (computed once per span and shared by its five fragments).
template <int L>
struct SpanIdx {
  uint32_t v[L == 3 ? 10 : Span<L>::words];
};

template <int L>
__device__ __forceinline__ void span_index(const uint32_t (&w)[Span<L>::words], SpanIdx<L>& x) {
  if constexpr (L == 3) {
    uint32_t q[5];
    trit_digits81(w[0], q);
#pragma unroll
    for (int k = 0; k < 5; ++k) x.v[k] = q[k];
    trit_digits81(w[1], q);
#pragma unroll
    for (int k = 0; k < 5; ++k) x.v[5 + k] = q[k];
  } else {
#pragma unroll
    for (int i = 0; i < Span<L>::words; ++i) x.v[i] = w[i];
  }
}

// Table entries of fragment f of a span: 8 fp16 centroids (4 pairs) of the lane's row, not
// yet scaled. f must be a compile-time constant after unrolling.
template <int L>
__device__ __forceinline__ u32x4_t span_lookup(const SpanIdx<L>& x, int f, const uint32_t* lut,
                                               uint32_t slot) {
  u32x4_t b;
  if constexpr (L == 16) {
    b[0] = lds_u32(lut, byte_addr<0>(x.v[f], slot));
    b[1] = lds_u32(lut, byte_addr<1>(x.v[f], slot));
    b[2] = lds_u32(lut, byte_addr<2>(x.v[f], slot));
    b[3] = lds_u32(lut, byte_addr<3>(x.v[f], slot));
  } else if constexpr (L == 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bit = 24 * f + 6 * j, lo = bit >> 5, sh = bit & 31;
      uint32_t fld;
      if (sh <= 26) fld = __builtin_amdgcn_ubfe(x.v[lo], sh, 6);
      else fld = __builtin_amdgcn_alignbit(x.v[lo + 1], x.v[lo], sh) & 63u;
      b[j] = lds_u32(lut, (fld << 8) | slot);
    }
  } else if constexpr (L == 4) {
    const uint32_t wf = x.v[f >> 1];
    uint2 e0, e1;
    if (f & 1) {
      e0 = lds_u64(lut, byte_addr<2>(wf, slot));
      e1 = lds_u64(lut, byte_addr<3>(wf, slot));
    } else {
      e0 = lds_u64(lut, byte_addr<0>(wf, slot));
      e1 = lds_u64(lut, byte_addr<1>(wf, slot));
    }
    b[0] = e0.x; b[1] = e0.y; b[2] = e1.x; b[3] = e1.y;
  } else {
    const uint2 e0 = lds_u64(lut, (x.v[2 * f] << 8) | slot);
    const uint2 e1 = lds_u64(lut, (x.v[2 * f + 1] << 8) | slot);
    b[0] = e0.x; b[1] = e0.y; b[2] = e1.x; b[3] = e1.y;
  }
  return b;
}

// Pairs times the fragment's fp16 scale s2 (the scale in both halves).
__device__ __forceinline__ u32x4_t scale_pairs(const u32x4_t& r, uint32_t s2) {
  u32x4_t b;
#pragma unroll
  for (int k = 0; k < 4; ++k) b[k] = pk_mul_h(r[k], s2);
  return b;
}

// B fragment f of a span: 8 fp16 weights (4 pairs) of the lane's row, multiplied by their
// scale s2.
template <int L>
__device__ __forceinline__ u32x4_t span_fragment(const SpanIdx<L>& x, int f, const uint32_t* lut,
                                                 uint32_t slot, uint32_t s2) {
  return scale_pairs(span_lookup<L>(x, f, lut, slot), s2);
}

// All MF fragments of one span; s2[f] is fragment f's fp16 scale in both halves.
template <int L>
__device__ __forceinline__ void span_fragments(const uint32_t (&w)[Span<L>::words],
                                               const uint32_t* lut, uint32_t slot,
                                               const uint32_t (&s2)[Span<L>::mf],
                                               u32x4_t (&b)[Span<L>::mf]) {
  SpanIdx<L> x;
  span_index<L>(w, x);
#pragma unroll
  for (int f = 0; f < Span<L>::mf; ++f) b[f] = span_fragment<L>(x, f, lut, slot, s2[f]);
}

__device__ __forceinline__ f32x4_t mfma_f16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

}  // namespace tq
