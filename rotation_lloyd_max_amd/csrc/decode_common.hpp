// Code-format constants and small helpers shared by the qmv kernel (gfx950).
//
// A lane decodes a "chunk" of one packed row: 32 elements for the bit formats (4 words at
// 4 bits, 3 words at 3 bits, 2 words at 2 bits) or one 20-trit word for the ternary
// format; Fmt<L> gives the words, elements, element pairs and table entries of a chunk.
// The lookups themselves are in qmv_decode.hpp. Element pairs: low half = even element.
#pragma once

#include "device_common.hpp"

namespace tq {

template <int L>
struct Fmt;
template <>
struct Fmt<16> { static constexpr int cw = 4, ce = 32, np = 16, entries = 256; };
template <>
struct Fmt<8> { static constexpr int cw = 3, ce = 32, np = 16, entries = 64; };
template <>
struct Fmt<4> { static constexpr int cw = 2, ce = 32, np = 16, entries = 16; };
template <>
struct Fmt<3> { static constexpr int cw = 1, ce = 20, np = 10, entries = 9; };

__device__ __forceinline__ float dot2_h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// Words of chunk c of the packed row starting `rowbyte` bytes after the expert's codes (c
// must be a valid chunk; rows are 16-byte aligned for 4-bit codes and 8-byte aligned for
// 2-bit codes because K is a multiple of 32).
template <int L>
__device__ __forceinline__ void load_chunk_words(const uint32_t* cexp, uint32_t rowbyte, int c,
                                                 uint32_t (&w)[Fmt<L>::cw]) {
  const uint32_t off = rowbyte + static_cast<uint32_t>(c) * (Fmt<L>::cw * 4);
  if constexpr (L == 16) {
    const u32x4_t v = ld_stream<u32x4_t>(cexp, off);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (L == 8) {
    const u32x3_t v = ld_stream<u32x3_t>(cexp, off);  // one 12-byte load
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (L == 4) {
    const u32x2_t v = ld_stream<u32x2_t>(cexp, off);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = ld_stream<uint32_t>(cexp, off);
  }
}

// The fp16 scales a chunk needs: .x = its first group, .y = the next group (for 16-element
// groups of the bit formats, and for trit words, which may span two groups; clamped to the
// row's last group). Each half is loaded straight into its half of the register (no
// shift or mask after the load), so nothing waits for the load before the value is used.
template <int L, bool G16>
__device__ __forceinline__ half2_t load_chunk_scales(const uint16_t* sexp, uint32_t rowbyte, int c,
                                                     int group, int ngroups) {
  half2_t r;
  if constexpr (L == 3) {
    const int g0 = (c * 20) / group;
    const int g1 = g0 + 1 < ngroups ? g0 + 1 : g0;
    r.x = ld_stream<_Float16>(sexp, rowbyte + 2 * g0);
    r.y = ld_stream<_Float16>(sexp, rowbyte + 2 * g1);
  } else if constexpr (G16) {
    r = ld_stream<half2_t>(sexp, rowbyte + 4 * c);
  } else {
    r.x = ld_stream<_Float16>(sexp, rowbyte + 2 * ((c * 32) / group));
    // .y unused (one group per chunk)
  }
  return r;
}

// Sum over a whole wave (lg = 6) without selects: the moves fold into the adds.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_plus(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
  return v + __int_as_float(moved);
}
__device__ __forceinline__ float wave_sum_to_last(float v) {
  v = dpp_plus<0xB1>(v);
  v = dpp_plus<0x4E>(v);
  v = dpp_plus<0x124>(v);
  v = dpp_plus<0x128>(v);
  v = dpp_plus<0x142, 0xA>(v);
  v = dpp_plus<0x143, 0xC>(v);
  return v;
}

// Sum of v over aligned segments of 2^lg lanes (lg = 0..6) with DPP lane moves (no LDS
// traffic); afterwards the segment's last lane holds the segment's total (row_ror moves
// data towards higher lanes: lane i receives lane (i - n) mod 16 of its row). Every step is
// done, and the moved value is dropped (a select on a uniform condition) when the step is
// beyond lg: straight-line code keeps the compiler's accounting of outstanding loads exact
// inside streaming loops.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_plus_if(float v, bool on) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
  return v + (on ? __int_as_float(moved) : 0.f);
}

__device__ __forceinline__ float segment_sum_flat(float v, int lg) {
  v = dpp_plus_if<0xB1>(v, lg >= 1);
  v = dpp_plus_if<0x4E>(v, lg >= 2);
  v = dpp_plus_if<0x124>(v, lg >= 3);
  v = dpp_plus_if<0x128>(v, lg >= 4);
  v = dpp_plus_if<0x142, 0xA>(v, lg >= 5);
  v = dpp_plus_if<0x143, 0xC>(v, lg >= 6);
  return v;
}

// Maximum of non-negative v over the wave, left in lane 63 (same lane moves as
// segment_sum; lanes without a source lane see 0, which leaves a non-negative max as is).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_max(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
  return fmaxf(v, __int_as_float(moved));
}

__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = dpp_max<0xB1>(v);
  v = dpp_max<0x4E>(v);
  v = dpp_max<0x124>(v);
  v = dpp_max<0x128>(v);
  v = dpp_max<0x142, 0xA>(v);
  v = dpp_max<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ bool seg_sum_lane(int lane, int lg) {
  const int seg = 1 << lg;
  return (lane & (seg - 1)) == seg - 1;
}

}  // namespace tq
