// Inline decoding of packed codes for the qmv family (gfx950).
//
// A lane decodes a "chunk" of one packed row: 32 elements for the bit formats (4 words at
// 4 bits, 3 words at 3 bits, 2 words at 2 bits) or one 20-trit word for the ternary
// format. Codes are turned into pairs of fp16 centroids by table lookups in LDS, two
// elements per lookup, and multiplied against pairs of the rotated input in fp16 with
// v_dot2 (fp32 accumulation). Tables are replicated 32 times, one copy per lane of a
// half-wave, so that a wave's lookups never collide in an LDS bank.
//
//   4 bits: index = one byte (two codes)         256 entries
//   3 bits: index = 6 stream bits (two codes)     64 entries
//   2 bits: index = one nibble (two codes)        16 entries
//   trits : index = t0 + 3 t1 (two digits)         9 entries
//
// The element-pair convention everywhere: low half = the even element.
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

constexpr int kLutCopies = 32;

// Table entry e as two fp16 centroids (low = even element).
template <int L>
__device__ __forceinline__ uint32_t lut_entry(int e, const uint16_t* h) {
  int a, b;
  if constexpr (L == 16) { a = e & 15; b = e >> 4; }
  else if constexpr (L == 8) { a = e & 7; b = e >> 3; }
  else if constexpr (L == 4) { a = e & 3; b = e >> 2; }
  else { a = e % 3; b = e / 3; }
  return static_cast<uint32_t>(h[a]) | (static_cast<uint32_t>(h[b]) << 16);
}

// Fill the replicated table from the fp16 centroids h (LDS); the caller synchronizes.
// The trip count is a compile-time constant, so all reads are issued before the writes.
template <int L, int NT = kBlock>
__device__ __forceinline__ void build_lut(uint32_t* lut, const uint16_t* h) {
  constexpr int total = Fmt<L>::entries * kLutCopies;
#pragma unroll
  for (int k = 0; k < (total + NT - 1) / NT; ++k) {
    const int i = threadIdx.x + k * NT;
    if (i < total) lut[i] = lut_entry<L>(i / kLutCopies, h);
  }
}

// Table indices of the np pairs of a chunk.
template <int L>
__device__ __forceinline__ void chunk_indices(const uint32_t (&w)[Fmt<L>::cw], int (&e)[Fmt<L>::np]) {
  if constexpr (L == 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) e[4 * i + k] = (w[i] >> (8 * k)) & 0xff;
  } else if constexpr (L == 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) e[8 * i + k] = (w[i] >> (4 * k)) & 0xf;
  } else if constexpr (L == 8) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int bit = 6 * p, lo = bit >> 5, sh = bit & 31;
      uint32_t v = w[lo] >> sh;
      if (sh > 26) v |= w[lo + 1] << (32 - sh);
      e[p] = v & 63;
    }
  } else {
    uint32_t v = w[0];
#pragma unroll
    for (int p = 0; p < 10; ++p) {
      const uint32_t q0 = v / 3u;
      const uint32_t t0 = v - 3u * q0;
      const uint32_t q1 = q0 / 3u;
      const uint32_t t1 = q0 - 3u * q1;
      v = q1;
      e[p] = static_cast<int>(t0 + 3u * t1);
    }
  }
}

__device__ __forceinline__ float dot2_h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

// Words of chunk c of a packed row (c must be a valid chunk; rows are 16-byte aligned for
// 4-bit codes and 8-byte aligned for 2-bit codes because K is a multiple of 32).
template <int L>
__device__ __forceinline__ void load_chunk_words(const uint32_t* crow, int c, uint32_t (&w)[Fmt<L>::cw]) {
  const uint32_t* p = crow + c * Fmt<L>::cw;
  if constexpr (L == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (L == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < Fmt<L>::cw; ++i) w[i] = p[i];
  }
}

// The fp16 scales a chunk needs: .x = its first group, .y = the next group (for 16-element
// groups of the bit formats, and for trit words, which may span two groups; clamped to the
// row's last group). Each half is loaded straight into its half of the register (no
// shift or mask after the load), so nothing waits for the load before the value is used.
template <int L, bool G16>
__device__ __forceinline__ half2_t load_chunk_scales(const uint16_t* srow, int c, int group, int ngroups) {
  const _Float16* sh = reinterpret_cast<const _Float16*>(srow);
  half2_t r;
  if constexpr (L == 3) {
    const int g0 = (c * 20) / group;
    const int g1 = g0 + 1 < ngroups ? g0 + 1 : g0;
    r.x = sh[g0];
    r.y = sh[g1];
  } else if constexpr (G16) {
    r = *reinterpret_cast<const half2_t*>(sh + 2 * c);
  } else {
    r.x = sh[(c * 32) / group];
    // .y unused (one group per chunk)
  }
  return r;
}

// Sum over a chunk of c[idx] * x' with x' pairs in registers, split at pair pb.
template <int L>
__device__ __forceinline__ void chunk_dot_regs(const uint32_t (&w)[Fmt<L>::cw], const uint32_t* lut,
                                               int lane31, const uint32_t (&xp)[Fmt<L>::np], int pb,
                                               float& a0, float& a1) {
  int e[Fmt<L>::np];
  chunk_indices<L>(w, e);
#pragma unroll
  for (int q = 0; q < Fmt<L>::np; ++q) {
    const uint32_t cw = lut[e[q] * kLutCopies + lane31];
    if (q < pb) a0 = dot2_h(cw, xp[q], a0);
    else a1 = dot2_h(cw, xp[q], a1);
  }
}

// Sum of v over aligned segments of 2^lg lanes (lg = 0..6) with DPP lane moves (no LDS
// traffic). Afterwards the segment's last lane holds the segment's total (row_ror moves
// data towards higher lanes: lane i receives lane (i - n) mod 16 of its row).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_plus(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false);
  return v + __int_as_float(moved);
}

// segment_sum without branches: every step is done, and the moved value is dropped (a
// select on a uniform condition) when the step is beyond lg. Straight-line code keeps the
// compiler's accounting of outstanding loads exact inside streaming loops.
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

__device__ __forceinline__ float segment_sum(float v, int lg) {
  if (lg >= 1) v = dpp_plus<0xB1>(v);        // quad_perm [1,0,3,2]: partner lane ^ 1
  if (lg >= 2) v = dpp_plus<0x4E>(v);        // quad_perm [2,3,0,1]: partner lane ^ 2
  if (lg >= 3) v = dpp_plus<0x124>(v);       // row_ror:4: quads q and q+1 of the row
  if (lg >= 4) v = dpp_plus<0x128>(v);       // row_ror:8: whole 16-lane row
  if (lg >= 5) v = dpp_plus<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (lg >= 6) v = dpp_plus<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
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
