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

template <int L>
__device__ __forceinline__ void build_lut(uint32_t* lut, const uint16_t* h) {
  for (int i = threadIdx.x; i < Fmt<L>::entries * kLutCopies; i += blockDim.x)
    lut[i] = lut_entry<L>(i / kLutCopies, h);
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

}  // namespace tq
