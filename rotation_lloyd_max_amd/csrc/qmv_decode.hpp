// Code-to-centroid lookups of the qmv kernels (gfx950).
//
// Every table entry occupies 256 bytes of LDS: 64 copies of a 4-byte entry (one fp16
// centroid pair) or 32 copies of an 8-byte entry (two pairs). A lane reads the copy of its
// own lane slot, so the 64 lookups of a wave touch 64 different banks whatever the codes,
// and the byte address of entry e for a lane is (e << 8) | slot with slot < 256. When the
// entry index is a whole byte of a code word, one v_perm_b32 builds that address from the
// code word and the slot.
//
//   4 bits: index = one byte (two codes)      256 entries x 4 bytes   64 KiB
//   3 bits: index = 6 stream bits (two codes)  64 entries x 4 bytes   16 KiB
//   2 bits: index = one byte (four codes)     256 entries x 8 bytes   64 KiB
//   trits : index = t0 + 3 t1 (two digits)      9 entries x 4 bytes  2.25 KiB
//
// Pairs follow the element order: the low half of a pair is the even element.
#pragma once

#include "decode_common.hpp"

namespace tq {

template <int L>
struct Lut;
template <>
struct Lut<16> { static constexpr int entries = 256, eb = 4; };
template <>
struct Lut<8> { static constexpr int entries = 64, eb = 4; };
template <>
struct Lut<4> { static constexpr int entries = 256, eb = 8; };
template <>
struct Lut<3> { static constexpr int entries = 9, eb = 4; };

template <int L>
constexpr int lut_bytes() {
  return Lut<L>::entries * 256;
}

// The lane's byte offset inside every entry.
template <int L>
__device__ __forceinline__ uint32_t lut_slot(int lane) {
  return Lut<L>::eb == 4 ? static_cast<uint32_t>(lane & 63) * 4u
                         : static_cast<uint32_t>(lane & 31) * 8u;
}

// 32-bit word i of the table (i < entries * 64), from the fp16 centroids h.
template <int L>
__device__ __forceinline__ uint32_t lut_word(int i, const uint16_t* h) {
  const int e = i >> 6;
  int a, b;
  if constexpr (L == 16) { a = e & 15; b = e >> 4; }
  else if constexpr (L == 8) { a = e & 7; b = e >> 3; }
  else if constexpr (L == 3) { a = e % 3; b = e / 3; }
  else {  // four 2-bit codes per entry; word d of the entry holds codes 2d and 2d + 1
    const int d = i & 1;
    a = (e >> (4 * d)) & 3;
    b = (e >> (4 * d + 2)) & 3;
  }
  return static_cast<uint32_t>(h[a]) | (static_cast<uint32_t>(h[b]) << 16);
}

// Fill the table (at LDS offset 0) with 16-byte writes; the caller synchronizes.
template <int L, int NT>
__device__ __forceinline__ void build_lut_v(uint32_t* lut, const uint16_t* h) {
  constexpr int quads = Lut<L>::entries * 64 / 4;
#pragma unroll
  for (int k = 0; k < (quads + NT - 1) / NT; ++k) {
    const int qi = threadIdx.x + k * NT;
    if (qi < quads) {
      const uint32_t v0 = lut_word<L>(4 * qi, h), v1 = lut_word<L>(4 * qi + 1, h);
      reinterpret_cast<uint4*>(lut)[qi] = make_uint4(v0, v1, v0, v1);
    }
  }
}

// The same fill by threads t = 0 .. nt - 1 of any subset of the workgroup.
template <int L>
__device__ __forceinline__ void build_lut_part(uint32_t* lut, const uint16_t* h, int t, int nt) {
  constexpr int quads = Lut<L>::entries * 64 / 4;
  for (int qi = t; qi < quads; qi += nt) {
    const uint32_t v0 = lut_word<L>(4 * qi, h), v1 = lut_word<L>(4 * qi + 1, h);
    reinterpret_cast<uint4*>(lut)[qi] = make_uint4(v0, v1, v0, v1);
  }
}

__device__ __forceinline__ uint32_t lds_u32(const uint32_t* lut, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + byte_addr);
}
__device__ __forceinline__ uint2 lds_u64(const uint32_t* lut, uint32_t byte_addr) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(lut) + byte_addr);
}

// (byte k of w) << 8 | slot, in one v_perm_b32: selector bytes pick slot byte 0, then
// byte k of w, then two zero bytes.
template <int K>
__device__ __forceinline__ uint32_t byte_addr(uint32_t w, uint32_t slot) {
  return __builtin_amdgcn_perm(w, slot, 0x0c0c0000u | ((4u + K) << 8));
}

// Table entries of one chunk: np fp16 centroid pairs, pair p = elements 2p, 2p + 1.
template <int L>
__device__ __forceinline__ void chunk_lookup(const uint32_t (&w)[Fmt<L>::cw], const uint32_t* lut,
                                             uint32_t slot, uint32_t (&cw)[Fmt<L>::np]) {
  if constexpr (L == 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cw[4 * i + 0] = lds_u32(lut, byte_addr<0>(w[i], slot));
      cw[4 * i + 1] = lds_u32(lut, byte_addr<1>(w[i], slot));
      cw[4 * i + 2] = lds_u32(lut, byte_addr<2>(w[i], slot));
      cw[4 * i + 3] = lds_u32(lut, byte_addr<3>(w[i], slot));
    }
  } else if constexpr (L == 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint2 e[4];
      e[0] = lds_u64(lut, byte_addr<0>(w[i], slot));
      e[1] = lds_u64(lut, byte_addr<1>(w[i], slot));
      e[2] = lds_u64(lut, byte_addr<2>(w[i], slot));
      e[3] = lds_u64(lut, byte_addr<3>(w[i], slot));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cw[8 * i + 2 * k] = e[k].x;
        cw[8 * i + 2 * k + 1] = e[k].y;
      }
    }
  } else if constexpr (L == 8) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int bit = 6 * p, lo = bit >> 5, sh = bit & 31;
      uint32_t f;
      if (sh <= 26) f = __builtin_amdgcn_ubfe(w[lo], sh, 6);
      else f = __builtin_amdgcn_alignbit(w[lo + 1], w[lo], sh) & 63u;
      cw[p] = lds_u32(lut, (f << 8) | slot);
    }
  } else {
    // twenty base-3 digits, least significant first; pair p = digits 2p, 2p + 1 is the
    // base-9 digit p of the word
    uint32_t v = w[0];
#pragma unroll
    for (int p = 0; p < 10; ++p) {
      const uint32_t q = v / 9u;
      const uint32_t e = v - 9u * q;
      v = q;
      cw[p] = lds_u32(lut, (e << 8) | slot);
    }
  }
}

// Pair products of one chunk's entries against the lane's rotated input pairs xp: pairs
// before pb accumulate into a0 and the rest into a1. With SPLIT (groups of 16) the split
// is after pair 8; trit words split at pb (pb = np when the word lies in one group).
template <int L, bool SPLIT>
__device__ __forceinline__ void chunk_dot_pairs(const uint32_t (&cw)[Fmt<L>::np],
                                                const uint32_t (&xp)[Fmt<L>::np], int pb,
                                                float& a0, float& a1) {
#pragma unroll
  for (int q = 0; q < Fmt<L>::np; ++q) {
    const bool second = L == 3 ? q >= pb : (SPLIT && q >= 8);
    if (second) a1 = dot2_h(cw[q], xp[q], a1);
    else a0 = dot2_h(cw[q], xp[q], a0);
  }
}

template <int L, bool SPLIT>
__device__ __forceinline__ void chunk_dot_v(const uint32_t (&w)[Fmt<L>::cw], const uint32_t* lut,
                                            uint32_t slot, const uint32_t (&xp)[Fmt<L>::np],
                                            int pb, float& a0, float& a1) {
  uint32_t cw[Fmt<L>::np];
  chunk_lookup<L>(w, lut, slot, cw);
  chunk_dot_pairs<L, SPLIT>(cw, xp, pb, a0, a1);
}

}  // namespace tq
