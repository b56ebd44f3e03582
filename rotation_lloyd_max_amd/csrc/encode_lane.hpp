// Pieces shared by the register encode kernels (encode_p2.hip, encode_m.hip): butterflies
// on a lane's 32 fp64 values, lane exchanges, and the per-lane tail of the encode (group
// RMS -> fp16 scale -> snap -> packed words) for a lane that holds 32 consecutive elements
// of one row.
//
// turboquant-mlx "How it works", "Quantizing a weight, with no data"; "The ternary tier
// (1.58 bits)": r = sqrt(mean_g v^2) over the unnormalized rotated group,
// scale = fp16(r / sqrt(K)), u = v / r (0 when r = 0), idx = #{k : u > t_k} decided in
// binary32.
#pragma once

#include "device_common.hpp"

namespace tq {

// Orders a wave's LDS writes before its later LDS reads (other lanes' data): the LDS
// executes one wave's instructions in order, so only the compiler has to be held back.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Butterfly stage on register index bit S of a lane's 32 values (Sylvester order: the lower
// element gets a + b, the upper a - b).
template <int S>
__device__ __forceinline__ void bfly(double (&v)[32]) {
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    if (j & (1 << S)) continue;
    const double a = v[j], b = v[j | (1 << S)];
    v[j] = a + b;
    v[j | (1 << S)] = a - b;
  }
}

// x of the lane M apart (M = 1, 2: DPP quad permutations; M = 8: row rotation by 8, which
// is lane ^ 8 inside each row of 16 lanes), as two 32-bit moves.
template <int M>
__device__ __forceinline__ double lane_xor(double x) {
  constexpr int ctrl = M == 1 ? 0xB1 : M == 2 ? 0x4E : 0x128;
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), ctrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), ctrl, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Bits per code of a bit format (8 for trits: one digit per byte, packed later).
template <int LEVELS>
constexpr int lane_code_bits() {
  return LEVELS == 4 ? 2 : LEVELS == 8 ? 3 : LEVELS == 16 ? 4 : 8;
}

// The encode of a lane's 32 consecutive transformed elements v (elements off .. off + 31 of
// row `row`; off a multiple of 32, and a group of 64 or 128 elements held by 2 or 4
// adjacent lanes of a DPP quad). Stores the fp16 scales of the lane's groups (if live; one
// lane per group) and returns the 32 codes packed into w (BITS words; one byte per code for
// trits). tbits: positive decision thresholds as binary32 bits, ascending (symmetric
// codebook); tk: the 127 positive thresholds of the 256-level codebook (LDS).
template <int LEVELS, int LG_G>
__device__ __forceinline__ void lane_encode(const double (&v)[32], const uint32_t* tbits,
                                            const uint32_t* tk, double inv_sqrt_k, int lane,
                                            int64_t row, int off, bool live, int K,
                                            uint16_t* scales,
                                            uint32_t (&w)[lane_code_bits<LEVELS>()]) {
  constexpr int G = 1 << LG_G;
  constexpr int GL = G < 32 ? G : 32;  // elements of one group inside a lane
  constexpr int NG = 32 / GL;          // groups (or parts of a group) per lane
  constexpr int NPOS = LEVELS == 3 ? 1 : LEVELS == 256 ? 8 : LEVELS / 2 - 1;
  constexpr int CPOS = LEVELS == 3 ? 1 : LEVELS / 2;      // idx of the smallest u > 0
  constexpr int CNEG = LEVELS == 3 ? 1 : LEVELS / 2 - 1;  // idx of u = 0
  constexpr int BITS = lane_code_bits<LEVELS>();

  // group RMS and fp16 scales
  double rinv[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    // eight independent partial sums (a single chain of GL dependent fp64 adds would leave
    // the wave waiting on each one)
    constexpr int NA = GL < 8 ? GL : 8;
    double part[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) part[a] = v[GL * k + a] * v[GL * k + a];
#pragma unroll
    for (int j = NA; j < GL; ++j) part[j % NA] = __builtin_fma(v[GL * k + j], v[GL * k + j], part[j % NA]);
#pragma unroll
    for (int s = NA / 2; s >= 1; s /= 2)
#pragma unroll
      for (int a = 0; a < s; ++a) part[a] += part[a + s];
    double sq = part[0];
    if constexpr (G >= 64) sq += lane_xor<1>(sq);
    if constexpr (G == 128) sq += lane_xor<2>(sq);
    const double rr = __builtin_sqrt(sq / G);
    rinv[k] = rr > 0.0 ? 1.0 / rr : 0.0;
    const uint16_t sc = double_to_half_rne_sat(rr * inv_sqrt_k);
    if (live && (G <= 32 || (lane & (G / 32 - 1)) == 0))
      scales[row * (K >> LG_G) + ((off + GL * k) >> LG_G)] = sc;
  }

  // snap: idx = #{k : u > t_k} in binary32, from the positive thresholds alone (the
  // codebook is symmetric): u > 0 takes CPOS + #{t > 0 : u > t}; u <= 0 takes
  // CNEG - #{t > 0 : |u| >= t}; key = bits(|u|) + (u <= 0) turns both into one count.
  // The indices go straight into their packed words.
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float u = static_cast<float>(v[j] * rinv[j / GL]);
    const uint32_t ub = __float_as_uint(u);
    const bool pos = static_cast<int32_t>(ub) > 0;  // u > 0 (never NaN here)
    const uint32_t key = (ub & 0x7fffffffu) + (pos ? 0u : 1u);
    uint32_t cnt = 0;
    if constexpr (LEVELS == 256) {
      // 127 positive thresholds: a branch-free binary search for #{q : key > tk[q]}
#pragma unroll
      for (int st = 64; st >= 1; st >>= 1) cnt += key > tk[cnt + st - 1] ? st : 0u;
    } else {
#pragma unroll
      for (int k = 0; k < NPOS; ++k) cnt += key > tbits[k] ? 1u : 0u;
    }
    const uint32_t idx = pos ? CPOS + cnt : CNEG - cnt;
    const int bp = BITS * j;
    w[bp >> 5] |= idx << (bp & 31);
    if ((bp & 31) + BITS > 32) w[(bp >> 5) + 1] |= idx >> (32 - (bp & 31));
  }
}

// The positive thresholds of the symmetric codebook of `levels` levels as binary32 bit
// patterns, ascending, into dst (levels / 2 - 1 of them; 1 for trits). False if the
// codebook is not symmetric about a zero threshold (never for the built-in codebooks).
bool positive_threshold_bits(int levels, uint32_t* dst);

}  // namespace tq
