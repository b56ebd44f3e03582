// The input rotation of the qmv kernels for K = 4096 (the Sylvester factor alone) on the
// matrix cores.
//
// The rotation x' = H_K diag(s) x / sqrt(K) (turboquant-mlx "How it works", "Running a
// quantized layer": the input gets the weights' rotation) with K = 64 * 64 is, since
// H_4096 = H_64 (x) H_64, the matrix product X' = H_64 X H_64 of the 64 x 64 view
// X[a][b] = s_i x_i, i = 64 a + b, read back as x'_{64 d + c} = X'[d][c]. Two
// v_mfma_f32_16x16x32 products replace the twelve butterfly stages:
//
//   Z = X H_64   waves 0..3, wave t: rows 16 t .. 16 t + 15 of Z, 8 instructions; the
//                16-bit input is exact in the operands, the sums are fp32
//   X' = H_64 Z  all 16 waves, one 16 x 16 tile each; Z is split into two bf16 terms
//                (hi + lo, 16 significant bits together) so the second product loses no
//                more than 2^-17 of each entry of Z, far below the fp16 rounding of x'
//
// Z goes through LDS transposed (row c of Zt holds column c of Z), so each lane reads its
// eight consecutive K positions of the second product with one 16-byte read. Entries of
// H are generated in registers: H_64[r][k] = (-1)^popcount(r & k) splits into the sign of
// the high bits of r & k times row r & 7 of H_8, whose eight signs are one byte of the
// constant kH8Rows.
//
// Lane layout of v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[l % 16][8 (l / 16) + j]
// and B[8 (l / 16) + j][l % 16] (j < 8) and gets D[4 (l / 16) + r][l % 16] (r < 4).
#pragma once

#include "decode_common.hpp"
#include "fwht_block.hpp"

namespace tq {

// Byte a = the signs of row a of H_8: bit j set when popcount(a & j) is odd.
constexpr uint64_t kH8Rows = 0x963C5AF066CCAA00ull;
constexpr uint32_t kNeg2 = 0x80008000u;  // both halves negated

// Sign-bit mask for the eight 16-bit values of a fragment (pairs p = 0..3) from eight sign
// bits: bit 2p goes to bit 15 of word p, bit 2p + 1 to bit 31.
__device__ __forceinline__ uint32_t pair_sign_mask(uint32_t bits, int p) {
  return ((bits << (15 - 2 * p)) & 0x8000u) | ((bits << (30 - 2 * p)) & 0x80000000u);
}

// Row a & 7 of H_8 as four 16-bit +-1 pairs (one2 = the 16-bit 1.0 twice).
__device__ __forceinline__ u32x4_t h8_row(int a, uint32_t one2) {
  const uint32_t bits = static_cast<uint32_t>(kH8Rows >> (8 * (a & 7))) & 0xffu;
  u32x4_t f;
#pragma unroll
  for (int p = 0; p < 4; ++p) f[p] = one2 | pair_sign_mask(bits, p);
  return f;
}

__device__ __forceinline__ u32x4_t xor4(const u32x4_t& v, uint32_t m) {
  return u32x4_t{v[0] ^ m, v[1] ^ m, v[2] ^ m, v[3] ^ m};
}

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_h16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// max |value| of the eight 16-bit inputs of a fragment (bf16 when BF, else fp16)
template <bool BF>
__device__ __forceinline__ float frag_absmax(const u32x4_t& v) {
  float m = 0.f;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float a, b;
    if constexpr (BF) {
      a = __uint_as_float(v[p] << 16);
      b = __uint_as_float(v[p] & 0xffff0000u);
    } else {
      a = static_cast<float>(__builtin_bit_cast(half2_t, v[p]).x);
      b = static_cast<float>(__builtin_bit_cast(half2_t, v[p]).y);
    }
    m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
  }
  return m;
}

// Two fp32 values as a pair of bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(a))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(b))) << 16);
}
__device__ __forceinline__ float bf16_lo_f(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Zt rows: 64 bf16 + 16 bytes, so the 16-byte reads of 8 consecutive rows fall on disjoint
// banks
constexpr int kZtRowBytes = 144;
constexpr int kZtBytes = 64 * kZtRowBytes;  // one term (hi or lo); the two need 18 KB

template <int NT>
struct Rot4096Mfma {
  static_assert(NT == 1024, "one 16 x 16 output tile per wave of a 1024-thread workgroup");
  u32x4_t xa[2];  // X[16 t + l % 16][32 s + 8 (l / 16) + j], s = 0, 1 (16-bit, raw)
  u32x2_t sw;     // the sign words of those 64 elements of row 16 t + l % 16

  // Loads of the input row (16-bit, K = 4096) and its sign words: two 16-byte loads and one
  // 8-byte load per lane of waves 0..3, the only ones that use them (the other waves issue
  // nothing here: loads they would not use only slow the issue of the code loads).
  __device__ __forceinline__ void issue(const void* x, const uint32_t* signs) {
    if (threadIdx.x >= 256) return;
    const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
    const int a = 16 * t + (lane & 15);
    const uint32_t e0 = 64u * a + 8u * (lane >> 4);
    xa[0] = ld_at<u32x4_t>(x, 2u * e0);
    xa[1] = ld_at<u32x4_t>(x, 2u * (e0 + 32u));
    sw = ld_at<u32x2_t>(signs, 8u * a);
  }

  // The whole rotation (BF: bf16 input, else fp16). zt: 2 kZtBytes of LDS (unused by
  // anything else meanwhile); red: 4 floats. Waves 0..3 compute Z and max |x_i| while
  // waves 4..15 run side(t, nt) (thread t of nt = 768: work that needs neither x nor Z);
  // after one barrier every wave runs between() and then computes its tile of X' and writes
  // it, scaled by sc and rounded to fp16, to the chunk layout of the sink. Ends with a
  // barrier. Returns sc; *out_scale gets 1 / (sc sqrt(K)).
  //
  // Signs of the H_64 fragments: for a lane with n = l % 16, q = l / 16 and a tile index u
  // (the column block of Z, or the row block of X'), the fragment of row 16 u + n at columns
  // 32 s + 8 q + j is row n & 7 of H_8 times (-1)^popcount((32 s + 8 q) & (16 u + n) & 56),
  // and that exponent is (q & 1)(n >> 3) + (q >> 1)(u & 1) + s (u >> 1): a lane mask, a lane
  // mask for odd u, and a sign that is uniform per instruction.
  template <bool BF, typename Side, typename Between>
  __device__ __forceinline__ float rotate(char* zt, float* red, int lk, float inv_sqrt_k,
                                          _Float16* xh, float* out_scale, Side side,
                                          Between between) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const uint32_t m_lane = ((q & 1) & (n >> 3)) ? kNeg2 : 0u;
    const uint32_t m_odd = (q >> 1) ? kNeg2 : 0u;
    // second product: A = H_64[16 di + n][32 s + 8 q + j] (bf16)
    const int di = wave >> 2, tj2 = wave & 3;
    u32x4_t a2[2];
    {
      const u32x4_t h = xor4(h8_row(n, 0x3F803F80u), m_lane ^ ((di & 1) ? m_odd : 0u));
      a2[0] = h;
      a2[1] = xor4(h, (di >> 1) ? kNeg2 : 0u);
    }
    if (wave < 4) {
      const int t = wave;
      const u32x4_t b0 = xor4(h8_row(n, BF ? 0x3F803F80u : 0x3C003C00u), m_lane);
      const u32x4_t b1 = xor4(b0, m_odd);
      u32x4_t xs[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t bits = (sw[s] >> (8 * q)) & 0xffu;
#pragma unroll
        for (int p = 0; p < 4; ++p) xs[s][p] = xa[s][p] ^ pair_sign_mask(bits, p);
      }
      float mx = fmaxf(frag_absmax<BF>(xa[0]), frag_absmax<BF>(xa[1]));
      // Z[16 t + m][16 tj + c] = sum_b X[16 t + m][b] H_64[b][16 tj + c]: B is the fragment
      // of row 16 tj + n of the symmetric H_64; four independent accumulators
      f32x4_t acc[4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          const u32x4_t b = xor4((tj & 1) ? b1 : b0, (s && (tj >> 1)) ? kNeg2 : 0u);
          const f32x4_t c = s ? acc[tj] : f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc[tj] = BF ? mfma_bf16(xs[s], b, c) : mfma_h16(xs[s], b, c);
        }
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        // acc[tj][r] = Z[16 t + 4 q + r][16 tj + n] -> Zt row 16 tj + n, column 16 t + 4 q + r
        const f32x4_t z = acc[tj];
        const uint32_t h01 = pack_bf16x2(z[0], z[1]), h23 = pack_bf16x2(z[2], z[3]);
        const uint32_t l01 = pack_bf16x2(z[0] - bf16_lo_f(h01), z[1] - bf16_hi_f(h01));
        const uint32_t l23 = pack_bf16x2(z[2] - bf16_lo_f(h23), z[3] - bf16_hi_f(h23));
        const uint32_t off = (16 * tj + n) * kZtRowBytes + (16 * t + 4 * q) * 2;
        *reinterpret_cast<u32x2_t*>(zt + off) = u32x2_t{h01, h23};
        *reinterpret_cast<u32x2_t*>(zt + kZtBytes + off) = u32x2_t{l01, l23};
      }
      mx = wave_max_nonneg(mx);
      if (lane == 63) red[t] = mx;
    } else {
      side(static_cast<int>(threadIdx.x) - 256, NT - 256);
    }
    __syncthreads();
    between();
    const float mall = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int ex = 0;
    if (mall > 0.f && mall <= 3.4028234663852886e38f) {
      ex = 14 - ilogbf(mall) - lk;
      ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
    }
    *out_scale = ldexpf(1.f, -ex) * inv_sqrt_k;
    const float sc = ldexpf(1.f, ex);

    // X'[16 di + m][16 tj + c] = sum_a H_64[16 di + m][a] Z[a][16 tj + c]
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t off = (16 * tj2 + n) * kZtRowBytes + (32 * s + 8 * q) * 2;
      const u32x4_t zh = *reinterpret_cast<const u32x4_t*>(zt + off);
      const u32x4_t zl = *reinterpret_cast<const u32x4_t*>(zt + kZtBytes + off);
      acc = mfma_bf16(a2[s], zh, acc);
      acc = mfma_bf16(a2[s], zl, acc);
    }
    // acc[r] = x'_e, e = 64 (16 di + 4 q + r) + 16 tj + n
    const HalfSink sink{xh, sc};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = 64 * (16 * di + 4 * q + r) + 16 * tj2 + n;
      sink.put_at(HalfSink::idx(e), acc[r]);
    }
    __syncthreads();
    return sc;
  }
};

}  // namespace tq
