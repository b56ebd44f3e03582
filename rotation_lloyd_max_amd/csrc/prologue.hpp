// Input rotation prologue of the qmv family: load one activation row with a few wide loads
// (all issued before any is used), apply the rotation signs and the butterflies of stride
// < 16 in registers, finish H_K in LDS (fwht_block.hpp), and hand every lane the rotated
// input of its chunks as scaled fp16 pairs.
//
// The rotation is x' = H_K diag(s) x / sqrt(K) (turboquant-mlx "How it works", "Running a
// quantized layer": the input gets the weights' rotation). The unnormalized H_K s x is kept
// in fp16 after multiplying by a power of two 2^e chosen from max |x_i| and K, so that no
// entry can overflow and each keeps fp16's 11 significant bits. The factor 2^-e (and
// 1/sqrt(K)) is applied to the row sums.
#pragma once

#include "decode_common.hpp"
#include "fwht_block.hpp"

namespace tq {

constexpr int kMaxK = 8192;

// X32: the input is fp32; otherwise a 16-bit type, bf16 or fp16 by the runtime dtype.
// Inside a wave the loads are unconditional (indices are clamped); a wave none of whose
// lanes has a segment skips them.
template <bool X32, int NT, int MAXK = kMaxK>
struct InputLoad {
  static constexpr int kSeg16 = (MAXK / 16 + NT - 1) / NT;  // 16-element segments per thread
  static constexpr int kW = X32 ? 16 : 8;
  uint32_t raw[kSeg16][kW];
  uint32_t sw[kSeg16];  // the sign word holding each segment's 16 sign bits
  float v[kSeg16][16];  // the segments after signs and small butterflies
  int dt;

  // Segment j of thread t covers elements 16 * (t + NT * j) + 0..15 of row `row`.
  // `signs` is null for an input that is already rotated: then no sign word is read (the
  // weight may have none) and finish() applies none.
  __device__ __forceinline__ void issue(const void* x, int xdt, int64_t row, int K,
                                        const uint32_t* signs) {
    dt = xdt;
    const int nseg = K >> 4;
#pragma unroll
    for (int j = 0; j < kSeg16; ++j) {
      int sgi = threadIdx.x + NT * j;
      // a wave with no segment here issues no load (finish_a() skips such segments)
      if ((static_cast<int>(threadIdx.x) & ~63) + NT * j >= nseg) continue;
      sgi = sgi < nseg ? sgi : nseg - 1;
      const int64_t e0 = row * K + 16 * static_cast<int64_t>(sgi);
      const uint4* q = X32 ? reinterpret_cast<const uint4*>(static_cast<const float*>(x) + e0)
                           : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e0);
#pragma unroll
      for (int v = 0; v < kW / 4; ++v) {
        const uint4 a = q[v];
        raw[j][4 * v + 0] = a.x; raw[j][4 * v + 1] = a.y;
        raw[j][4 * v + 2] = a.z; raw[j][4 * v + 3] = a.w;
      }
      sw[j] = signs ? signs[sgi >> 1] : 0u;
    }
  }

  __device__ __forceinline__ float elem(int j, int k) const {
    if constexpr (X32) {
      return __uint_as_float(raw[j][k]);
    } else {
      const uint32_t v = raw[j][k >> 1];
      const uint16_t h = static_cast<uint16_t>((k & 1) ? (v >> 16) : (v & 0xffff));
      return dt == 1 ? bf16_bits_to_float(h) : half_bits_to_float(h);
    }
  }

  // First half of the rotation: apply the signs and the butterflies of stride < 16 to
  // every segment in registers and write them to xf (padded layout; a rotated input that
  // goes straight to the fp16 layout stays in registers), and find max |x_i| (one float per
  // wave in `red`, NT / 64 floats of LDS). Ends with a barrier. Returns the power of two sc
  // for the fp16 conversion; *out_scale gets 1 / sc, times 1 / sqrt(K) when the rotation
  // is applied here.
  //
  // Every entry of the unnormalized H_K s x is a sum of K terms of size at most
  // max |x_i| < 2^(e + 1), e = ilogb(max |x_i|), so with K <= 2^lk it is below
  // 2^(e + 1 + lk), and sc = 2^(14 - e - lk) keeps every scaled entry below 2^15 (fp16 holds
  // up to 65504). A rotated input is its own bound (lk = 0).
  template <bool HALF>
  __device__ __forceinline__ float finish_a(float* xf, float* red, int K, int lk, int P,
                                            bool rotated, float inv_sqrt_k, float* out_scale) {
    const int nseg = K >> 4;
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < kSeg16; ++j) {
      const int sgi = threadIdx.x + NT * j;
      if (sgi >= nseg) continue;
      const uint32_t bits = rotated ? 0u : (sw[j] >> (16 * (sgi & 1))) & 0xffffu;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float a = elem(j, k);
        mx = fmaxf(mx, fabsf(a));
        v[j][k] = __uint_as_float(__float_as_uint(a) ^ (((bits >> k) & 1u) << 31));
      }
      if (!rotated) seg16_butterflies<float>(v[j], P);
      if (!(HALF && rotated)) {
        float* dst = xf + 17 * sgi;  // pidx(16 * sgi + k) = 17 * sgi + k
#pragma unroll
        for (int k = 0; k < 16; ++k) dst[k] = v[j][k];
      }
    }
    mx = wave_max_nonneg(mx);
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    float mall = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) mall = fmaxf(mall, red[w]);
    int ex = 0;
    if (mall > 0.f && mall <= 3.4028234663852886e38f) {
      ex = 14 - ilogbf(mall) - (rotated ? 0 : lk);
      ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
    }
    *out_scale = ldexpf(1.f, -ex) * (rotated ? 1.f : inv_sqrt_k);
    return ldexpf(1.f, ex);
  }

  // Second half: the remaining stages of H_K in LDS (none for a rotated input). With HALF
  // the results go, scaled by sc and rounded to fp16, to the chunk layout xh (bit formats:
  // 32 elements per chunk); otherwise they stay in xf. Ends with a barrier.
  template <bool HALF>
  __device__ __forceinline__ void finish_b(float* xf, uint32_t* xh, int K, int m, int P,
                                           bool rotated, float sc) {
    const HalfSink sink{reinterpret_cast<_Float16*>(xh), sc};
    if (rotated) {
      if constexpr (HALF) {
        const int nseg = K >> 4;
#pragma unroll
        for (int j = 0; j < kSeg16; ++j) {
          const int sgi = threadIdx.x + NT * j;
          if (sgi >= nseg) continue;
          // the 16 elements of a segment are one half of chunk sgi / 2
          uint32_t hw[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            hw[k] = static_cast<uint32_t>(float_to_half_rne(v[j][2 * k] * sc)) |
                    (static_cast<uint32_t>(float_to_half_rne(v[j][2 * k + 1] * sc)) << 16);
          uint4* dst = reinterpret_cast<uint4*>(
              reinterpret_cast<_Float16*>(xh) + (sgi >> 1) * kChunkHalves + (sgi & 1) * 16);
          dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          dst[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
        }
        __syncthreads();
      }
      return;
    }
    const int lp = __builtin_ctz(P);
    if (m == 1) {
      sylvester_from16<float, NT, HALF>(xf, K, lp, sink);
    } else {
      sylvester_from16<float, NT, false>(xf, K, lp);
      hadamard_factor<float, NT, HALF>(xf, m, P, sink);
    }
  }
};

// Words between the fp16 pair slices of consecutive chunks in LDS: the chunk's pairs plus
// padding, so that the 16-byte reads of 16 consecutive lanes (one chunk each) fall on 16
// disjoint groups of 4 banks (stride 20 words for 16 pairs, 12 words for 10 pairs). The
// bit formats' stride is the HalfSink layout the rotation can write directly.
template <int L>
constexpr int pair_stride() {
  return Fmt<L>::np == 16 ? kChunkHalves / 2 : 12;
}

// Convert the rotated row (padded fp32 in xf) once per workgroup to scaled fp16 pairs laid
// out chunk by chunk in xh (Q chunks of pair_stride words, 16-byte aligned); pairs past K
// are zero. Pair k holds elements 2k and 2k + 1, which is pair k % np of chunk k / np
// because a chunk holds 2 np consecutive elements. Ends synchronized.
template <int L, int NT>
__device__ __forceinline__ void pairs_to_lds(const float* xf, uint32_t* xh, int K, int Q, float sc) {
  using F = Fmt<L>;
  constexpr int S = pair_stride<L>();
  const int total = Q * F::np;
  for (int k = threadIdx.x; k < total; k += NT) {
    const int c = k / F::np, q = k - c * F::np;
    const int e0 = 2 * k;
    const float ra = xf[pidx(e0 < K ? e0 : K - 1)];
    const float rb = xf[pidx(e0 + 1 < K ? e0 + 1 : K - 1)];
    const float a = e0 < K ? ra * sc : 0.f;
    const float b = e0 + 1 < K ? rb * sc : 0.f;
    xh[c * S + q] = static_cast<uint32_t>(float_to_half_rne(a)) |
                    (static_cast<uint32_t>(float_to_half_rne(b)) << 16);
  }
  __syncthreads();
}

// The fp16 pairs of a lane's chunks (chunk cbase + c0 + j * lpr of the slice of slice_q
// chunks starting at cbase; positions past the slice read its last chunk, whose products
// the caller discards), with 16-byte LDS reads.
template <int L, int CPL>
__device__ __forceinline__ void lane_pairs(const uint32_t* xh, int cbase, int c0, int lpr,
                                           int slice_q, uint32_t (&xr)[CPL][Fmt<L>::np]) {
  using F = Fmt<L>;
  constexpr int S = pair_stride<L>();
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int cr = c0 + j * lpr;
    const int c = cbase + (cr < slice_q ? cr : slice_q - 1);
    const uint4* src = reinterpret_cast<const uint4*>(xh + c * S);
#pragma unroll
    for (int v = 0; v < F::np / 4; ++v) {
      const uint4 a = src[v];
      xr[j][4 * v + 0] = a.x; xr[j][4 * v + 1] = a.y;
      xr[j][4 * v + 2] = a.z; xr[j][4 * v + 3] = a.w;
    }
    if constexpr (F::np % 4 == 2) {
      const uint2 a = reinterpret_cast<const uint2*>(src + F::np / 4)[0];
      xr[j][F::np - 2] = a.x; xr[j][F::np - 1] = a.y;
    }
  }
}

}  // namespace tq
