// Input rotation prologue of the qmv family: load one activation row with a few wide loads
// (all issued before any is used), apply the rotation signs and the butterflies of stride
// < 16 in registers, finish H_K in LDS (fwht_block.hpp), and hand every lane the rotated
// input of its chunks as scaled fp16 pairs.
//
// The rotation is x' = H_K diag(s) x / sqrt(K) (turboquant-mlx "How it works", "Running a
// quantized layer": the input gets the weights' rotation). Every |x'_j| is at most
// ||x'|| = ||x||, so x' is kept in fp16 after multiplying by 2^e with e chosen from ||x||
// (computed in fp64 from the loaded registers): no entry can overflow and each keeps
// fp16's 11 significant bits. The factor 2^-e (and 1/sqrt(K)) is applied to the row sums.
#pragma once

#include "decode_common.hpp"
#include "fwht_block.hpp"

namespace tq {

constexpr int kMaxK = 8192;

// X32: the input is fp32; otherwise a 16-bit type, bf16 or fp16 by the runtime dtype.
// All loads are unconditional (indices are clamped) so that no branch separates them from
// the loads the caller issues next, and the compiler can wait for exactly these.
template <bool X32, int NT>
struct InputLoad {
  static constexpr int kSeg16 = (kMaxK / 16 + NT - 1) / NT;  // 16-element segments per thread
  static constexpr int kW = X32 ? 16 : 8;
  uint32_t raw[kSeg16][kW];
  uint32_t sw[kSeg16];  // the sign word holding each segment's 16 sign bits
  int dt;

  // Segment j of thread t covers elements 16 * (t + NT * j) + 0..15 of row `row`.
  // `signs` must be a valid pointer (finish() ignores the signs of a rotated input).
  __device__ __forceinline__ void issue(const void* x, int xdt, int64_t row, int K,
                                        const uint32_t* signs) {
    dt = xdt;
    const int nseg = K >> 4;
#pragma unroll
    for (int j = 0; j < kSeg16; ++j) {
      int sgi = threadIdx.x + NT * j;
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
      sw[j] = signs[sgi >> 1];
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

  // Write s * x into xf (padded layout) with the small butterflies applied, reduce ||x||^2,
  // then finish H_K in LDS unless `rotated`. `red` holds NT / 64 doubles of LDS scratch. Ends
  // synchronized. Returns the power of two sc for the fp16 conversion; *out_scale gets
  // 1 / sc, times 1 / sqrt(K) when the rotation was applied here.
  __device__ __forceinline__ float finish(float* xf, double* red, int K, int m, int P,
                                          bool rotated, float inv_sqrt_k, float* out_scale) {
    const int nseg = K >> 4;
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kSeg16; ++j) {
      const int sgi = threadIdx.x + NT * j;
      if (sgi >= nseg) continue;
      const uint32_t bits = rotated ? 0u : (sw[j] >> (16 * (sgi & 1))) & 0xffffu;
      float v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float a = elem(j, k);
        v[k] = ((bits >> k) & 1u) ? -a : a;
        ss += static_cast<double>(a) * static_cast<double>(a);
      }
      if (!rotated) seg16_butterflies<float>(v, P);
      float* dst = xf + 17 * sgi;  // pidx(16 * sgi + k) = 17 * sgi + k
#pragma unroll
      for (int k = 0; k < 16; ++k) dst[k] = v[k];
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    if (!rotated) {
      sylvester_rest<float, NT>(xf, K, P, P < 16 ? P : 16);
      hadamard_factor<float, NT>(xf, m, P);
    }
    // |x'_j| <= ||x'||; unnormalized, ||H_K s x|| = sqrt(K) ||x||
    const double bound =
        __builtin_sqrt(tot) * (rotated ? 1.0 : __builtin_sqrt(static_cast<double>(K)));
    int ex = 0;
    if (bound > 0.0 && bound < 1e300) {
      ex = 14 - ilogb(bound);
      ex = ex < -120 ? -120 : (ex > 120 ? 120 : ex);
    }
    *out_scale = ldexpf(1.f, -ex) * (rotated ? 1.f : inv_sqrt_k);
    return ldexpf(1.f, ex);
  }
};

// The rotated input of a lane's chunks (chunk c = c0 + j * lpr) as fp16 pairs, read from
// the padded fp32 row; zero past K and for chunks past the row.
template <int L, int CPL>
__device__ __forceinline__ void lane_pairs(const float* xf, int K, int Q, int c0, int lpr, float sc,
                                           uint32_t (&xr)[CPL][Fmt<L>::np]) {
  using F = Fmt<L>;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = c0 + j * lpr;
    const bool okc = c < Q;
    const int cc = okc ? c : 0;
#pragma unroll
    for (int q = 0; q < F::np; ++q) {
      // unconditional reads at clamped addresses, then a select: no branch per element
      const int e0 = cc * F::ce + 2 * q;
      const float ra = xf[pidx(e0 < K ? e0 : K - 1)];
      const float rb = xf[pidx(e0 + 1 < K ? e0 + 1 : K - 1)];
      const float a = (okc && e0 < K) ? ra * sc : 0.f;
      const float b = (okc && e0 + 1 < K) ? rb * sc : 0.f;
      xr[j][q] = static_cast<uint32_t>(float_to_half_rne(a)) |
                 (static_cast<uint32_t>(float_to_half_rne(b)) << 16);
    }
  }
}

}  // namespace tq
