// Block-wide randomized Hadamard transform of one row held in LDS (NT threads, wave64).
//
// The row v of length K = m * P (element (a, b) at a * P + b) is transformed in place to
// H_K v with H_K = H_m (x) H_P (turboquant-mlx "How it works", "Quantizing a weight, with
// no data": a Hadamard matrix with random signs; "Running a quantized layer": the input is
// rotated the same way). The layout in LDS is padded with one unused word after every 16
// (element i lives at i + i / 16), which makes every access pattern below free of bank
// conflicts: 16-lane runs of consecutive elements, runs at a stride of 16 or more elements
// between lane groups, and columns of the m x P view.
//
// Stages: the caller applies the butterflies of stride < 16 in registers while loading
// (segments of 16 consecutive elements per thread); passes of up to 16 points at
// compile-time strides then finish the Sylvester part, and the m-point factor combines the
// m rows of each column, several threads per column.
#pragma once

#include <utility>

#include "device_common.hpp"

namespace tq {

__device__ __forceinline__ int pidx(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int padded_len(int n) { return n + n / 16 + 1; }

// One radix-2^R pass pairing elements at stride 2^LH (LH >= 4) over `total` elements. The
// padded distance of 2^LH elements is the constant 17 * 2^(LH-4) words, so every access of
// a group is a fixed offset from its first element.
template <typename T, int R, int LH, int NT>
__device__ __forceinline__ void sylvester_pass_c(T* buf, int total) {
  constexpr int n = 1 << R, h = 1 << LH, step = 17 * (h / 16);
  const int ngroups = total >> R;
  for (int g = threadIdx.x; g < ngroups; g += NT) {
    const int blk = g >> LH, off = g & (h - 1);
    T* base = buf + pidx((blk << (LH + R)) + off);
    T v[n];
#pragma unroll
    for (int j = 0; j < n; ++j) v[j] = base[j * step];
#pragma unroll
    for (int s = 0; s < R; ++s)
#pragma unroll
      for (int j = 0; j < n; ++j) {
        if ((j >> s) & 1) continue;
        const T a = v[j], b = v[j + (1 << s)];
        v[j] = a + b;
        v[j + (1 << s)] = a - b;
      }
#pragma unroll
    for (int j = 0; j < n; ++j) base[j * step] = v[j];
  }
  __syncthreads();
}

// STAGES butterfly stages starting at stride 2^LH, in ceil(STAGES / 4) passes of nearly
// equal radix.
template <typename T, int NT, int LH, int STAGES>
__device__ __forceinline__ void sylvester_stages(T* buf, int total) {
  if constexpr (STAGES > 0) {
    constexpr int passes = (STAGES + 3) / 4;
    constexpr int R = (STAGES + passes - 1) / passes;
    sylvester_pass_c<T, R, LH, NT>(buf, total);
    sylvester_stages<T, NT, LH + R, STAGES - R>(buf, total);
  }
}

// The Sylvester stages of stride 16 .. P/2 on runs of length P = 2^lp.
template <typename T, int NT>
__device__ __forceinline__ void sylvester_from16(T* buf, int total, int lp) {
  switch (lp) {
    case 5: sylvester_stages<T, NT, 4, 1>(buf, total); break;
    case 6: sylvester_stages<T, NT, 4, 2>(buf, total); break;
    case 7: sylvester_stages<T, NT, 4, 3>(buf, total); break;
    case 8: sylvester_stages<T, NT, 4, 4>(buf, total); break;
    case 9: sylvester_stages<T, NT, 4, 5>(buf, total); break;
    case 10: sylvester_stages<T, NT, 4, 6>(buf, total); break;
    case 11: sylvester_stages<T, NT, 4, 7>(buf, total); break;
    case 12: sylvester_stages<T, NT, 4, 8>(buf, total); break;
    case 13: sylvester_stages<T, NT, 4, 9>(buf, total); break;
    default: break;  // P <= 16: done in registers
  }
}

// ---------------------------------------------------------------------------------------
// The m-point factor on every column b of the m x P view. Entries are template constants,
// so each output is a fixed chain of adds and subtracts.
//
// H_12 and H_20 (Paley I) are applied row by row (m - 1 additions per output). H_28 is
// Paley II, S (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]] with S the symmetric
// conference matrix of order 14, which needs fewer additions: with u_C = x_2C + x_2C+1 and
// v_C = x_2C - x_2C+1,  y_2R = sum_C S[R][C] u_C + v_R  and  y_2R+1 = sum_C S[R][C] v_C - u_R.
template <int M, int A, int C>
inline constexpr int kHad = hadamard_entry(M, A, C);

constexpr int conference14(int r, int c) {
  return r == c ? 0 : (r == 0 || c == 0) ? 1 : qchar((r - 1) - (c - 1), 13);
}
template <int R, int C>
inline constexpr int kConf = conference14(R, C);

template <typename T, int M, int A, int... C>
__device__ __forceinline__ T hadamard_row(const T (&x)[M], std::integer_sequence<int, C...>) {
  T acc = 0;
  ((acc = (kHad<M, A, C> > 0) ? acc + x[C] : acc - x[C]), ...);
  return acc;
}

template <typename T, int R, int... C>
__device__ __forceinline__ T conference_row(const T (&u)[14], std::integer_sequence<int, C...>) {
  T acc = 0;
  ((acc = kConf<R, C> == 0 ? acc : (kConf<R, C> > 0 ? acc + u[C] : acc - u[C])), ...);
  return acc;
}

// TPC threads per column (a power of two, the same for a whole wave when P >= 64): thread
// part q computes the outputs a (or row pairs R) with a % TPC == q. All inputs are read
// before any output is written; the function synchronizes at the end.
template <typename T, int M, int TPC, int NT>
__device__ __forceinline__ void hadamard_factor_split(T* buf, int P) {
  const int t = threadIdx.x;
  const bool active = t < P * TPC;
  const int q = t / P, b = t - q * P;
  T x[M];
  if (active) {
#pragma unroll
    for (int a = 0; a < M; ++a) x[a] = buf[pidx(a * P + b)];
  }
  if constexpr (TPC > 1) __syncthreads();  // other parts of the column read the same inputs
  if (active) {
    if constexpr (M == 28) {
      T u[14], v[14];
#pragma unroll
      for (int c = 0; c < 14; ++c) { u[c] = x[2 * c] + x[2 * c + 1]; v[c] = x[2 * c] - x[2 * c + 1]; }
      [&]<int... R>(std::integer_sequence<int, R...>) {
        (((R % TPC) == q
              ? (buf[pidx(2 * R * P + b)] =
                     conference_row<T, R>(u, std::make_integer_sequence<int, 14>{}) + v[R],
                 buf[pidx((2 * R + 1) * P + b)] =
                     conference_row<T, R>(v, std::make_integer_sequence<int, 14>{}) - u[R],
                 0)
              : 0),
         ...);
      }(std::make_integer_sequence<int, 14>{});
    } else {
      [&]<int... A>(std::integer_sequence<int, A...>) {
        (((A % TPC) == q
              ? (buf[pidx(A * P + b)] =
                     hadamard_row<T, M, A>(x, std::make_integer_sequence<int, M>{}),
                 0)
              : 0),
         ...);
      }(std::make_integer_sequence<int, M>{});
    }
  }
  __syncthreads();
}

template <typename T, int M, int NT>
__device__ __forceinline__ void hadamard_factor_m(T* buf, int P) {
  if (P < 64) {
    hadamard_factor_split<T, M, 1, NT>(buf, P);
    return;
  }
  const int tpc = NT / P;  // 1 .. NT / 64, a power of two
  if (tpc >= 8) hadamard_factor_split<T, M, 8, NT>(buf, P);
  else if (tpc == 4) hadamard_factor_split<T, M, 4, NT>(buf, P);
  else if (tpc == 2) hadamard_factor_split<T, M, 2, NT>(buf, P);
  else hadamard_factor_split<T, M, 1, NT>(buf, P);
}

template <typename T, int NT>
__device__ __forceinline__ void hadamard_factor(T* buf, int m, int P) {
  switch (m) {
    case 12: hadamard_factor_m<T, 12, NT>(buf, P); break;
    case 20: hadamard_factor_m<T, 20, NT>(buf, P); break;
    case 28: hadamard_factor_m<T, 28, NT>(buf, P); break;
    default: break;
  }
}

// Butterflies of stride 1 .. R0/2 on 16 consecutive elements in registers (R0 = min(16, P)
// so that no butterfly crosses a row of length P).
template <typename T>
__device__ __forceinline__ void seg16_butterflies(T (&v)[16], int P) {
  const int stages = P >= 16 ? 4 : __builtin_ctz(P);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s >= stages) break;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j >> s) & 1) continue;
      const T a = v[j], b = v[j + (1 << s)];
      v[j] = a + b;
      v[j + (1 << s)] = a - b;
    }
  }
}

}  // namespace tq
