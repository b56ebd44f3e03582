// Block-wide randomized Hadamard transform of one row held in LDS (NT threads, wave64).
//
// The row v of length K = m * P (element (a, b) at a * P + b) is transformed in place to
// H_K v with H_K = H_m (x) H_P (turboquant-mlx "How it works", "Quantizing a weight, with
// no data": a Hadamard matrix with random signs; "Running a quantized layer": the input is
// rotated the same way). The layout in LDS is padded with one unused word after every 16
// (element i lives at i + i / 16), which makes every access pattern below free of bank
// conflicts: 16-lane runs of consecutive elements, runs at a stride of 8 or 16 elements
// between lane groups, and columns of the m x P view.
//
// Stages: the caller applies the butterflies of stride < R0 in registers while loading
// (segments of 16 consecutive elements per thread); passes of up to 16 points then finish
// the Sylvester part, and the m-point factor combines the m rows of each column.
#pragma once

#include <utility>

#include "device_common.hpp"

namespace tq {

__device__ __forceinline__ int pidx(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int padded_len(int n) { return n + n / 16 + 1; }

// One radix-2^R pass of the Sylvester transform over rows of length P (total elements
// `total`), pairing elements at stride h = 2^lh.
template <typename T, int R, int NT = kBlock>
__device__ __forceinline__ void sylvester_pass_p(T* buf, int total, int lh) {
  constexpr int n = 1 << R;
  const int ngroups = total >> R;
  const int h = 1 << lh;
  for (int g = threadIdx.x; g < ngroups; g += NT) {
    const int blk = g >> lh, off = g & (h - 1);
    const int base = (blk << (lh + R)) + off;
    T v[n];
#pragma unroll
    for (int j = 0; j < n; ++j) v[j] = buf[pidx(base + j * h)];
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
    for (int j = 0; j < n; ++j) buf[pidx(base + j * h)] = v[j];
  }
  __syncthreads();
}

// Remaining Sylvester stages of stride h0 .. P/2 (h0 a power of two <= P).
template <typename T, int NT = kBlock>
__device__ __forceinline__ void sylvester_rest(T* buf, int total, int P, int h0) {
  int lh = __builtin_ctz(h0);
  const int lp = __builtin_ctz(P);
  while (lh < lp) {
    const int left = lp - lh;
    if (left >= 4) { sylvester_pass_p<T, 4, NT>(buf, total, lh); lh += 4; }
    else if (left == 3) { sylvester_pass_p<T, 3, NT>(buf, total, lh); lh += 3; }
    else if (left == 2) { sylvester_pass_p<T, 2, NT>(buf, total, lh); lh += 2; }
    else { sylvester_pass_p<T, 1, NT>(buf, total, lh); lh += 1; }
  }
}

// The m-point factor on every column b of the m x P view. Every entry is a template
// constant (kHad), so each output is a fixed chain of adds and subtracts.
template <int M, int A, int C>
inline constexpr int kHad = hadamard_entry(M, A, C);

template <typename T, int M, int A, int... C>
__device__ __forceinline__ T hadamard_row(const T (&x)[M], std::integer_sequence<int, C...>) {
  T acc = 0;
  ((acc = (kHad<M, A, C> > 0) ? acc + x[C] : acc - x[C]), ...);
  return acc;
}

template <typename T, int M, int NT = kBlock>
__device__ __forceinline__ void hadamard_factor_cols(T* buf, int P) {
  for (int b = threadIdx.x; b < P; b += NT) {
    T x[M];
#pragma unroll
    for (int a = 0; a < M; ++a) x[a] = buf[pidx(a * P + b)];
    T y[M];
    [&]<int... A>(std::integer_sequence<int, A...>) {
      ((y[A] = hadamard_row<T, M, A>(x, std::make_integer_sequence<int, M>{})), ...);
    }(std::make_integer_sequence<int, M>{});
#pragma unroll
    for (int a = 0; a < M; ++a) buf[pidx(a * P + b)] = y[a];
  }
  __syncthreads();
}

template <typename T, int NT = kBlock>
__device__ __forceinline__ void hadamard_factor(T* buf, int m, int P) {
  switch (m) {
    case 12: hadamard_factor_cols<T, 12, NT>(buf, P); break;
    case 20: hadamard_factor_cols<T, 20, NT>(buf, P); break;
    case 28: hadamard_factor_cols<T, 28, NT>(buf, P); break;
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
