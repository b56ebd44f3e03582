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

// Where the last stage of the transform may put its results instead of the fp32 row: the
// fp16 chunk layout of the decode kernels, scaled by sc. Element e is half e % 32 of chunk
// e / 32, and chunks are kChunkHalves halves apart (32 used, 8 of padding).
constexpr int kChunkHalves = 40;
struct HalfSink {
  _Float16* h;  // LDS
  float sc;
  __device__ __forceinline__ static int idx(int e) { return (e >> 5) * kChunkHalves + (e & 31); }
  __device__ __forceinline__ void put_at(int hi, float v) const {
    h[hi] = static_cast<_Float16>(v * sc);
  }
};

// One radix-2^R pass pairing elements at stride 2^LH (LH >= 4) over `total` elements. The
// padded distance of 2^LH elements is the constant 17 * 2^(LH-4) words, so every access of
// a group is a fixed offset from its first element.
template <typename T, int R, int LH, int NT, bool OUT = false>
__device__ __forceinline__ void sylvester_pass_c(T* buf, int total, HalfSink sink = {}) {
  constexpr int n = 1 << R, h = 1 << LH, step = 17 * (h / 16);
  const int ngroups = total >> R;
  for (int g = threadIdx.x; g < ngroups; g += NT) {
    const int blk = g >> LH, off = g & (h - 1);
    const int e0 = (blk << (LH + R)) + off;
    T* base = buf + pidx(e0);
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
    if constexpr (OUT) {
      // e0 % 32 < 16 when h == 16, and j * h is a multiple of 32 when h >= 32, so the
      // half index of element e0 + j * h is a fixed offset from that of e0
      const int h0 = HalfSink::idx(e0);
#pragma unroll
      for (int j = 0; j < n; ++j) {
        const int d = h >= 32 ? (j * h / 32) * kChunkHalves
                              : ((j * 16) >> 5) * kChunkHalves + ((j * 16) & 31);
        sink.put_at(h0 + d, v[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < n; ++j) base[j * step] = v[j];
    }
  }
  __syncthreads();
}

// STAGES butterfly stages starting at stride 2^LH, in ceil(STAGES / 4) passes of nearly
// equal radix.
// With OUT the last pass writes its results to the sink.
template <typename T, int NT, int LH, int STAGES, bool OUT>
__device__ __forceinline__ void sylvester_stages(T* buf, int total, HalfSink sink) {
  if constexpr (STAGES > 0) {
    constexpr int passes = (STAGES + 3) / 4;
    constexpr int R = (STAGES + passes - 1) / passes;
    sylvester_pass_c<T, R, LH, NT, OUT && (STAGES == R)>(buf, total, sink);
    sylvester_stages<T, NT, LH + R, STAGES - R, OUT>(buf, total, sink);
  }
}

// The Sylvester stages of stride 16 .. P/2 on runs of length P = 2^lp (lp >= 5 when OUT,
// so that there is a last pass to write the sink).
template <typename T, int NT, bool OUT = false>
__device__ __forceinline__ void sylvester_from16(T* buf, int total, int lp, HalfSink sink = {}) {
  switch (lp) {
    case 5: sylvester_stages<T, NT, 4, 1, OUT>(buf, total, sink); break;
    case 6: sylvester_stages<T, NT, 4, 2, OUT>(buf, total, sink); break;
    case 7: sylvester_stages<T, NT, 4, 3, OUT>(buf, total, sink); break;
    case 8: sylvester_stages<T, NT, 4, 4, OUT>(buf, total, sink); break;
    case 9: sylvester_stages<T, NT, 4, 5, OUT>(buf, total, sink); break;
    case 10: sylvester_stages<T, NT, 4, 6, OUT>(buf, total, sink); break;
    case 11: sylvester_stages<T, NT, 4, 7, OUT>(buf, total, sink); break;
    case 12: sylvester_stages<T, NT, 4, 8, OUT>(buf, total, sink); break;
    case 13: sylvester_stages<T, NT, 4, 9, OUT>(buf, total, sink); break;
    default: break;  // P <= 16: done in registers
  }
}

// ---------------------------------------------------------------------------------------
// The m-point factor on every column b of the m x P view. Entries are template constants,
// so each output is a fixed chain of adds and subtracts.
//
// H_12 and H_20 (Paley I) are applied row by row (m - 1 additions per output). H_28 is
// Paley II, S (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]] with S the symmetric
// conference matrix of order 14: with u_C = x_2C + x_2C+1 and v_C = x_2C - x_2C+1,
//   y_2R = sum_C S[R][C] u_C + v_R   and   y_2R+1 = sum_C S[R][C] v_C - u_R.
// The 13 x 13 core of S is the circulant chi(R - C) of the quadratic character mod 13,
// whose +1 set {1, 3, 4, 9, 10, 12} is symmetric, so with w_c = a_{c+1} and W = sum_c w_c,
//   sum_C S[r+1][C] a_C = a_0 - W + w_r + 2 (w_{r-4} + w_{r-3} + w_{r+3} + w_{r+4} + w_{r-1} + w_{r+1})
// (indices mod 13), and the pair sums w_k + w_{k+1} are shared between rows: about 105
// additions per side instead of 14 * 13.
template <int M, int A, int C>
inline constexpr int kHad = hadamard_entry(M, A, C);

template <typename T, int M, int A, int... C>
__device__ __forceinline__ T hadamard_row(const T (&x)[M], std::integer_sequence<int, C...>) {
  T acc = 0;
  ((acc = (kHad<M, A, C> > 0) ? acc + x[C] : acc - x[C]), ...);
  return acc;
}

// One side of H_28 x (SIDE 0: the 14 outputs y_2R; SIDE 1: the outputs y_2R+1), each
// handed to put(R, y) as soon as it is computed (few registers live at once).
template <typename T, int SIDE, typename Put>
__device__ __forceinline__ void hadamard28_side(const T (&x)[28], Put put) {
  T u[14], v[14];
#pragma unroll
  for (int c = 0; c < 14; ++c) { u[c] = x[2 * c] + x[2 * c + 1]; v[c] = x[2 * c] - x[2 * c + 1]; }
  const T(&a)[14] = SIDE == 0 ? u : v;
  T W = a[1];
#pragma unroll
  for (int c = 2; c < 14; ++c) W += a[c];
  T pr[13];  // pr[k] = w_k + w_{k+1}
#pragma unroll
  for (int k = 0; k < 13; ++k) pr[k] = a[1 + k] + a[1 + (k + 1) % 13];
  const T base = a[0] - W;
  put(0, SIDE == 0 ? W + v[0] : W - u[0]);
#pragma unroll
  for (int r = 0; r < 13; ++r) {
    const T q = a[1 + (r + 12) % 13] + a[1 + (r + 1) % 13];
    const T A = pr[(r + 9) % 13] + pr[(r + 3) % 13] + q;
    const T sum = 2 * A + (base + a[1 + r]);
    put(r + 1, SIDE == 0 ? sum + v[r + 1] : sum - u[r + 1]);
  }
}

// H_m along the strided dimension of rows held in LDS (padding-free layout): row r of
// `nrows` rows of length M*P, element (a, b) at r*M*P + a*P + b; y[a][b] = sum_a'
// H_m[a][a'] x[a'][b], one column per thread: the rows of H_12 and H_20 as fixed chains of
// m - 1 adds and subtracts, H_28 by its Paley II structure (about 120 adds per side
// instead of 28 * 28 products). P is a power of two.
template <typename T, int M, int NT>
__device__ __forceinline__ void hadamard_m_lds(T* buf, int nrows, int P) {
  const int lp = __builtin_ctz(P);
  const int cols = nrows * P;
  for (int col = threadIdx.x; col < cols; col += NT) {
    const int r = col >> lp, b = col & (P - 1);
    T* base = buf + r * M * P + b;
    T x[M];
#pragma unroll
    for (int a = 0; a < M; ++a) x[a] = base[a * P];
    if constexpr (M == 28) {
      hadamard28_side<T, 0>(x, [&](int R, T y) { base[(2 * R) * P] = y; });
      hadamard28_side<T, 1>(x, [&](int R, T y) { base[(2 * R + 1) * P] = y; });
    } else {
      T y[M];
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ((y[A] = hadamard_row<T, M, A>(x, std::make_integer_sequence<int, M>{})), ...);
      }(std::make_integer_sequence<int, M>{});
#pragma unroll
      for (int a = 0; a < M; ++a) base[a * P] = y[a];
    }
  }
  __syncthreads();
}

// Full unnormalized H_K = H_m (x) H_P on `nrows` rows of length m*P held in LDS
// (padding-free layout, NT threads).
template <typename T, int NT>
__device__ __forceinline__ void hadamard_lds(T* buf, int nrows, int m, int P) {
  sylvester_lds<T>(buf, nrows * m * P, P);
  switch (m) {
    case 12: hadamard_m_lds<T, 12, NT>(buf, nrows, P); break;
    case 20: hadamard_m_lds<T, 20, NT>(buf, nrows, P); break;
    case 28: hadamard_m_lds<T, 28, NT>(buf, nrows, P); break;
    default: break;
  }
}

// Outputs of part Q of TPC parts of one column: rows a (or row pairs R) with
// a % TPC == Q. Q is a template constant, so only this part's rows are computed. For H_28
// TPC is 1 or 2, and part Q computes side Q. Element (a, b) goes to col[a * pstride], or
// with OUT to half index hb + half_off(a) of the sink: for P a multiple of 32,
// idx(a P + b) = a (P / 32) kChunkHalves + idx(b), and for P = 16 the offset of row a is
// (a / 2) kChunkHalves + 16 (a % 2); either way a uniform value, so no per-element index
// arithmetic (with P a template constant, PC > 0, an immediate offset).
template <typename T, int M, int TPC, int Q, bool OUT, int PC>
__device__ __forceinline__ void hadamard_part(T* col, int pstride, const T (&x)[M], int hb,
                                              int P, HalfSink sink) {
  const int Pv = PC > 0 ? PC : P;
  auto put = [&](int a, T v) {
    if constexpr (OUT) {
      const int off = Pv == 16 ? (a >> 1) * kChunkHalves + (a & 1) * 16
                               : a * ((Pv >> 5) * kChunkHalves);
      sink.put_at(hb + off, v);
    } else {
      col[a * pstride] = v;
    }
  };
  if constexpr (M == 28) {
    static_assert(TPC <= 2, "H_28 is split into at most two sides");
    if constexpr (TPC == 1 || Q == 0) hadamard28_side<T, 0>(x, [&](int R, T y) { put(2 * R, y); });
    if constexpr (TPC == 1 || Q == 1) hadamard28_side<T, 1>(x, [&](int R, T y) { put(2 * R + 1, y); });
  } else {
    [&]<int... A>(std::integer_sequence<int, A...>) {
      ((A % TPC == Q ? (put(A, hadamard_row<T, M, A>(x, std::make_integer_sequence<int, M>{})), 0)
                     : 0),
       ...);
    }(std::make_integer_sequence<int, M>{});
  }
}

// TPC threads per column (a power of two, the same for a whole wave when P >= 64); thread
// part q = t / P computes the outputs of its part. All inputs are read before any output is
// written; the function synchronizes at the end. With OUT the outputs go to the sink.
template <typename T, int M, int TPC, int NT, bool OUT, int PC = 0>
__device__ __forceinline__ void hadamard_factor_split(T* buf, int Pr, HalfSink sink) {
  const int P = PC > 0 ? PC : Pr;  // a template constant for the common row lengths
  // TPC == 1 loops over the columns when there are more columns than threads; with
  // TPC > 1 (P * TPC <= NT) there is one pass
  const int span = TPC == 1 ? P : NT;
  for (int t0 = 0; t0 < span; t0 += NT) {
    const int t = t0 + static_cast<int>(threadIdx.x);
    const bool active = t < P * TPC;
    const int q = t / P, b = t - q * P;
    T x[M];
    if (P % 16 == 0) {
      // element (a, b) is at pidx(a * P + b) = pidx(b) + a * (P + P / 16)
      const int pstride = P + (P >> 4);
      T* col = buf + pidx(b);
      if (active) {
#pragma unroll
        for (int a = 0; a < M; ++a) x[a] = col[a * pstride];
      }
      if constexpr (TPC > 1) __syncthreads();  // the other parts read the same inputs
      if (active) {
        const int hb = HalfSink::idx(b);
        [&]<int... Q>(std::integer_sequence<int, Q...>) {
          ((q == Q ? (hadamard_part<T, M, TPC, Q, OUT, PC>(col, pstride, x, hb, P, sink), 0) : 0),
           ...);
        }(std::make_integer_sequence<int, TPC>{});
      }
    } else if (active) {
      // rows shorter than 16 (only with TPC == 1): general indexing
#pragma unroll
      for (int a = 0; a < M; ++a) x[a] = buf[pidx(a * P + b)];
      T y[M];
      [&]<int... A>(std::integer_sequence<int, A...>) {
        ((y[A] = hadamard_row<T, M, A>(x, std::make_integer_sequence<int, M>{})), ...);
      }(std::make_integer_sequence<int, M>{});
#pragma unroll
      for (int a = 0; a < M; ++a) {
        if constexpr (OUT) sink.put_at(HalfSink::idx(a * P + b), y[a]);
        else buf[pidx(a * P + b)] = y[a];
      }
    }
  }
  __syncthreads();
}

template <typename T, int M, int NT, bool OUT>
__device__ __forceinline__ void hadamard_factor_m(T* buf, int P, HalfSink sink) {
  if (P < 64) {
    hadamard_factor_split<T, M, 1, NT, OUT>(buf, P, sink);
    return;
  }
  const int tpc = NT / P;  // 0 (more columns than threads) .. NT / 64, a power of two
  if constexpr (M == 28 && NT == 1024) {
    // K = 7168, the common 28-point width: every offset an immediate
    if (P == 256) {
      hadamard_factor_split<T, M, 2, NT, OUT, 256>(buf, P, sink);
      return;
    }
  }
  if constexpr (M == 28) {
    if (tpc >= 2) hadamard_factor_split<T, M, 2, NT, OUT>(buf, P, sink);
    else hadamard_factor_split<T, M, 1, NT, OUT>(buf, P, sink);
  } else {
    if (tpc >= 8) hadamard_factor_split<T, M, 8, NT, OUT>(buf, P, sink);
    else if (tpc == 4) hadamard_factor_split<T, M, 4, NT, OUT>(buf, P, sink);
    else if (tpc == 2) hadamard_factor_split<T, M, 2, NT, OUT>(buf, P, sink);
    else hadamard_factor_split<T, M, 1, NT, OUT>(buf, P, sink);
  }
}

template <typename T, int NT, bool OUT = false>
__device__ __forceinline__ void hadamard_factor(T* buf, int m, int P, HalfSink sink = {}) {
  switch (m) {
    case 12: hadamard_factor_m<T, 12, NT, OUT>(buf, P, sink); break;
    case 20: hadamard_factor_m<T, 20, NT, OUT>(buf, P, sink); break;
    case 28: hadamard_factor_m<T, 28, NT, OUT>(buf, P, sink); break;
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
