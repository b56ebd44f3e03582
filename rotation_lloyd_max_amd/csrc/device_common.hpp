// Device-side building blocks shared by the libtq kernels (gfx950, wave64).
//
// * SplitMix64 counter form for the rotation signs.
// * The m-point Hadamard factors (Paley I for m = 12, 20; Paley II for m = 28) as
//   compile-time sign tables, and the Sylvester transform as radix-2^r butterfly passes
//   over a row held in LDS. Together they apply H_K = H_m (x) H_{2^k}, the Hadamard matrix
//   of the rotation in turboquant-mlx "How it works", "Quantizing a weight, with no data"
//   (first bullet) and "Running a quantized layer" (the input is rotated the same way).
// * fp16 / bf16 conversions with explicit rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kBlock = 256;  // threads per workgroup for every libtq kernel

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// three words at a 4-byte aligned address (a 3-bit chunk): one 12-byte load
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Rotation signs: SplitMix64 output i of the generator seeded with `seed` is
// mix64(seed + (i + 1) * golden_gamma); s_i = -1 when its top bit is set.
__host__ __device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------------------
// m-point Hadamard factors, evaluated at compile time.
//   chi: quadratic character mod prime q; Jacobsthal Q[a][b] = chi(a - b).
//   Paley I  (q = 3 mod 4): H = I + [[0, 1^T], [-1, Q]]                    order q + 1
//   Paley II (q = 1 mod 4): H = S (x) [[1,1],[1,-1]] + I (x) [[1,-1],[-1,-1]],
//                           S = [[0, 1^T], [1, Q]]                          order 2(q + 1)
constexpr int qchar(int a, int q) {
  a %= q;
  if (a < 0) a += q;
  if (a == 0) return 0;
  for (int x = 1; x < q; ++x)
    if ((x * x) % q == a) return 1;
  return -1;
}

constexpr int paley1_entry(int q, int r, int c) {
  int cm = 0;
  if (r == 0 && c == 0) cm = 0;
  else if (r == 0) cm = 1;
  else if (c == 0) cm = -1;
  else cm = qchar((r - 1) - (c - 1), q);
  return (r == c ? 1 : 0) + cm;
}

constexpr int paley2_entry(int q, int r, int c) {
  const int R = r / 2, C = c / 2, i = r % 2, j = c % 2;
  int s = 0;
  if (R == 0 && C == 0) s = 0;
  else if (R == 0 || C == 0) s = 1;
  else s = qchar((R - 1) - (C - 1), q);
  const int a = (i == 1 && j == 1) ? -1 : 1;  // [[1, 1], [1, -1]]
  const int b = (i == 0 && j == 0) ? 1 : -1;  // [[1, -1], [-1, -1]]
  return s * a + (R == C ? b : 0);
}

constexpr int hadamard_entry(int m, int r, int c) {
  return m == 1 ? 1 : m == 12 ? paley1_entry(11, r, c)
                    : m == 20 ? paley1_entry(19, r, c)
                              : paley2_entry(13, r, c);
}

template <int M>
struct HadamardFactor {
  float sgn[M][M];  // H_m[r][c] as +-1.0f
  constexpr HadamardFactor() : sgn{} {
    for (int r = 0; r < M; ++r)
      for (int c = 0; c < M; ++c) sgn[r][c] = hadamard_entry(M, r, c) < 0 ? -1.0f : 1.0f;
  }
};

template <int M>
struct HadamardTable {
  static constexpr HadamardFactor<M> value{};
};

// ---------------------------------------------------------------------------------------
// Sylvester transform (unnormalized) along contiguous runs of length P (a power of two)
// of buf[0 .. total), in place in LDS, by radix-2^R passes: a pass of stride h combines
// the 2^R elements base + j*h, doing R butterfly stages in registers. All threads of the
// block take part; the caller synchronizes before and the function synchronizes after
// every pass.
template <typename T, int R>
__device__ __forceinline__ void sylvester_pass(T* buf, int total, int h) {
  constexpr int n = 1 << R;
  const int ngroups = total >> R;
  const int lh = __builtin_ctz(h);  // h is a power of two
  for (int g = threadIdx.x; g < ngroups; g += kBlock) {
    const int blk = g >> lh, off = g & (h - 1);
    T* base = buf + blk * (h << R) + off;
    T v[n];
#pragma unroll
    for (int j = 0; j < n; ++j) v[j] = base[j * h];
#pragma unroll
    for (int s = 0; s < R; ++s) {
#pragma unroll
      for (int j = 0; j < n; ++j) {
        if ((j >> s) & 1) continue;
        const T a = v[j], b = v[j + (1 << s)];
        v[j] = a + b;
        v[j + (1 << s)] = a - b;
      }
    }
#pragma unroll
    for (int j = 0; j < n; ++j) base[j * h] = v[j];
  }
  __syncthreads();
}

// Stages h0, 2*h0, ..., P/2 (the stages below h0 already applied by the caller).
template <typename T>
__device__ __forceinline__ void sylvester_lds(T* buf, int total, int P, int h0 = 1) {
  int h = h0;
  while (h < P) {
    const int left = __builtin_ctz(P / h);
    if (left >= 4) { sylvester_pass<T, 4>(buf, total, h); h <<= 4; }
    else if (left == 3) { sylvester_pass<T, 3>(buf, total, h); h <<= 3; }
    else if (left == 2) { sylvester_pass<T, 2>(buf, total, h); h <<= 2; }
    else { sylvester_pass<T, 1>(buf, total, h); h <<= 1; }
  }
}

// ---------------------------------------------------------------------------------------
// Conversions.
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even; the hardware conversion (v_cvt_pk_bf16_f32 on gfx950), NaN stays NaN
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint16_t float_to_half_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// fp64 -> fp16 bits, round to nearest even in one step (no double rounding through fp32),
// saturating at 65504. Input is >= 0 (an RMS) or NaN.
__device__ __forceinline__ uint16_t double_to_half_rne_sat(double r) {
  if (!(r < 65520.0)) return (r != r) ? 0x7e00 : 0x7bff;
  if (r <= 0.0) return 0;
  const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(r));
  const int e = static_cast<int>((bits >> 52) & 0x7ff) - 1023;
  const uint64_t mant = (bits & ((1ull << 52) - 1)) | ((bits >> 52) & 0x7ff ? (1ull << 52) : 0);
  // drop `shift` low bits of the 53-bit significand: normal results keep 11 bits,
  // subnormal ones are multiples of 2^-24
  const int shift = (e >= -14) ? 42 : (28 - e);
  uint64_t q;
  if (shift >= 64) {
    q = 0;
  } else {
    q = mant >> shift;
    const uint64_t rem = mant & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
  }
  if (e >= -14) return static_cast<uint16_t>(((e + 15) << 10) + static_cast<int>(q) - 1024);
  return static_cast<uint16_t>(q);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (DT == 0) return static_cast<const float*>(p)[i];
  else if constexpr (DT == 1) return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
  else return half_bits_to_float(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ float load_any(const void* p, int dt, int64_t i) {
  return dt == 0 ? load_elem<0>(p, i) : dt == 1 ? load_elem<1>(p, i) : load_elem<2>(p, i);
}

__device__ __forceinline__ void store_any(void* p, int dt, int64_t i, float v) {
  if (dt == 0) static_cast<float*>(p)[i] = v;
  else if (dt == 1) static_cast<uint16_t*>(p)[i] = float_to_bf16_rne(v);
  else static_cast<uint16_t*>(p)[i] = float_to_half_rne(v);
}

// A load at a 32-bit byte offset from a uniform base: a single global load with a scalar
// base address and a 32-bit vector offset (no 64-bit address arithmetic per lane).
template <typename T>
__device__ __forceinline__ T ld_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off);
}

// The same load with the nontemporal hint, for the qmv kernels' packed codes and scales,
// which a call reads once: on gfx950 such a stream completes sooner (a 6.5 MB decode-layer
// call measured 8 % faster). The matrix kernels keep plain loads: there the hint measured
// slower (their codes are reread by other row tiles, or read by coalesced 4-byte loads).
// T must be a scalar or an ext_vector type.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* base, uint32_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off));
}

}  // namespace tq
