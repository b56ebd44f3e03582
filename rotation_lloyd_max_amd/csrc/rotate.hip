// Rotation kernels: sign bits and the stand-alone row rotation out = R x.
//
// R = H_K diag(s) / sqrt(K) (turboquant-mlx "How it works", "Quantizing a weight, with no
// data", first bullet; "Running a quantized layer": the layer's input gets the same
// rotation as the weight rows). One workgroup rotates one row at a time in LDS, in fp32,
// looping over rows with a grid stride.
#include "device_common.hpp"
#include "fwht_block.hpp"
#include "internal.hpp"

namespace tq {

__global__ __launch_bounds__(kBlock) void k_signs(uint64_t seed, int K, uint32_t* bits) {
  const int nw = (K + 31) / 32;
  for (int w = blockIdx.x * kBlock + threadIdx.x; w < nw; w += gridDim.x * kBlock) {
    uint32_t b = 0;
    for (int j = 0; j < 32; ++j) {
      const int i = 32 * w + j;
      if (i < K && (splitmix64_at(seed, static_cast<uint64_t>(i)) >> 63)) b |= 1u << j;
    }
    bits[w] = b;
  }
}

hipError_t launch_signs(uint64_t seed, int K, uint32_t* bits, hipStream_t s) {
  const int nw = (K + 31) / 32;
  const int grid = (nw + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_signs, dim3(grid), dim3(kBlock), 0, s, seed, K, bits);
  return hipGetLastError();
}

// Fill sign words for (seed, K) into LDS, from `signbits` when given.
__device__ __forceinline__ void load_sign_words(uint32_t* sb, int K, const uint32_t* signbits,
                                       uint64_t seed) {
  const int nw = (K + 31) / 32;
  for (int w = threadIdx.x; w < nw; w += kBlock) {
    if (signbits) {
      sb[w] = signbits[w];
    } else {
      uint32_t b = 0;
      for (int j = 0; j < 32; ++j) {
        const int i = 32 * w + j;
        if (i < K && (splitmix64_at(seed, static_cast<uint64_t>(i)) >> 63)) b |= 1u << j;
      }
      sb[w] = b;
    }
  }
}

template <int XDT>
__global__ __launch_bounds__(kBlock) void k_fwht(const void* x, int64_t rows, int K, int m,
                                                 int P, const uint32_t* signbits,
                                                 uint64_t seed, void* out, int odt,
                                                 float inv_sqrt_k) {
  extern __shared__ float smem_f[];
  float* buf = smem_f;
  uint32_t* sb = reinterpret_cast<uint32_t*>(buf + K);
  load_sign_words(sb, K, signbits, seed);
  __syncthreads();
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * K;
    for (int i = threadIdx.x; i < K; i += kBlock) {
      const float v = load_elem<XDT>(x, base + i);
      buf[i] = ((sb[i >> 5] >> (i & 31)) & 1u) ? -v : v;
    }
    __syncthreads();
    hadamard_lds<float, kBlock>(buf, 1, m, P);
    for (int i = threadIdx.x; i < K; i += kBlock) store_any(out, odt, base + i, buf[i] * inv_sqrt_k);
    __syncthreads();
  }
}

hipError_t launch_fwht(const void* x, int xdt, int64_t rows, int K, int m, int P,
                       const uint32_t* signbits, uint64_t seed, void* out, int odt,
                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const size_t lds = static_cast<size_t>(K) * 4 + ((K + 31) / 32) * 4;
  const int grid = static_cast<int>(rows < 4096 ? rows : 4096);
  const float isk = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(K)));
  switch (xdt) {
    case 0: hipLaunchKernelGGL(k_fwht<0>, dim3(grid), dim3(kBlock), lds, s, x, rows, K, m, P, signbits, seed, out, odt, isk); break;
    case 1: hipLaunchKernelGGL(k_fwht<1>, dim3(grid), dim3(kBlock), lds, s, x, rows, K, m, P, signbits, seed, out, odt, isk); break;
    default: hipLaunchKernelGGL(k_fwht<2>, dim3(grid), dim3(kBlock), lds, s, x, rows, K, m, P, signbits, seed, out, odt, isk); break;
  }
  return hipGetLastError();
}

}  // namespace tq
