// Encode kernel: rotate -> group RMS -> fp16 scale -> snap -> pack, one row at a time per
// workgroup (grid-stride over rows). Power-of-two rows up to 4096 take k_encode_p2
// (encode_p2.hip) and rows of 12, 20 or 28 times 32 .. 256 take k_encode_m (encode_m.hip);
// this kernel takes the other lengths (rows of 8192, factors with fewer than 32 or more
// than 256 columns), power-of-two sources not 16-byte aligned, trit rows of 4096, and
// rows already rotated by a dense rotation.
//
// Steps (turboquant-mlx "How it works", "Quantizing a weight, with no data"; "The ternary
// tier (1.58 bits)"):
//   v = H_K (s * w) (unnormalized; the 1/sqrt(K) of R cancels in v / r and is applied
//   to the stored scale only), r = sqrt(mean_g v^2), scale = fp16(r / sqrt(K)),
//   u = v / r (0 when r = 0), idx = #{k : u > t_k} decided in binary32, then bit or trit
//   packing. Rotation and RMS are computed in double precision, so the decision sees the
//   same u, to within a few units of the 53-bit significand, as an fp64 evaluation.
#include "device_common.hpp"
#include "fwht_block.hpp"
#include "internal.hpp"

namespace tq {

__device__ __forceinline__ void fill_sign_words(uint32_t* sb, int K, uint64_t seed) {
  const int nw = (K + 31) / 32;
  for (int w = threadIdx.x; w < nw; w += kBlock) {
    uint32_t b = 0;
    for (int j = 0; j < 32; ++j) {
      const int i = 32 * w + j;
      if (i < K && (splitmix64_at(seed, static_cast<uint64_t>(i)) >> 63)) b |= 1u << j;
    }
    sb[w] = b;
  }
}

template <int WDT, int LEVELS>
__global__ __launch_bounds__(kBlock) void k_encode(const void* W, int64_t rows, int K, int m,
                                                   int P, int group, uint64_t seed,
                                                   CodebookArgs cb, uint32_t* codes,
                                                   uint16_t* scales, int wpr,
                                                   double inv_sqrt_k) {
  constexpr int nthr = LEVELS - 1;
  extern __shared__ double smem_d[];
  const int run = group < 16 ? group : 16;  // run of consecutive elements per partial sum
  const int ngroups = K / group;
  double* v = smem_d;                  // K
  double* part = v + K;                // K / run
  double* rinv = part + K / run;       // K / group
  uint32_t* sb = reinterpret_cast<uint32_t*>(rinv + ngroups);  // ceil(K / 32)
  uint8_t* idx = reinterpret_cast<uint8_t*>(sb + (K + 31) / 32);  // K

  // WDT 3: rows already rotated (fp64, a dense rotation applied by k_dense_rot): no signs,
  // no Hadamard transform, and the caller passes inv_sqrt_k = 1
  if constexpr (WDT != 3) fill_sign_words(sb, K, seed);
  __syncthreads();

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t base = row * K;
    for (int i = threadIdx.x; i < K; i += kBlock) {
      if constexpr (WDT == 3) {
        v[i] = static_cast<const double*>(W)[base + i];
      } else {
        const double w = static_cast<double>(load_elem<WDT>(W, base + i));
        v[i] = ((sb[i >> 5] >> (i & 31)) & 1u) ? -w : w;
      }
    }
    __syncthreads();
    if constexpr (WDT != 3) hadamard_lds<double, kBlock>(v, 1, m, P);

    // group sums of squares: partial sums over runs, then per group
    for (int r = threadIdx.x; r < K / run; r += kBlock) {
      double s = 0.0;
      for (int j = 0; j < run; ++j) {
        const double a = v[r * run + j];
        s += a * a;
      }
      part[r] = s;
    }
    __syncthreads();
    const int per = group / run;
    for (int g = threadIdx.x; g < ngroups; g += kBlock) {
      double s = 0.0;
      for (int j = 0; j < per; ++j) s += part[g * per + j];
      const double rr = __builtin_sqrt(s / group);  // RMS of the unnormalized rotated group
      scales[row * ngroups + g] = double_to_half_rne_sat(rr * inv_sqrt_k);
      rinv[g] = rr > 0.0 ? 1.0 / rr : 0.0;
    }
    __syncthreads();

    // snap: count thresholds below u, in binary32
    const int lg_group = __builtin_ctz(group);  // groups are powers of two
    for (int i = threadIdx.x; i < K; i += kBlock) {
      const float u = static_cast<float>(v[i] * rinv[i >> lg_group]);
      int q = 0;
#pragma unroll
      for (int k = 0; k < nthr; ++k) q += (u > cb.t[k]) ? 1 : 0;
      idx[i] = static_cast<uint8_t>(q);
    }
    __syncthreads();

    // pack
    uint32_t* crow = codes + row * static_cast<int64_t>(wpr);
    for (int wd = threadIdx.x; wd < wpr; wd += kBlock) {
      uint32_t word = 0;
      if constexpr (LEVELS == 3) {
        for (int k = 19; k >= 0; --k) {
          const int j = 20 * wd + k;
          word = word * 3u + (j < K ? idx[j] : 0u);
        }
      } else {
        constexpr int b = LEVELS == 4 ? 2 : LEVELS == 8 ? 3 : 4;
        const int j0 = (32 * wd) / b;
        int j1 = (32 * wd + 31) / b;
        if (j1 > K - 1) j1 = K - 1;
        uint64_t acc = 0;
        for (int j = j0; j <= j1; ++j) acc |= static_cast<uint64_t>(idx[j]) << (b * (j - j0));
        word = static_cast<uint32_t>(acc >> (32 * wd - b * j0));
      }
      crow[wd] = word;
    }
    __syncthreads();
  }
}

template <int WDT>
static hipError_t launch_encode_l(const void* W, int64_t rows, int K, int m, int P, int levels,
                                  int group, uint64_t seed, uint32_t* codes, uint16_t* scales,
                                  hipStream_t s) {
  const CodebookArgs* cb = codebook_for(levels);
  const int run = group < 16 ? group : 16;
  const size_t lds = static_cast<size_t>(K) * 8 + (K / run) * 8 + (K / group) * 8 +
                     ((K + 31) / 32) * 4 + K;
  int wpr = levels == 3 ? (K + 19) / 20 : (K * (levels == 4 ? 2 : levels == 8 ? 3 : 4) + 31) / 32;
  const int grid = static_cast<int>(rows < 4096 ? rows : 4096);
  const double isk = WDT == 3 ? 1.0 : 1.0 / __builtin_sqrt(static_cast<double>(K));
  void (*kern)(const void*, int64_t, int, int, int, int, uint64_t, CodebookArgs, uint32_t*,
               uint16_t*, int, double) = nullptr;
  switch (levels) {
    case 3: kern = k_encode<WDT, 3>; break;
    case 4: kern = k_encode<WDT, 4>; break;
    case 8: kern = k_encode<WDT, 8>; break;
    default: kern = k_encode<WDT, 16>; break;
  }
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), lds, s, W, rows, K, m, P, group, seed, *cb,
                     codes, scales, wpr, isk);
  return hipGetLastError();
}

hipError_t launch_encode(const void* W, int wdt, int64_t rows, int K, int m, int P, int levels,
                         int group, uint64_t seed, uint32_t* codes, uint16_t* scales,
                         hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // power-of-two rows up to 4096 long, read with 16-byte loads: the register kernel
  if (encode_p2_supported(K, m, levels) && (reinterpret_cast<uintptr_t>(W) & 15) == 0)
    return launch_encode_p2(W, wdt, rows, K, levels, group, seed, codes, scales, s);
  // rows of 12, 20 or 28 times 32 .. 256: the register kernel with the m-point factor
  if (encode_m_supported(K, m))
    return launch_encode_m(W, wdt, rows, K, m, levels, group, seed, codes, scales, s);
  switch (wdt) {
    case 0: return launch_encode_l<0>(W, rows, K, m, P, levels, group, seed, codes, scales, s);
    case 1: return launch_encode_l<1>(W, rows, K, m, P, levels, group, seed, codes, scales, s);
    default: return launch_encode_l<2>(W, rows, K, m, P, levels, group, seed, codes, scales, s);
  }
}

hipError_t launch_encode_rotated(const double* V, int64_t rows, int K, int levels, int group,
                                 uint32_t* codes, uint16_t* scales, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  return launch_encode_l<3>(V, rows, K, 1, K, levels, group, 0, codes, scales, s);
}

}  // namespace tq
