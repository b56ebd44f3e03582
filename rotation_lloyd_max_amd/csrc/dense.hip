// Dense rotations for input dimensions the Hadamard transform does not cover (VeloxQuant-MLX,
// "What already existed" and "Where the time actually went": a QR-derived orthogonal matrix
// for dimensions such as 4864): out = X R^T, i.e. every row x becomes R x, with R a caller-
// supplied K x K binary32 matrix. The product runs on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64): rows are converted exactly to fp64, products are exact, and the
// sums keep fp64 precision, so the encode that follows makes the same decisions as an fp64
// evaluation; activations are rounded once to their output type.
//
// Up to eight rows (decode) take k_dense_rot_vec, a streaming read of R. More rows:
// tiling: one 256-thread workgroup per 64 x 64 output tile, each wave a 32 x 32 quarter as
// 2 x 2 MFMA tiles; K in steps of 16 through LDS (rows padded to 17 values, so the 16 rows
// a fragment reads fall on distinct banks). Fragment layout of the 16x16x4 f64 instruction:
// lane l holds A[l % 16][l / 16] and B[l / 16][l % 16] and receives D[l / 16 + 4 r][l % 16]
// in its r-th result (unlike the 16-bit and f32 forms, whose rows are 4 (l / 16) + r).
#include "device_common.hpp"
#include "internal.hpp"

namespace tq {
namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kDrThreads = 256, kDrTile = 64, kDrStep = 16;

struct DenseParams {
  const void* x;
  const float* R;
  void* out;
  int64_t rows;
  int K;
};

template <int XDT>
__device__ __forceinline__ double dr_load(const void* x, int64_t i) {
  if constexpr (XDT == 3) return static_cast<const double*>(x)[i];
  else return static_cast<double>(load_elem<XDT>(x, i));
}

// ODT: 0 fp32, 1 bf16, 2 fp16, 3 fp64
template <int XDT, int ODT>
__global__ __launch_bounds__(kDrThreads) void k_dense_rot(DenseParams p) {
  __shared__ double xs[kDrTile][kDrStep + 1];
  __shared__ double rs[kDrTile][kDrStep + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kDrTile;
  const int n0 = blockIdx.x * kDrTile;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int K = p.K;
  f64x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < K; k0 += kDrStep) {
#pragma unroll
    for (int q = 0; q < kDrTile * kDrStep / kDrThreads; ++q) {
      const int idx = threadIdx.x + kDrThreads * q;
      const int r = idx / kDrStep, kk = idx % kDrStep;
      const int64_t m = m0 + r;
      const int n = n0 + r;
      xs[r][kk] = m < p.rows ? dr_load<XDT>(p.x, m * K + k0 + kk) : 0.0;
      rs[r][kk] = n < K ? static_cast<double>(p.R[static_cast<int64_t>(n) * K + k0 + kk]) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kDrStep; kk += 4) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = xs[wm + 16 * i + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = rs[wn + 16 * j + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + 16 * i + (lane >> 4) + 4 * r;
        const int n = n0 + wn + 16 * j + (lane & 15);
        if (m >= p.rows || n >= K) continue;
        const double v = acc[i][j][r];
        if constexpr (ODT == 3) static_cast<double*>(p.out)[m * K + n] = v;
        else store_any(p.out, ODT, m * K + n, static_cast<float>(v));
      }
}

// Few rows (decode): the product is a read of R, so one wave per output element i streams
// row i of R with coalesced 16-byte loads and multiplies it by up to kDrVecRows input rows
// held in LDS as fp64; fp64 sums as in k_dense_rot, reduced across the wave at the end.
constexpr int kDrVecRows = 8;
constexpr int kDrVecWaves = 4;

template <int XDT, int ODT>
__global__ __launch_bounds__(64 * kDrVecWaves) void k_dense_rot_vec(DenseParams p) {
  extern __shared__ double xv[];  // [rows][K]
  const int K = p.K, rows = static_cast<int>(p.rows);
  for (int i = threadIdx.x; i < rows * K; i += 64 * kDrVecWaves) xv[i] = dr_load<XDT>(p.x, i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kDrVecWaves + (threadIdx.x >> 6);
  if (n >= K) return;
  const float* rrow = p.R + static_cast<int64_t>(n) * K;
  double acc[kDrVecRows];
#pragma unroll
  for (int t = 0; t < kDrVecRows; ++t) acc[t] = 0.0;
  for (int k = 4 * lane; k < K; k += 256) {
    const float4 r = *reinterpret_cast<const float4*>(rrow + k);
    const double rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int t = 0; t < kDrVecRows; ++t) {
      if (t >= rows) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[t] = __builtin_fma(rv[q], xv[t * K + k + q], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kDrVecRows; ++t) {
    if (t >= rows) break;
    double v = acc[t];
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) {
      if constexpr (ODT == 3) static_cast<double*>(p.out)[static_cast<int64_t>(t) * K + n] = v;
      else store_any(p.out, ODT, static_cast<int64_t>(t) * K + n, static_cast<float>(v));
    }
  }
}

template <int XDT>
hipError_t launch_dr_vec(const DenseParams& p, int odt, hipStream_t s) {
  const dim3 grid((p.K + kDrVecWaves - 1) / kDrVecWaves);
  const size_t lds = static_cast<size_t>(p.rows) * p.K * 8;
  void (*k)(DenseParams) = odt == 0 ? k_dense_rot_vec<XDT, 0>
                           : odt == 1 ? k_dense_rot_vec<XDT, 1>
                           : odt == 2 ? k_dense_rot_vec<XDT, 2> : k_dense_rot_vec<XDT, 3>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, grid, dim3(64 * kDrVecWaves), lds, s, p);
  return hipGetLastError();
}

template <int XDT>
hipError_t launch_dr_x(const DenseParams& p, int odt, hipStream_t s) {
  // up to kDrVecRows rows whose fp64 copies fit LDS: the streaming product
  if (p.rows <= kDrVecRows && p.rows * p.K * 8 <= 160 * 1024) return launch_dr_vec<XDT>(p, odt, s);
  const dim3 grid((p.K + kDrTile - 1) / kDrTile, static_cast<unsigned>((p.rows + kDrTile - 1) / kDrTile));
  switch (odt) {
    case 0: hipLaunchKernelGGL((k_dense_rot<XDT, 0>), grid, dim3(kDrThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL((k_dense_rot<XDT, 1>), grid, dim3(kDrThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_dense_rot<XDT, 2>), grid, dim3(kDrThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((k_dense_rot<XDT, 3>), grid, dim3(kDrThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

// out = x R^T for `rows` rows of length K; xdt 0/1/2 (fp32/bf16/fp16), odt 0/1/2 or 3 (fp64).
hipError_t launch_dense_rot(const void* x, int xdt, int64_t rows, int K, const float* R, void* out,
                            int odt, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if ((rows + kDrTile - 1) / kDrTile > 65535) return hipErrorInvalidValue;
  DenseParams p{x, R, out, rows, K};
  switch (xdt) {
    case 0: return launch_dr_x<0>(p, odt, s);
    case 1: return launch_dr_x<1>(p, odt, s);
    default: return launch_dr_x<2>(p, odt, s);
  }
}

}  // namespace tq
