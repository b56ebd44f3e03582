// gather_qmm: batched gather-GEMM over rows sorted by expert,
//   y[m] = W_e R x[row_token[m]]   for offsets[e] <= m < offsets[e+1].
//
// turboquant-mlx "How it works", "Running a quantized layer", kernel table, third row (a
// large batch sorted by expert). Three launches on the caller's stream:
//   1. rotate the T input rows once into a bf16 workspace (x' = R x);
//   2. a tile schedule: tile_start[e] = sum over experts before e of ceil(rows_e / BM);
//   3. the GEMM: one workgroup per (row tile of one expert, BN output columns). Weights
//      are decoded (centroid * group scale, rounded to bf16) into an LDS tile, the routed
//      input rows are gathered into another, and bf16 MFMA 16x16x32 accumulates in fp32.
#include "device_common.hpp"
#include "internal.hpp"

namespace tq {

constexpr int kBM = 64, kBN = 64, kBK = 32, kLdsK = kBK + 8;

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

size_t gather_qmm_workspace(const WeightArgs& w, int64_t M, int64_t T) {
  (void)M;
  return align256(static_cast<size_t>(T) * w.K * 2) + align256(static_cast<size_t>(w.E + 1) * 4);
}

__global__ void k_schedule(const int32_t* offsets, int E, int32_t* tile_start) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int acc = 0;
  for (int e = 0; e < E; ++e) {
    tile_start[e] = acc;
    const int rows = offsets[e + 1] - offsets[e];
    acc += rows > 0 ? (rows + kBM - 1) / kBM : 0;
  }
  tile_start[E] = acc;
}

__global__ __launch_bounds__(kBlock) void k_to_bf16(const void* x, int xdt, int64_t n, uint16_t* out) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock)
    out[i] = float_to_bf16_rne(load_any(x, xdt, i));
}

struct QmmParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* xr;  // bf16 [T][K], rotated
  const int32_t* row_token;
  const int32_t* offsets;
  const int32_t* tile_start;
  void* y;
  int64_t T, M;
  int K, N, E, wpr, group, ydt;
  CodebookArgs cb;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Codebook indices of the 8 elements j0 .. j0+7 of a packed row (j0 a multiple of 8).
template <int L>
__device__ __forceinline__ void decode8(const uint32_t* crow, int j0, int (&idx)[8]) {
  if constexpr (L == 16) {
    const uint32_t w = crow[j0 >> 3];
#pragma unroll
    for (int k = 0; k < 8; ++k) idx[k] = (w >> (4 * k)) & 15;
  } else if constexpr (L == 4) {
    const uint32_t w = crow[j0 >> 4] >> (2 * (j0 & 15));
#pragma unroll
    for (int k = 0; k < 8; ++k) idx[k] = (w >> (2 * k)) & 3;
  } else if constexpr (L == 8) {
    const int bit = 3 * j0, lo = bit >> 5, sh = bit & 31;
    uint64_t v = crow[lo] >> sh;
    if (sh > 8) v |= static_cast<uint64_t>(crow[lo + 1]) << (32 - sh);
#pragma unroll
    for (int k = 0; k < 8; ++k) idx[k] = static_cast<int>((v >> (3 * k)) & 7);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      uint32_t w = crow[j / 20];
      for (int d = j % 20; d > 0; --d) w /= 3u;
      idx[k] = static_cast<int>(w % 3u);
    }
  }
}

template <int L>
__global__ __launch_bounds__(kBlock) void k_gqmm(QmmParams p) {
  const int t = blockIdx.x;
  const int total = p.tile_start[p.E];
  if (t >= total) return;
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tile_start[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int m0 = p.offsets[e] + (t - p.tile_start[e]) * kBM;
  int mrows = p.offsets[e + 1] - m0;
  if (mrows > kBM) mrows = kBM;
  if (m0 < 0 || m0 >= p.M) return;  // inconsistent offsets: never touch memory past y
  if (mrows > p.M - m0) mrows = static_cast<int>(p.M - m0);
  const int n0 = blockIdx.y * kBN;

  __shared__ uint16_t As[kBM * kLdsK];
  __shared__ uint16_t Bs[kBN * kLdsK];
  __shared__ int tok[kBM];
  __shared__ float cent[16];
  const int tid = threadIdx.x;
  if (tid < kBM) {
    int v = -1;  // -1: padding row of the tile; -2: token id out of range (row of NaN)
    if (tid < mrows) {
      v = p.row_token[m0 + tid];
      if (v < 0 || v >= p.T) v = -2;
    }
    tok[tid] = v;
  }
  if (tid < 16) cent[tid] = tid < p.cb.levels ? p.cb.c[tid] : 0.f;
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lr = tid >> 2, seg = tid & 3;  // loader row and 8-element segment
  const int ngroups = p.K / p.group;
  const int nrow = n0 + lr;
  const bool nvalid = nrow < p.N;
  const int64_t wrow = static_cast<int64_t>(e) * p.N + (nvalid ? nrow : 0);
  const uint32_t* crow = p.codes + wrow * p.wpr;
  const uint16_t* srow = p.scales + wrow * ngroups;
  const int tk = tok[lr];

  for (int k0 = 0; k0 < p.K; k0 += kBK) {
    const int j0 = k0 + 8 * seg;
    uint4 a = {0u, 0u, 0u, 0u};
    if (tk >= 0) a = *reinterpret_cast<const uint4*>(p.xr + static_cast<int64_t>(tk) * p.K + j0);
    *reinterpret_cast<uint4*>(&As[lr * kLdsK + 8 * seg]) = a;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (nvalid) {
      int idx[8];
      decode8<L>(crow, j0, idx);
      const float sc = half_bits_to_float(srow[j0 / p.group]);
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        const uint32_t lo16 = float_to_bf16_rne(cent[idx[k]] * sc);
        const uint32_t hi16 = float_to_bf16_rne(cent[idx[k + 1]] * sc);
        packed[k >> 1] = lo16 | (hi16 << 16);
      }
    }
    *reinterpret_cast<uint4*>(&Bs[lr * kLdsK + 8 * seg]) = uint4{packed[0], packed[1], packed[2], packed[3]};
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int arow = 32 * wm + 16 * i + (lane & 15);
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&As[arow * kLdsK + 8 * (lane >> 4)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int brow = 32 * wn + 16 * j + (lane & 15);
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&Bs[brow * kLdsK + 8 * (lane >> 4)]);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 32 * wm + 16 * i + 4 * (lane >> 4) + r;
        const int col = n0 + 32 * wn + 16 * j + (lane & 15);
        if (row < mrows && col < p.N)
          store_any(p.y, p.ydt, static_cast<int64_t>(m0 + row) * p.N + col,
                    tok[row] == -2 ? __builtin_nanf("") : acc[i][j][r]);
      }
}

hipError_t launch_gather_qmm(const WeightArgs& w, const void* x, int xdt, int64_t T,
                             const int32_t* row_token, const int32_t* offsets, int64_t M,
                             bool x_rotated, void* y, int ydt, void* ws, hipStream_t s) {
  if (M == 0 || w.N == 0) return hipSuccess;
  uint16_t* xr = static_cast<uint16_t*>(ws);
  int32_t* tile_start = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                                   align256(static_cast<size_t>(T) * w.K * 2));
  hipError_t err;
  if (!x_rotated) {
    err = launch_fwht(x, xdt, T, w.K, w.m, w.P, w.signs, 0, xr, 1, s);
  } else if (xdt == 1) {
    xr = const_cast<uint16_t*>(static_cast<const uint16_t*>(x));
    err = hipSuccess;
  } else {
    const int64_t n = T * w.K;
    const int grid = static_cast<int>((n + kBlock - 1) / kBlock < 65536 ? (n + kBlock - 1) / kBlock : 65536);
    hipLaunchKernelGGL(k_to_bf16, dim3(grid > 0 ? grid : 1), dim3(kBlock), 0, s, x, xdt, n, xr);
    err = hipGetLastError();
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(64), 0, s, offsets, w.E, tile_start);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  QmmParams p{};
  p.codes = w.codes; p.scales = w.scales; p.xr = xr; p.row_token = row_token;
  p.offsets = offsets; p.tile_start = tile_start; p.y = y;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group; p.ydt = ydt;
  p.T = T; p.M = M;
  p.cb = *codebook_for(w.levels);
  const int gx = static_cast<int>((M + kBM - 1) / kBM + w.E);
  const int gy = (w.N + kBN - 1) / kBN;
  switch (w.levels) {
    case 16: hipLaunchKernelGGL(k_gqmm<16>, dim3(gx, gy), dim3(kBlock), 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_gqmm<8>, dim3(gx, gy), dim3(kBlock), 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_gqmm<4>, dim3(gx, gy), dim3(kBlock), 0, s, p); break;
    default: hipLaunchKernelGGL(k_gqmm<3>, dim3(gx, gy), dim3(kBlock), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace tq
