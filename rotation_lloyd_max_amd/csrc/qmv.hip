// qmv and gather_qmv: y = W R x with W decoded inline from packed codes.
//
// turboquant-mlx "How it works", "Running a quantized layer": the layer rotates its input
// and multiplies by the packed weights, decoding them inline, so full-precision weights
// never exist in memory: y_i = sum_g scale_{i,g} sum_{j in g} c[idx_ij] x'_j. The kernel
// table of that section has gather_qmv for one token, each routed expert reading the
// same (shared) input.
//
// Work split. Every workgroup rotates x itself (LDS, fp32), scales it by a power of two
// so that its largest entry lies in [2^14, 2^15), and keeps it as fp16 pairs in LDS. It
// then streams a contiguous range of output rows: a row is split into chunks (32
// elements, or one 20-trit word), lanes of a wave take chunks with a stride, decode them
// through LDS tables into fp16 centroid pairs and accumulate v_dot2 products in fp32;
// each group's partial sum is multiplied by its fp16 scale. A row is finished by a
// butterfly reduction over the lanes that shared it.
#include "decode_common.hpp"
#include "internal.hpp"

namespace tq {

struct QmvParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  const int32_t* ids;
  const void* x;
  void* y;
  int K, N, E, wpr, group, m, P;
  int n_slots;  // routed experts (1 for a dense qmv)
  int xdt, ydt, rotated;
  int Q;        // chunks per row
  int lpr_log;  // log2(lanes per row)
  int rows_per_block;
  float inv_sqrt_k;
  CodebookArgs cb;
};

// Rotate one input vector into fp16 pairs (xh2, Q*ce/2 words, zero past K). Uses xf (K
// floats), red (32 floats) and sb (sign words) as scratch. Returns the factor that maps
// accumulated products back to y: 2^-e, times 1/sqrt(K) when the input was rotated here.
template <int XDT>
__device__ __forceinline__ float prepare_input(const void* x, int64_t xoff, int K, int m, int P,
                                      bool rotated, const uint32_t* sb, float* xf, float* red,
                                      uint32_t* xh2, int xwords, float inv_sqrt_k) {
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    float v = load_elem<XDT>(x, xoff + i);
    if (!rotated && ((sb[i >> 5] >> (i & 31)) & 1u)) v = -v;
    xf[i] = v;
  }
  __syncthreads();
  if (!rotated) hadamard_lds<float>(xf, 1, m, P);
  float mx = 0.f;
  for (int i = threadIdx.x; i < K; i += blockDim.x) mx = fmaxf(mx, fabsf(xf[i]));
  mx = block_max(mx, red);
  int ex = 0;
  if (mx > 0.f && mx <= 3.0e38f) {
    ex = 14 - ilogbf(mx);
    ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  }
  const float sc = ldexpf(1.f, ex);
  for (int q = threadIdx.x; q < xwords; q += blockDim.x) {
    const int i0 = 2 * q, i1 = 2 * q + 1;
    const float a = i0 < K ? xf[i0] * sc : 0.f;
    const float b = i1 < K ? xf[i1] * sc : 0.f;
    xh2[q] = static_cast<uint32_t>(float_to_half_rne(a)) |
             (static_cast<uint32_t>(float_to_half_rne(b)) << 16);
  }
  __syncthreads();
  return ldexpf(1.f, -ex) * (rotated ? 1.f : inv_sqrt_k);
}

// Load the words of chunk c of a packed row (zeros when !ok).
template <int L>
__device__ __forceinline__ void load_chunk(const uint32_t* crow, int c, bool ok, uint32_t (&w)[Fmt<L>::cw]) {
  using F = Fmt<L>;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < F::cw; ++i) w[i] = 0;
    return;
  }
  const uint32_t* p = crow + c * F::cw;
  if constexpr (L == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (L == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < F::cw; ++i) w[i] = p[i];
  }
}

// Group layout of chunk c: scale indices g0, g1 and the first pair that uses g1.
template <int L>
__device__ __forceinline__ void chunk_groups(int c, int group, int ngroups, int& g0, int& g1, int& pb) {
  using F = Fmt<L>;
  const int e0 = c * F::ce;
  g0 = e0 / group;
  const int bound = (g0 + 1) * group - e0;  // elements of the chunk in group g0
  pb = bound >= F::ce ? F::np : bound / 2;
  g1 = g0 + 1 < ngroups ? g0 + 1 : g0;
}

// Sum over the chunk of c[idx] * x' (fp16 x' pairs from xh2), split at pair pb.
template <int L>
__device__ __forceinline__ void chunk_dot(const uint32_t (&w)[Fmt<L>::cw], const uint32_t* lut, int lane31,
                                 const uint32_t* xp, int pb, float& a0, float& a1) {
  using F = Fmt<L>;
  int e[F::np];
  chunk_indices<L>(w, e);
#pragma unroll
  for (int q = 0; q < F::np; ++q) {
    const uint32_t cw = lut[e[q] * kLutCopies + lane31];
    if (q < pb) a0 = dot2_h(cw, xp[q], a0);
    else a1 = dot2_h(cw, xp[q], a1);
  }
}

template <int L, int CPL, int XDT>
__global__ __launch_bounds__(kBlock) void k_qmv(QmvParams p) {
  using F = Fmt<L>;
  extern __shared__ uint32_t smem_u[];
  const int xwords = p.Q * F::ce / 2;
  uint32_t* lut = smem_u;
  uint32_t* xh2 = lut + F::entries * kLutCopies;
  float* xf = reinterpret_cast<float*>(xh2 + xwords);
  float* red = xf + p.K;
  uint32_t* sb = reinterpret_cast<uint32_t*>(red + 32);

  build_lut<L>(lut, p.cb.h);
  if (!p.rotated)
    for (int w = threadIdx.x; w < (p.K + 31) / 32; w += blockDim.x) sb[w] = p.signs[w];
  __syncthreads();
  const float out_scale = prepare_input<XDT>(p.x, 0, p.K, p.m, p.P, p.rotated != 0, sb, xf, red,
                                             xh2, xwords, p.inv_sqrt_k);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lane31 = lane & 31;
  const int lpr = 1 << p.lpr_log;
  const int sub = lane >> p.lpr_log, c0 = lane & (lpr - 1);
  const int rpw = 64 >> p.lpr_log;
  const int64_t total_rows = static_cast<int64_t>(p.n_slots) * p.N;
  const int64_t row_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_block;
  int64_t row_end = row_begin + p.rows_per_block;
  if (row_end > total_rows) row_end = total_rows;
  const int ngroups = p.K / p.group;

  for (int64_t rb = row_begin + wave * rpw; rb < row_end; rb += 4 * rpw) {
    const int64_t row = rb + sub;
    const bool active = row < row_end;
    bool bad = false;
    int64_t wrow = 0;
    if (active) {
      const int slot = static_cast<int>(row / p.N);
      const int n = static_cast<int>(row - static_cast<int64_t>(slot) * p.N);
      const int e = p.ids ? p.ids[slot] : 0;
      bad = e < 0 || e >= p.E;
      wrow = bad ? 0 : static_cast<int64_t>(e) * p.N + n;
    }
    const bool live = active && !bad;
    const uint32_t* crow = p.codes + wrow * p.wpr;
    const uint16_t* srow = p.scales + wrow * ngroups;

    uint32_t w[CPL][F::cw];
    float s0[CPL], s1[CPL];
    int pb[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + j * lpr;
      const bool ok = live && c < p.Q;
      load_chunk<L>(crow, c, ok, w[j]);
      int g0, g1;
      chunk_groups<L>(ok ? c : 0, p.group, ngroups, g0, g1, pb[j]);
      s0[j] = ok ? half_bits_to_float(srow[g0]) : 0.f;
      s1[j] = ok ? half_bits_to_float(srow[g1]) : 0.f;
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + j * lpr;
      if (live && c < p.Q) {
        float a0 = 0.f, a1 = 0.f;
        chunk_dot<L>(w[j], lut, lane31, xh2 + c * (F::ce / 2), pb[j], a0, a1);
        acc += a0 * s0[j] + a1 * s1[j];
      }
    }
    for (int off = lpr >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (active && c0 == 0)
      store_any(p.y, p.ydt, row, bad ? __builtin_nanf("") : acc * out_scale);
  }
}

static int pow2_ceil_log(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int L>
static hipError_t launch_qmv_l(QmvParams& p, hipStream_t s) {
  using F = Fmt<L>;
  p.Q = (p.wpr + F::cw - 1) / F::cw;
  int lpr_log = pow2_ceil_log(p.Q);
  if (lpr_log > 6) lpr_log = 6;
  p.lpr_log = lpr_log;
  const int lpr = 1 << lpr_log;
  const int cpl_need = (p.Q + lpr - 1) / lpr;
  const int rpw = 64 / lpr;
  const int64_t total_rows = static_cast<int64_t>(p.n_slots) * p.N;
  // about 512 workgroups, at least one row step per wave
  int64_t rpb = (total_rows + 511) / 512;
  const int step = 4 * rpw;
  rpb = ((rpb + step - 1) / step) * step;
  p.rows_per_block = static_cast<int>(rpb);
  const int grid = static_cast<int>((total_rows + rpb - 1) / rpb);
  const size_t lds = (F::entries * kLutCopies + p.Q * F::ce / 2) * 4 + (p.K + 32) * 4 +
                     ((p.K + 31) / 32) * 4;
  void (*kern)(QmvParams) = nullptr;
#define TQ_PICK(C)                                                          \
  switch (p.xdt) {                                                          \
    case 0: kern = k_qmv<L, C, 0>; break;                                   \
    case 1: kern = k_qmv<L, C, 1>; break;                                   \
    default: kern = k_qmv<L, C, 2>; break;                                  \
  }
  if (cpl_need <= 1) { TQ_PICK(1) }
  else if (cpl_need <= 2) { TQ_PICK(2) }
  else if (cpl_need <= 4) { TQ_PICK(4) }
  else { TQ_PICK(8) }
#undef TQ_PICK
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_qmv(const WeightArgs& w, const int32_t* ids, int n, const void* x, int xdt,
                      bool x_rotated, void* y, int ydt, hipStream_t s) {
  if (n == 0 || w.N == 0) return hipSuccess;
  QmvParams p{};
  p.codes = w.codes; p.scales = w.scales; p.signs = w.signs; p.ids = ids;
  p.x = x; p.y = y;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group; p.m = w.m; p.P = w.P;
  p.n_slots = n; p.xdt = xdt; p.ydt = ydt; p.rotated = x_rotated ? 1 : 0;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  p.cb = *codebook_for(w.levels);
  switch (w.levels) {
    case 16: return launch_qmv_l<16>(p, s);
    case 8: return launch_qmv_l<8>(p, s);
    case 4: return launch_qmv_l<4>(p, s);
    default: return launch_qmv_l<3>(p, s);
  }
}

}  // namespace tq
