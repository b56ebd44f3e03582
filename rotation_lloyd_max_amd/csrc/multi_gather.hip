// multi_gather_qmv: y[p] = W_{ids[p]} R x[p] for P (input, expert) pairs.
//
// turboquant-mlx "How it works", "Running a quantized layer", kernel table, second row:
// prefill with a different input per expert. Pairs are first bucketed by expert on the
// device (counting sort into the workspace); then each workgroup owns one (expert, row
// block), rotates the inputs routed to that expert in batches of up to kBatch, and streams
// the expert's rows once per batch, decoding each chunk once and multiplying it against
// every input of the batch.
#include "decode_common.hpp"
#include "internal.hpp"

namespace tq {

constexpr int kBatch = 8;
constexpr int kBucketThreads = 1024;
constexpr int kMaxExperts = 8192;

// Workspace layout: offsets [E+1] int32 | order [P] int32 (16-byte aligned sections).
static size_t align16(size_t v) { return (v + 15) & ~static_cast<size_t>(15); }

size_t multi_gather_workspace(const WeightArgs& w, int64_t P) {
  return align16(static_cast<size_t>(w.E + 1) * 4) + align16(static_cast<size_t>(P) * 4);
}

__global__ __launch_bounds__(kBucketThreads) void k_bucket(const int32_t* ids, int64_t P, int E,
                                                           int32_t* offsets, int32_t* order,
                                                           void* y, int ydt, int N) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t wsum[kBucketThreads / 64];
  for (int e = threadIdx.x; e < E; e += kBucketThreads) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < P; p += kBucketThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
    } else {
      for (int n = 0; n < N; ++n) store_any(y, ydt, p * N + n, __builtin_nanf(""));
    }
  }
  __syncthreads();
  // exclusive scan of cnt[0..E) in chunks of kBucketThreads, carried by thread 0's running sum
  int carry = 0;
  for (int base = 0; base < E; base += kBucketThreads) {
    const int e = base + threadIdx.x;
    int v = e < E ? cnt[e] : 0;
    // inclusive wave scan
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = carry;
    for (int k = 0; k < wave; ++k) before += wsum[k];
    const int incl = before + v;
    int excl = incl - (e < E ? cnt[e] : 0);
    __syncthreads();
    if (e < E) {
      offsets[e] = excl;
      cnt[e] = excl;  // becomes the scatter cursor
    }
    int total = carry;
    for (int k = 0; k < static_cast<int>(kBucketThreads >> 6); ++k) total += wsum[k];
    carry = total;
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < P; p += kBucketThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&cnt[e], 1);
      order[pos] = static_cast<int32_t>(p);
    }
  }
}

struct MultiParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  const int32_t* offsets;
  const int32_t* order;
  const void* x;
  void* y;
  int K, N, E, wpr, group, m, P;
  int xdt, ydt, rotated;
  int Q, lpr_log, rows_per_block;
  float inv_sqrt_k;
  CodebookArgs cb;
};

template <int XDT>
__device__ __forceinline__ float prepare_input_m(const void* x, int64_t xoff, int K, int m, int P,
                                        bool rotated, const uint32_t* sb, float* xf, float* red,
                                        uint32_t* xh2, int xwords, float inv_sqrt_k) {
  for (int i = threadIdx.x; i < K; i += kBlock) {
    float v = load_elem<XDT>(x, xoff + i);
    if (!rotated && ((sb[i >> 5] >> (i & 31)) & 1u)) v = -v;
    xf[i] = v;
  }
  __syncthreads();
  if (!rotated) hadamard_lds<float>(xf, 1, m, P);
  float mx = 0.f;
  for (int i = threadIdx.x; i < K; i += kBlock) mx = fmaxf(mx, fabsf(xf[i]));
  mx = block_max(mx, red);
  int ex = 0;
  if (mx > 0.f && mx <= 3.0e38f) {
    ex = 14 - ilogbf(mx);
    ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
  }
  const float sc = ldexpf(1.f, ex);
  for (int q = threadIdx.x; q < xwords; q += kBlock) {
    const int i0 = 2 * q, i1 = 2 * q + 1;
    const float a = i0 < K ? xf[i0] * sc : 0.f;
    const float b = i1 < K ? xf[i1] * sc : 0.f;
    xh2[q] = static_cast<uint32_t>(float_to_half_rne(a)) |
             (static_cast<uint32_t>(float_to_half_rne(b)) << 16);
  }
  __syncthreads();
  return ldexpf(1.f, -ex) * (rotated ? 1.f : inv_sqrt_k);
}

template <int L>
__device__ __forceinline__ void load_chunk_m(const uint32_t* crow, int c, bool ok, uint32_t (&w)[Fmt<L>::cw]) {
  using F = Fmt<L>;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < F::cw; ++i) w[i] = 0;
    return;
  }
  const uint32_t* p = crow + c * F::cw;
#pragma unroll
  for (int i = 0; i < F::cw; ++i) w[i] = p[i];
}

template <int L, int CPL, int XDT>
__global__ __launch_bounds__(kBlock) void k_multi(MultiParams p) {
  using F = Fmt<L>;
  const int e = blockIdx.y;
  const int off = p.offsets[e];
  const int cnt = p.offsets[e + 1] - off;
  if (cnt <= 0) return;
  const int64_t row_begin = static_cast<int64_t>(blockIdx.x) * p.rows_per_block;
  if (row_begin >= p.N) return;
  int64_t row_end = row_begin + p.rows_per_block;
  if (row_end > p.N) row_end = p.N;

  extern __shared__ uint32_t smem_u[];
  const int xwords = p.Q * F::ce / 2;
  uint32_t* lut = smem_u;
  uint32_t* xh2 = lut + F::entries * kLutCopies;           // kBatch * xwords
  float* xf = reinterpret_cast<float*>(xh2 + kBatch * xwords);  // K
  float* red = xf + p.K;                                   // 32
  float* oscale = red + 32;                                // kBatch
  int* pidx = reinterpret_cast<int*>(oscale + kBatch);     // kBatch
  uint32_t* sb = reinterpret_cast<uint32_t*>(pidx + kBatch);

  build_lut<L>(lut, p.cb.h);
  if (!p.rotated)
    for (int w = threadIdx.x; w < (p.K + 31) / 32; w += kBlock) sb[w] = p.signs[w];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lane31 = lane & 31;
  const int lpr = 1 << p.lpr_log;
  const int sub = lane >> p.lpr_log, c0 = lane & (lpr - 1);
  const int rpw = 64 >> p.lpr_log;
  const int ngroups = p.K / p.group;

  for (int b0 = 0; b0 < cnt; b0 += kBatch) {
    const int nb = cnt - b0 < kBatch ? cnt - b0 : kBatch;
    for (int j = 0; j < nb; ++j) {
      const int pp = p.order[off + b0 + j];
      const float os = prepare_input_m<XDT>(p.x, static_cast<int64_t>(pp) * p.K, p.K, p.m, p.P,
                                            p.rotated != 0, sb, xf, red, xh2 + j * xwords, xwords,
                                            p.inv_sqrt_k);
      if (threadIdx.x == 0) { oscale[j] = os; pidx[j] = pp; }
    }
    __syncthreads();

    for (int64_t rb = row_begin + wave * rpw; rb < row_end; rb += 4 * rpw) {
      const int64_t n = rb + sub;
      const bool active = n < row_end;
      const int64_t wrow = active ? static_cast<int64_t>(e) * p.N + n : 0;
      const uint32_t* crow = p.codes + wrow * p.wpr;
      const uint16_t* srow = p.scales + wrow * ngroups;
      float acc[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) acc[j] = 0.f;
#pragma unroll
      for (int jc = 0; jc < CPL; ++jc) {
        const int c = c0 + jc * lpr;
        const bool ok = active && c < p.Q;
        if (!ok) continue;
        uint32_t w[F::cw];
        load_chunk_m<L>(crow, c, true, w);
        int g0, g1, pb;
        {
          const int e0 = c * F::ce;
          g0 = e0 / p.group;
          const int bound = (g0 + 1) * p.group - e0;
          pb = bound >= F::ce ? F::np : bound / 2;
          g1 = g0 + 1 < ngroups ? g0 + 1 : g0;
        }
        const float s0 = half_bits_to_float(srow[g0]);
        const float s1 = half_bits_to_float(srow[g1]);
        int idx[F::np];
        chunk_indices<L>(w, idx);
        uint32_t cwv[F::np];
#pragma unroll
        for (int q = 0; q < F::np; ++q) cwv[q] = lut[idx[q] * kLutCopies + lane31];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (j < nb) {
            const uint32_t* xp = xh2 + j * xwords + c * (F::ce / 2);
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int q = 0; q < F::np; ++q) {
              if (q < pb) a0 = dot2_h(cwv[q], xp[q], a0);
              else a1 = dot2_h(cwv[q], xp[q], a1);
            }
            acc[j] += a0 * s0 + a1 * s1;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float a = acc[j];
        for (int o = lpr >> 1; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
        if (active && c0 == 0 && j < nb)
          store_any(p.y, p.ydt, static_cast<int64_t>(pidx[j]) * p.N + n, a * oscale[j]);
      }
    }
    __syncthreads();
  }
}

static int pow2_ceil_log_m(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int L>
static hipError_t launch_multi_l(MultiParams& p, hipStream_t s) {
  using F = Fmt<L>;
  p.Q = (p.wpr + F::cw - 1) / F::cw;
  int lpr_log = pow2_ceil_log_m(p.Q);
  if (lpr_log > 6) lpr_log = 6;
  p.lpr_log = lpr_log;
  const int lpr = 1 << lpr_log;
  const int cpl_need = (p.Q + lpr - 1) / lpr;
  const int rpw = 64 / lpr;
  // row blocks per expert: aim for ~8 blocks per expert, at least one row step per wave
  int rpb = (p.N + 7) / 8;
  const int step = 4 * rpw;
  rpb = ((rpb + step - 1) / step) * step;
  p.rows_per_block = rpb;
  const int gx = (p.N + rpb - 1) / rpb;
  const size_t lds = (F::entries * kLutCopies + kBatch * (p.Q * F::ce / 2)) * 4 +
                     (p.K + 32 + 2 * kBatch) * 4 + ((p.K + 31) / 32) * 4;
  void (*kern)(MultiParams) = nullptr;
#define TQ_PICK(C)                                                  \
  switch (p.xdt) {                                                  \
    case 0: kern = k_multi<L, C, 0>; break;                         \
    case 1: kern = k_multi<L, C, 1>; break;                         \
    default: kern = k_multi<L, C, 2>; break;                        \
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
  hipLaunchKernelGGL(kern, dim3(gx, p.E), dim3(kBlock), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_multi_gather(const WeightArgs& w, const int32_t* ids, int64_t P, const void* x,
                               int xdt, bool x_rotated, void* y, int ydt, void* ws,
                               hipStream_t s) {
  if (P == 0 || w.N == 0) return hipSuccess;
  int32_t* offsets = static_cast<int32_t*>(ws);
  int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                              align16(static_cast<size_t>(w.E + 1) * 4));
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(kBucketThreads), 0, s, ids, P, w.E, offsets, order, y,
                     ydt, w.N);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  MultiParams p{};
  p.codes = w.codes; p.scales = w.scales; p.signs = w.signs; p.offsets = offsets; p.order = order;
  p.x = x; p.y = y;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group; p.m = w.m; p.P = w.P;
  p.xdt = xdt; p.ydt = ydt; p.rotated = x_rotated ? 1 : 0;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  p.cb = *codebook_for(w.levels);
  switch (w.levels) {
    case 16: return launch_multi_l<16>(p, s);
    case 8: return launch_multi_l<8>(p, s);
    case 4: return launch_multi_l<4>(p, s);
    default: return launch_multi_l<3>(p, s);
  }
}

}  // namespace tq
