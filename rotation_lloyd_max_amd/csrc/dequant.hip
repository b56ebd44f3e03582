// dequant: the decoded weights of n experts in the rotated basis, for any shape of work the
// three fused kernels do not cover (turboquant-mlx "How it works", "Running a quantized
// layer", kernel table, fourth row: dequantize the experts, then a regular matrix
// multiply with the rotated input).
//
// out[k][i][j] = scale(ids[k], i, j / group) * c[idx(ids[k], i, j)]: the fp32 centroid times
// the fp16 scale in fp32, rounded once to the output type. One thread per chunk of a row
// (32 elements, or one 20-trit word): the chunk's words and scales are read with
// nontemporal loads (read once) and its outputs written with 8- or 16-byte stores, so a
// wave writes whole contiguous runs of the output row. The work is bound by the output
// bytes (2 or 4 per weight against 0.2..0.6 read).
#include "decode_common.hpp"
#include "internal.hpp"

namespace tq {

constexpr int kDeqThreads = 256;

struct DequantParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const int32_t* ids;  // or nullptr: block k is expert k
  void* out;
  int64_t chunks;      // chunks per expert (N * Q)
  int K, N, E, wpr, group, ngk, Q;
  CodebookArgs cb;
};

// Plain stores: with the nontemporal hint the kernel measured a third slower.
template <typename T>
__device__ __forceinline__ void store_vec(T* p, T v) {
  *p = v;
}

template <int L>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[Fmt<L>::cw], int j) {
  if constexpr (L == 3) {
    return 0;  // trits are split by the caller
  } else {
    constexpr int b = L == 16 ? 4 : L == 8 ? 3 : 2;
    const int bit = b * j, lo = bit >> 5, sh = bit & 31;
    uint32_t v = w[lo] >> sh;
    if (sh + b > 32) v |= w[lo + 1] << (32 - sh);
    return v & ((1u << b) - 1u);
  }
}

template <int L, int ODT>
__global__ __launch_bounds__(kDeqThreads) void k_dequant(DequantParams p) {
  using F = Fmt<L>;
  constexpr int CE = F::ce;
  __shared__ float cbs[16];
  if (threadIdx.x < 16) cbs[threadIdx.x] = p.cb.c[threadIdx.x];
  __syncthreads();
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * kDeqThreads + threadIdx.x;
  if (chunk >= p.chunks) return;
  const int k = blockIdx.y;
  const int e = p.ids ? p.ids[k] : k;
  const bool bad = e < 0 || e >= p.E;
  const int row = static_cast<int>(chunk / p.Q), c = static_cast<int>(chunk - static_cast<int64_t>(row) * p.Q);
  const int64_t erow = static_cast<int64_t>(bad ? 0 : e) * p.N + row;
  uint32_t w[F::cw];
  load_chunk_words<L>(p.codes + erow * p.wpr, 0u, c, w);
  // the (at most two) groups the chunk touches
  const int e0 = c * CE;
  const int g0 = e0 / p.group;
  const int g1 = g0 + 1 < p.ngk ? g0 + 1 : g0;
  const uint16_t* srow = p.scales + erow * p.ngk;
  const float s0 = static_cast<float>(ld_stream<_Float16>(srow, 2u * g0));
  const float s1 = static_cast<float>(ld_stream<_Float16>(srow, 2u * g1));
  const int split = (g0 + 1) * p.group - e0;  // first element of the second group
  float v[CE];
  if constexpr (L == 3) {
    uint32_t t = w[0];
#pragma unroll
    for (int j = 0; j < CE; ++j) {
      const uint32_t q = t / 3u;
      v[j] = cbs[t - 3u * q] * (j < split ? s0 : s1);
      t = q;
    }
  } else {
#pragma unroll
    for (int j = 0; j < CE; ++j) v[j] = cbs[code_at<L>(w, j)] * (j < split ? s0 : s1);
  }
  if (bad) {
#pragma unroll
    for (int j = 0; j < CE; ++j) v[j] = __builtin_nanf("");
  }
  const int64_t o = (static_cast<int64_t>(k) * p.N + row) * p.K + e0;  // first output element
  // elements of the chunk inside the row: all of them, except in a row's last trit word
  // (K is a multiple of 32, so the count is a multiple of 4)
  const int cnt = p.K - e0 < CE ? p.K - e0 : CE;
  if constexpr (ODT == 0) {
    // fp32: 16-byte stores at 16-byte aligned offsets (K and e0 are multiples of 4)
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<float*>(p.out) + o);
#pragma unroll
    for (int q = 0; q < CE / 4; ++q)
      if (4 * q < cnt)
        store_vec(dst + q, u32x4_t{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                   __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])});
  } else {
    uint32_t h[CE / 2];
#pragma unroll
    for (int q = 0; q < CE / 2; ++q) {
      const uint16_t a = ODT == 1 ? float_to_bf16_rne(v[2 * q]) : float_to_half_rne(v[2 * q]);
      const uint16_t b = ODT == 1 ? float_to_bf16_rne(v[2 * q + 1]) : float_to_half_rne(v[2 * q + 1]);
      h[q] = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
    }
    uint16_t* base = static_cast<uint16_t*>(p.out) + o;
    if constexpr (CE % 8 == 0) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(base);  // 64 bytes, 16-byte aligned
#pragma unroll
      for (int q = 0; q < CE / 8; ++q)
        store_vec(dst + q, u32x4_t{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]});
    } else {
      u32x2_t* dst = reinterpret_cast<u32x2_t*>(base);  // up to 40 bytes, 8-byte aligned
#pragma unroll
      for (int q = 0; q < CE / 4; ++q)
        if (4 * q < cnt) store_vec(dst + q, u32x2_t{h[2 * q], h[2 * q + 1]});
    }
  }
}

template <int L>
static hipError_t launch_dequant_l(DequantParams& p, int n, int odt, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.chunks + kDeqThreads - 1) / kDeqThreads), n);
  if (odt == 0) hipLaunchKernelGGL((k_dequant<L, 0>), grid, dim3(kDeqThreads), 0, s, p);
  else if (odt == 1) hipLaunchKernelGGL((k_dequant<L, 1>), grid, dim3(kDeqThreads), 0, s, p);
  else hipLaunchKernelGGL((k_dequant<L, 2>), grid, dim3(kDeqThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dequant(const WeightArgs& w, const int32_t* ids, int n, void* out, int odt,
                          hipStream_t s) {
  if (n == 0 || w.N == 0) return hipSuccess;
  DequantParams p{};
  p.codes = w.codes; p.scales = w.scales; p.ids = ids; p.out = out;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group;
  p.ngk = w.K / w.group;
  p.Q = w.levels == 3 ? w.wpr : w.K / 32;
  p.chunks = static_cast<int64_t>(w.N) * p.Q;
  p.cb = *codebook_for(w.levels);
  switch (w.levels) {
    case 16: return launch_dequant_l<16>(p, n, odt, s);
    case 8: return launch_dequant_l<8>(p, n, odt, s);
    case 4: return launch_dequant_l<4>(p, n, odt, s);
    default: return launch_dequant_l<3>(p, n, odt, s);
  }
}

}  // namespace tq
