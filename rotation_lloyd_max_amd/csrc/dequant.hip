// dequant: the decoded weights of n experts in the rotated basis, for any shape of work the
// three fused kernels do not cover (turboquant-mlx "How it works", "Running a quantized
// layer", kernel table, fourth row: dequantize the experts, then a regular matrix
// multiply with the rotated input).
//
// out[k][i][j] = scale(ids[k], i, j / group) * c[idx(ids[k], i, j)]: the fp32 centroid times
// the fp16 scale in fp32, rounded once to the output type. One thread per chunk of a row
// (32 elements, or one 20-trit word): the chunk's words and scales are read with
// nontemporal loads (read once); a wave's outputs, one contiguous block of the row, leave
// through an LDS exchange so that each store instruction writes 1 KB of consecutive bytes
// (plain stores: with the nontemporal hint the kernel measured a third slower). The work
// is bound by the output bytes (2 or 4 per weight against 0.2..0.6 read).
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
  // the output of the chunk as 16-byte units (bit formats: 4 for 16-bit types, 8 for fp32)
  constexpr int BYTES = CE * (ODT == 0 ? 4 : 2);
  if constexpr (BYTES % 16 == 0) {
    constexpr int U = BYTES / 16;
    u32x4_t u[U];
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if constexpr (ODT == 0) {
        u[q] = u32x4_t{__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                       __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
      } else {
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = v[8 * q + 2 * r], b = v[8 * q + 2 * r + 1];
          const uint16_t ha = ODT == 1 ? float_to_bf16_rne(a) : float_to_half_rne(a);
          const uint16_t hb = ODT == 1 ? float_to_bf16_rne(b) : float_to_half_rne(b);
          h[r] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
        }
        u[q] = u32x4_t{h[0], h[1], h[2], h[3]};
      }
    }
    // When the wave's 64 chunks are consecutive chunks of one row, their outputs are one
    // contiguous block of 64 U units: exchange them through LDS so that every store
    // instruction of the wave writes 1 KB of consecutive bytes (measured a third faster
    // than each lane storing its own 64 or 128 bytes). Units are padded by one per 64 so
    // that both sides of the exchange are free of bank conflicts.
    const int lane = threadIdx.x & 63;
    const int64_t c0 = chunk - lane;
    // (a block ending with a partial last trit word of its row takes the per-lane path)
    const bool block = c0 + 63 < p.chunks && c0 / p.Q == (c0 + 63) / p.Q &&
                       (L != 3 || (c0 + 63) % p.Q != p.Q - 1 || p.K % CE == 0);
    if (block) {
      __shared__ u32x4_t xch[kDeqThreads / 64][64 * U + U];
      u32x4_t* wx = xch[threadIdx.x >> 6];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int pos = U * lane + q;
        wx[pos + (pos >> 6)] = u[q];
      }
      __builtin_amdgcn_wave_barrier();
      const int64_t ob = (static_cast<int64_t>(k) * p.N + c0 / p.Q) * p.K + (c0 % p.Q) * CE;
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.out) + ob * (ODT == 0 ? 4 : 2));
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int pos = 64 * q + lane;
        dst[pos] = wx[pos + (pos >> 6)];
      }
    } else {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.out) + o * (ODT == 0 ? 4 : 2));
      constexpr int EPU = ODT == 0 ? 4 : 8;  // elements per 16-byte unit
#pragma unroll
      for (int q = 0; q < U; ++q)
        if (EPU * q < cnt) dst[q] = u[q];
    }
  } else {
    // trit chunks of 16-bit outputs: 40 bytes, 8-byte aligned
    u32x2_t* dst = reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + o);
#pragma unroll
    for (int q = 0; q < CE / 4; ++q) {
      if (4 * q < cnt) {
        uint32_t h2[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float a = v[4 * q + 2 * r], b = v[4 * q + 2 * r + 1];
          const uint16_t ha = ODT == 1 ? float_to_bf16_rne(a) : float_to_half_rne(a);
          const uint16_t hb = ODT == 1 ? float_to_bf16_rne(b) : float_to_half_rne(b);
          h2[r] = static_cast<uint32_t>(ha) | (static_cast<uint32_t>(hb) << 16);
        }
        dst[q] = u32x2_t{h2[0], h2[1]};
      }
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
