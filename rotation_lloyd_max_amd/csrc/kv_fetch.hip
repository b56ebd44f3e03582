// The fetch half of a compressed KV cache: every stored row dequantized and rotated back,
//     out[r] = R^T w'_r,   w'_r[j] = c[idx_rj] * scale_{r, j / group},
//     R^T = diag(s) H_d / sqrt(d)   (H_d is a symmetric Sylvester matrix for d = 2^p).
// (turboquant-mlx "How it works", "The KV cache": the weights' rotation and codebook compress
// the cache, 8-bit keys and 3-bit values; "your SSD is a GPU", the KV-cache section: rotate,
// quantize, store, then dequantize and de-rotate on the way out.)
//
// Work layout: a lane holds 32 consecutive elements of one row, d / 32 lanes per row,
// 2048 / d rows per wave. Its packed codes are b whole words (b bits per code) and its signs
// one sign word. The Sylvester transform runs its five low stages in registers and the
// rest across the row's lanes with lane exchanges (no LDS buffer, no barrier). fp32
// throughout; the output is rounded once.
#include "device_common.hpp"
#include "internal.hpp"

namespace tq {
namespace {

constexpr int kKvThreads = 256;
constexpr int kKvEl = 32;  // elements per lane

struct KvParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  void* out;
  int64_t rows;
  int K, wpr, ngk, lg_group, lg_tr;
  float inv_sqrt_k;
  float lut[256];  // centroids, binary32 (the first n_levels used)
};

template <int S>
__device__ __forceinline__ void kv_bfly(float (&v)[kKvEl]) {
#pragma unroll
  for (int j = 0; j < kKvEl; ++j) {
    if (j & (1 << S)) continue;
    const float a = v[j], b = v[j | (1 << S)];
    v[j] = a + b;
    v[j | (1 << S)] = a - b;
  }
}

// One butterfly stage between lanes `lane` and `lane ^ M`: the lower lane keeps the sum, the
// upper one the difference (partner - own). M = 1 and 2 move data with DPP quad
// permutations (no LDS instruction), larger strides with a lane shuffle.
template <int M>
__device__ __forceinline__ float kv_partner(float x) {
  if constexpr (M == 1 || M == 2) {
    constexpr int sel = M == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), sel, 0xf, 0xf, true));
  } else {
    return __shfl_xor(x, M);
  }
}

template <int M>
__device__ __forceinline__ void kv_lane_stage(float (&v)[kKvEl]) {
  // the upper lane's partner - own as partner + (-own), the sign flipped in the bits (exact)
  const uint32_t flip = (threadIdx.x & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < kKvEl; ++j) {
    const float o = kv_partner<M>(v[j]);
    v[j] = o + __uint_as_float(__float_as_uint(v[j]) ^ flip);
  }
}

// A lane's packed codes and scales of one batch.
template <int NW>
struct KvIn {
  uint32_t w[NW];
  uint16_t s0, s1;
};

// G16: groups of 16 (two scales per lane); otherwise one scale per lane.
//
// Each wave works through batches of 2048 / d rows, the next batch's codes and scales
// loaded while the current one is decoded. A full batch's outputs are consecutive in memory
// (the wave's rows are consecutive, a lane's 32 elements contiguous within its row), so
// they go through a per-wave LDS buffer and leave in store instructions that each write
// 1 KB of consecutive bytes; a partial last batch stores lane by lane.
template <int LEVELS, bool G16, int ODT>
__global__ __launch_bounds__(kKvThreads) void k_kv_fetch(KvParams p) {
  constexpr int B = LEVELS == 4 ? 2 : LEVELS == 8 ? 3 : LEVELS == 16 ? 4 : 8;
  constexpr int NW = kKvEl * B / 32;          // code words per lane
  constexpr int SU = kKvEl * (ODT == 0 ? 4 : 2) / 16;  // 16-byte output units per lane
  __shared__ float lut[LEVELS];
  __shared__ u32x4_t stage[kKvThreads / 64][64 * SU];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tr = 1 << p.lg_tr;    // lanes per row
  const int rpw = 64 >> p.lg_tr;  // rows per wave batch
  const int rl = lane >> p.lg_tr, t = lane & (tr - 1);
  const int col0 = t * kKvEl;     // first element of this lane's chunk
  for (int k = threadIdx.x; k < LEVELS; k += kKvThreads) lut[k] = p.lut[k];
  __syncthreads();
  const uint32_t sgn = p.signs[t];  // sign bits of elements col0 .. col0 + 31
  // 16-bit outputs: the signs of elements 2k, 2k + 1 as the sign bits of packed pair k
  // (negating before or after the rounding to nearest is the same)
  uint32_t pmask[ODT == 0 ? 1 : kKvEl / 2];
  if constexpr (ODT != 0) {
#pragma unroll
    for (int k = 0; k < kKvEl / 2; ++k)
      pmask[k] = (((sgn >> (2 * k)) & 1u) << 15) | (((sgn >> (2 * k + 1)) & 1u) << 31);
  }
  const int gi0 = col0 >> p.lg_group;
  u32x4_t* st = stage[wave];

  const int64_t nb = (p.rows + rpw - 1) / rpw;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (kKvThreads / 64);
  int64_t b = static_cast<int64_t>(blockIdx.x) * (kKvThreads / 64) + wave;
  auto fetch = [&](int64_t bb, KvIn<NW>& in) {
    int64_t row = bb * rpw + rl;
    row = row < p.rows ? row : p.rows - 1;  // lanes past the rows load a valid row
    const uint32_t* src = p.codes + row * p.wpr + t * NW;
#pragma unroll
    for (int k = 0; k < NW; ++k) in.w[k] = src[k];
    const uint16_t* srow = p.scales + row * p.ngk + gi0;
    in.s0 = srow[0];
    in.s1 = G16 ? srow[1] : in.s0;
  };
  KvIn<NW> nxt;
  if (b < nb) fetch(b, nxt);
  for (; b < nb; b += stride) {
    const KvIn<NW> in = nxt;
    if (b + stride < nb) fetch(b + stride, nxt);
    const int64_t row = b * rpw + rl;
    // the 1/sqrt(d) of R^T is folded into the group scales
    const float s0 = half_bits_to_float(in.s0) * p.inv_sqrt_k;
    const float s1 = G16 ? half_bits_to_float(in.s1) * p.inv_sqrt_k : s0;
    float v[kKvEl];
#pragma unroll
    for (int j = 0; j < kKvEl; ++j) {
      const int bp = B * j;
      uint32_t idx = in.w[bp >> 5] >> (bp & 31);
      if ((bp & 31) + B > 32) idx |= in.w[(bp >> 5) + 1] << (32 - (bp & 31));
      idx &= (1u << B) - 1u;
      v[j] = lut[idx] * (G16 && j >= 16 ? s1 : s0);
    }
    // H_d: the five low index bits in registers, the rest across the row's lanes
    kv_bfly<0>(v); kv_bfly<1>(v); kv_bfly<2>(v); kv_bfly<3>(v); kv_bfly<4>(v);
    if (tr > 1) kv_lane_stage<1>(v);
    if (tr > 2) kv_lane_stage<2>(v);
    if (tr > 4) kv_lane_stage<4>(v);
    if (tr > 8) kv_lane_stage<8>(v);
    if (tr > 16) kv_lane_stage<16>(v);
    if (tr > 32) kv_lane_stage<32>(v);
    // R^T = diag(s) H / sqrt(d): the signs (1/sqrt(d) is in the scales)
    u32x4_t u[SU];
    if constexpr (ODT == 0) {
#pragma unroll
      for (int j = 0; j < kKvEl; ++j) v[j] = ((sgn >> j) & 1u) ? -v[j] : v[j];
#pragma unroll
      for (int k = 0; k < SU; ++k)
        u[k] = u32x4_t{__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                       __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3])};
    } else {
      uint32_t hw[kKvEl / 2];
#pragma unroll
      for (int k = 0; k < kKvEl / 2; ++k) {
        // round to nearest even (bf16: the hardware conversion, v_cvt_pk_bf16_f32)
        uint16_t a, c;
        if constexpr (ODT == 1) {
          a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k]));
          c = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[2 * k + 1]));
        } else {
          a = float_to_half_rne(v[2 * k]);
          c = float_to_half_rne(v[2 * k + 1]);
        }
        hw[k] = (static_cast<uint32_t>(a) | (static_cast<uint32_t>(c) << 16)) ^ pmask[k];
      }
#pragma unroll
      for (int k = 0; k < SU; ++k) u[k] = u32x4_t{hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]};
    }
    const int esz = ODT == 0 ? 4 : 2;
    if ((b + 1) * rpw <= p.rows) {  // uniform: a full batch, one contiguous block
      // unit q (16 bytes of the block) of lane q / SU; slot q ^ ((q >> 4) & 3) spreads the
      // lanes' writes over the banks
#pragma unroll
      for (int k = 0; k < SU; ++k) {
        const int q = SU * lane + k;
        st[q ^ ((q >> 4) & 3)] = u[k];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      char* dst = static_cast<char*>(p.out) + (b * rpw) * static_cast<int64_t>(p.K) * esz;
#pragma unroll
      for (int k = 0; k < SU; ++k) {
        const int q = 64 * k + lane;
        reinterpret_cast<u32x4_t*>(dst)[q] = st[q ^ ((q >> 4) & 3)];
      }
      // the next batch's LDS writes come after these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else if (row < p.rows) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.out) +
                                                (row * p.K + col0) * static_cast<int64_t>(esz));
#pragma unroll
      for (int k = 0; k < SU; ++k) dst[k] = u[k];
    }
  }
}

template <int LEVELS, bool G16>
hipError_t launch_kv_l(const KvParams& p, int odt, int grid, hipStream_t s) {
  switch (odt) {
    case 0: hipLaunchKernelGGL((k_kv_fetch<LEVELS, G16, 0>), dim3(grid), dim3(kKvThreads), 0, s, p); break;
    case 1: hipLaunchKernelGGL((k_kv_fetch<LEVELS, G16, 1>), dim3(grid), dim3(kKvThreads), 0, s, p); break;
    default: hipLaunchKernelGGL((k_kv_fetch<LEVELS, G16, 2>), dim3(grid), dim3(kKvThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

template <int LEVELS>
hipError_t launch_kv_g(const KvParams& p, bool g16, int odt, int grid, hipStream_t s) {
  return g16 ? launch_kv_l<LEVELS, true>(p, odt, grid, s) : launch_kv_l<LEVELS, false>(p, odt, grid, s);
}

}  // namespace

bool kv_fetch_supported(int K, int levels) {
  return levels != 3 && K >= 64 && K <= 2048 && (K & (K - 1)) == 0;
}

hipError_t launch_kv_fetch(const WeightArgs& w, int64_t rows, void* out, int odt, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  KvParams p{};
  p.codes = w.codes; p.scales = w.scales; p.signs = w.signs; p.out = out; p.rows = rows;
  p.K = w.K; p.wpr = w.wpr; p.ngk = w.K / w.group;
  p.lg_group = __builtin_ctz(w.group);
  int lg = 0;
  while ((1 << lg) < w.K) ++lg;
  p.lg_tr = lg - 5;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  const float* c = w.levels == 256 ? codebook256()->c : codebook_for(w.levels)->c;
  for (int k = 0; k < w.levels; ++k) p.lut[k] = c[k];
  const int64_t rpw = 64 >> p.lg_tr;
  const int64_t nb = (rows + rpw - 1) / rpw;
  const int64_t want = (nb + 3) / 4;
  const int grid = static_cast<int>(want < 2048 ? want : 2048);
  const bool g16 = w.group == 16;
  switch (w.levels) {
    case 4: return launch_kv_g<4>(p, g16, odt, grid, s);
    case 8: return launch_kv_g<8>(p, g16, odt, grid, s);
    case 16: return launch_kv_g<16>(p, g16, odt, grid, s);
    default: return launch_kv_g<256>(p, g16, odt, grid, s);
  }
}

}  // namespace tq
