// Encode of weight rows whose length is a power of two, K = 2^p with 6 <= p <= 12:
// rotate -> group RMS -> fp16 scale -> snap -> pack, with the row held in registers.
//
// Steps (turboquant-mlx "How it works", "Quantizing a weight, with no data"; "The ternary
// tier (1.58 bits)"): v = H_K (s * w) (unnormalized: the 1/sqrt(K) of R cancels in v / r
// and is applied to the stored scale only), r = sqrt(mean_g v^2), scale = fp16(r / sqrt(K)),
// u = v / r (0 when r = 0), idx = #{k : u > t_k} decided in binary32, then bit or trit
// packing. Rotation and RMS are computed in double precision, as in k_encode.
//
// Work layout. Each wave works alone on batches of 4096 elements: 4096 / K whole rows,
// K / 64 lanes per row, 64 values per lane (128 registers of fp64). The Sylvester
// transform of a row is the product of one butterfly stage per bit of the element index,
// in any order, so it is done in two or three register phases with LDS exchanges between
// them, each phase running the stages of the index bits a lane holds in registers:
//   A (as loaded): lane t of a row holds the 8-element chunks t + c K/8 (c < 8), i.e.
//       element bits 0-2 and p-3..p-1 in registers: 6 stages;
//   B (only for p >= 10): lane (e, h) holds elements e + 8 j + 512 h (j < 64): element bits
//       3-8 in registers; the stages of bits 3..p-4 that phase A left;
//   C (final): lane t holds elements 64 t .. 64 t + 63; for p <= 9 the stages of bits
//       3..p-4 are run here; then group sums, scales, snap and packing are lane-local
//       (a 128-element group spans a lane pair).
// The exchanges go through a 32 KB LDS buffer per wave, addressed so that every exchange
// is free of bank conflicts (pair_slot), and need no workgroup barrier: only the wave's
// own lanes touch its buffer.
#include "device_common.hpp"
#include "internal.hpp"

namespace tq {
namespace {

constexpr int kP2Waves = 4;                        // waves per workgroup
constexpr int kP2Threads = 64 * kP2Waves;
constexpr int kP2Batch = 4096;                     // elements per wave batch
constexpr int kP2BufBytes = kP2Batch * 8;          // fp64 exchange buffer per wave

struct EncP2Params {
  const void* W;
  int64_t rows;
  uint64_t seed;
  uint32_t* codes;
  uint16_t* scales;
  double inv_sqrt_k;
  uint32_t tbits[8];    // the positive decision thresholds (binary32 bit patterns), ascending
  uint32_t tbig[128];   // the same for the 256-level codebook (127 used)
  int lg_k, wpr;
};

// 16-byte slot of element pair P (elements 2P, 2P + 1) in a wave's buffer. Banks repeat
// every 8 slots; the low three bits of P are XORed with a function f of y = P >> 3 so that
// each exchange's accesses fall on distinct banks:
//   A writes (16 B, 8 lanes): P = 4u + s, u consecutive   -> f(y) low bits follow u >> 1
//   C reads  (16 B, 8 lanes): P = 32 t + const           -> (y >> 2) & 7 follows t
//   B reads/writes (8 B, 16 lanes): P = 4 j + e/2 + 256 h -> (y >> 3) & 4 follows h
__device__ __forceinline__ int pair_slot(int P) {
  const int y = P >> 3;
  return P ^ ((y & 3) ^ ((y >> 2) & 7) ^ ((y >> 3) & 4));
}

// Orders a wave's LDS writes before its later LDS reads (other lanes' data): the LDS
// executes one wave's instructions in order, so only the compiler has to be held back.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int S>
__device__ __forceinline__ void bfly(double (&v)[64]) {
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    if (j & (1 << S)) continue;
    const double a = v[j], b = v[j | (1 << S)];
    v[j] = a + b;
    v[j | (1 << S)] = a - b;
  }
}

// WDT: 0 fp32, 1 bf16, 2 fp16 source rows.
template <int WDT>
struct P2Raw {
  static constexpr int kW = WDT == 0 ? 8 : 4;  // words per 8-element chunk
  uint32_t w[8][kW];
};

template <int WDT>
__device__ __forceinline__ void p2_load(P2Raw<WDT>& raw, const char* row_base, int t, int tr) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t off = static_cast<uint32_t>(8 * (t + tr * c)) * (WDT == 0 ? 4u : 2u);
    const u32x4_t a = ld_at<u32x4_t>(row_base, off);
    raw.w[c][0] = a.x; raw.w[c][1] = a.y; raw.w[c][2] = a.z; raw.w[c][3] = a.w;
    if constexpr (WDT == 0) {
      const u32x4_t b = ld_at<u32x4_t>(row_base, off + 16u);
      raw.w[c][4] = b.x; raw.w[c][5] = b.y; raw.w[c][6] = b.z; raw.w[c][7] = b.w;
    }
  }
}

// Element e of chunk c as fp64, times the sign s_e (bit e of `sbits`): the sign bit is
// flipped in the source format, which is exact.
template <int WDT>
__device__ __forceinline__ double p2_elem(const P2Raw<WDT>& raw, int c, int e, uint32_t sbits) {
  if constexpr (WDT == 0) {
    const uint32_t f = raw.w[c][e] ^ ((sbits << (31 - e)) & 0x80000000u);
    return static_cast<double>(__uint_as_float(f));
  } else {
    const uint32_t wd = raw.w[c][e >> 1];
    const uint32_t h = (e & 1) ? (wd >> 16) : (wd & 0xffffu);
    const uint32_t hs = h ^ (((sbits >> e) & 1u) << 15);
    if constexpr (WDT == 1) {
      return static_cast<double>(__uint_as_float(hs << 16));
    } else {
      return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hs))));
    }
  }
}

// The low-three-bit term of pair_slot as a function of P (linear over GF(2), so the slot
// of a sum of parts with disjoint bits is the XOR of the parts' terms).
__device__ __forceinline__ constexpr int slot_mix(int P) {
  return ((P >> 3) & 3) ^ ((P >> 5) & 7) ^ ((P >> 6) & 4);
}

template <int WDT, int LEVELS, int LG_G, bool BP>
__global__ __launch_bounds__(kP2Threads) void k_encode_p2(EncP2Params p) {
  extern __shared__ u32x4_t p2_smem[];
  __shared__ uint32_t sw[kP2Batch / 32];
  __shared__ uint32_t tk[LEVELS == 256 ? 128 : 1];  // 8-bit codebook: searched thresholds
  if constexpr (LEVELS == 256)
    if (threadIdx.x < 128) tk[threadIdx.x] = p.tbig[threadIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = p.lg_k, K = 1 << lg;
  const int lg_tr = lg - 6, tr = 1 << lg_tr;  // lanes per row
  const int rpb = 64 >> lg_tr;                // rows per batch
  const int rl = lane >> lg_tr, t = lane & (tr - 1);
  char* buf = reinterpret_cast<char*>(p2_smem) + wave * kP2BufBytes;

  // the rotation's sign bits, once per workgroup
  for (int w = threadIdx.x; w < (K >> 5); w += kP2Threads) {
    uint32_t b = 0;
    for (int j = 0; j < 32; ++j)
      if (splitmix64_at(p.seed, static_cast<uint64_t>(32 * w + j)) >> 63) b |= 1u << j;
    sw[w] = b;
  }
  __syncthreads();
  // the eight sign bytes of this lane's chunks t + c tr (the same in every batch)
  uint32_t sbyte[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int u = t + tr * c;
    sbyte[c] = (sw[u >> 2] >> (8 * (u & 3))) & 0xffu;
  }

  // LDS byte addresses, as precomputed bases plus compile-time offsets (see pair_slot):
  const int rowpair = rl * (K >> 1);  // first element pair of this lane's row
  // C reads: pair rowpair + 32 t + jj -> cbase[c] + 16 (jj & 24), c = (jj & 7) ^ mix(jj)
  int cbase[8];
  {
    const int A = rowpair + 32 * t, F = slot_mix(A);
#pragma unroll
    for (int c = 0; c < 8; ++c) cbase[c] = 16 * (A + (c ^ F));
  }
  // A writes: pair rowpair + 4 t + (4 tr c + s): the lane's part, then a uniform XOR
  const int abase = 16 * ((rowpair + 4 * t) & ~7);
  const int alow = (4 * (t & 1)) ^ slot_mix(rowpair + 4 * t);

  constexpr int G = 1 << LG_G;
  constexpr int GL = G < 64 ? G : 64;  // elements of one group inside a lane
  constexpr int NG = 64 / GL;          // groups (or half groups) per lane
  constexpr int NPOS = LEVELS == 3 ? 1 : LEVELS == 256 ? 8 : LEVELS / 2 - 1;
  constexpr int CPOS = LEVELS == 3 ? 1 : LEVELS / 2;      // idx of the smallest u > 0
  constexpr int CNEG = LEVELS == 3 ? 1 : LEVELS / 2 - 1;  // idx of u = 0
  const int64_t nbatch = (p.rows + rpb - 1) / rpb;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kP2Waves;
  int64_t b = static_cast<int64_t>(blockIdx.x) * kP2Waves + wave;
  if (b >= nbatch) return;

  const size_t esz = WDT == 0 ? 4 : 2;
  auto row_of = [&](int64_t bb) {
    const int64_t r = bb * rpb + rl;
    return r < p.rows ? r : p.rows - 1;
  };
  P2Raw<WDT> raw;
  p2_load<WDT>(raw, static_cast<const char*>(p.W) + row_of(b) * K * esz, t, tr);

  for (; b < nbatch; b += stride) {
    const int64_t row = b * rpb + rl;
    const bool live = row < p.rows;
    double v[64];
    // layout A: v[8 c + e] = s_i w_i for element i = 8 (t + c tr) + e
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * c + e] = p2_elem<WDT>(raw, c, e, sbyte[c]);
    if (b + stride < nbatch)
      p2_load<WDT>(raw, static_cast<const char*>(p.W) + row_of(b + stride) * K * esz, t, tr);

    // phase A: element bits 0-2 and p-3..p-1
    bfly<0>(v); bfly<1>(v); bfly<2>(v); bfly<3>(v); bfly<4>(v); bfly<5>(v);

    if (lg > 6) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int R = 4 * tr * c;  // uniform part of the pair index
        const int mix = slot_mix(R);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int addr = abase + 16 * R + 16 * (alow ^ s ^ mix);
          *reinterpret_cast<double2*>(buf + addr) = make_double2(v[8 * c + 2 * s], v[8 * c + 2 * s + 1]);
        }
      }
      wave_lds_sync();
      if constexpr (BP) {
        // phase B: lane (e, h) holds elements e + 8 j + 512 h; pair rowpair + 256 h +
        // (e >> 1) + 4 j -> bbase[c] + 128 (j >> 1), c = 4 (j & 1) ^ mix(4 j)
        const int e = t & 7, h = t >> 3;
        int bbase[8];
        {
          const int Ahi = rowpair + 256 * h;
          const int F = (e >> 1) | (4 * (h & 1));
#pragma unroll
          for (int c = 0; c < 8; ++c) bbase[c] = 16 * (Ahi + (F ^ c)) + 8 * (e & 1);
        }
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const int c = (4 * (j & 1)) ^ slot_mix(4 * j);
          v[j] = *reinterpret_cast<const double*>(buf + bbase[c] + 128 * (j >> 1));
        }
        bfly<0>(v); bfly<1>(v); bfly<2>(v); bfly<3>(v);
        if (lg >= 11) bfly<4>(v);
        if (lg >= 12) bfly<5>(v);
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const int c = (4 * (j & 1)) ^ slot_mix(4 * j);
          *reinterpret_cast<double*>(buf + bbase[c] + 128 * (j >> 1)) = v[j];
        }
        wave_lds_sync();
      }
      // layout C: lane t holds elements 64 t + j
#pragma unroll
      for (int jj = 0; jj < 32; ++jj) {
        const int c = (jj & 7) ^ slot_mix(jj);
        const double2 d = *reinterpret_cast<const double2*>(buf + cbase[c] + 16 * (jj & 24));
        v[2 * jj] = d.x;
        v[2 * jj + 1] = d.y;
      }
      if constexpr (!BP) {
        bfly<3>(v);
        if (lg >= 8) bfly<4>(v);
        if (lg >= 9) bfly<5>(v);
      }
    }

    // group RMS and fp16 scales
    double rinv[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      // eight independent partial sums (a single chain of GL dependent fp64 adds would
      // leave the wave waiting on each one)
      constexpr int NA = GL < 8 ? GL : 8;
      double part[NA];
#pragma unroll
      for (int a = 0; a < NA; ++a) part[a] = v[GL * k + a] * v[GL * k + a];
#pragma unroll
      for (int j = NA; j < GL; ++j) part[j % NA] = __builtin_fma(v[GL * k + j], v[GL * k + j], part[j % NA]);
#pragma unroll
      for (int w = NA / 2; w >= 1; w /= 2)
#pragma unroll
        for (int a = 0; a < w; ++a) part[a] += part[a + w];
      double s = part[0];
      if constexpr (G == 128) s += __shfl_xor(s, 1);
      const double rr = __builtin_sqrt(s / G);
      rinv[k] = rr > 0.0 ? 1.0 / rr : 0.0;
      const uint16_t sc = double_to_half_rne_sat(rr * p.inv_sqrt_k);
      if (live && (G < 128 || (t & 1) == 0)) {
        const int gi = G == 128 ? (t >> 1) : t * NG + k;
        p.scales[row * (K >> LG_G) + gi] = sc;
      }
    }

    // snap: idx = #{k : u > t_k} in binary32, from the positive thresholds alone (the
    // codebook is symmetric): u > 0 takes CPOS + #{t > 0 : u > t}; u <= 0 takes
    // CNEG - #{t > 0 : |u| >= t}; key = bits(|u|) + (u <= 0) turns both into one count.
    // The indices go straight into their packed words.
    constexpr int BITS = LEVELS == 4 ? 2 : LEVELS == 8 ? 3 : LEVELS == 16 ? 4 : 8;
    constexpr int NW = 2 * BITS;  // words of 64 codes (bytes for trits)
    uint32_t w[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) w[k] = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float u = static_cast<float>(v[j] * rinv[j / GL]);
      const uint32_t ub = __float_as_uint(u);
      const bool pos = static_cast<int32_t>(ub) > 0;  // u > 0 (never NaN here)
      const uint32_t key = (ub & 0x7fffffffu) + (pos ? 0u : 1u);
      uint32_t cnt = 0;
      if constexpr (LEVELS == 256) {
        // 127 positive thresholds: a branch-free binary search for #{q : key > tk[q]}
#pragma unroll
        for (int st = 64; st >= 1; st >>= 1) cnt += key > tk[cnt + st - 1] ? st : 0u;
      } else {
#pragma unroll
        for (int q = 0; q < NPOS; ++q) cnt += key > p.tbits[q] ? 1u : 0u;
      }
      const uint32_t idx = pos ? CPOS + cnt : CNEG - cnt;
      const int bp = BITS * j;
      w[bp >> 5] |= idx << (bp & 31);
      if ((bp & 31) + BITS > 32) w[(bp >> 5) + 1] |= idx >> (32 - (bp & 31));
    }

    if constexpr (LEVELS != 3) {
      if (live) {
        uint32_t* dst = p.codes + row * p.wpr + NW * t;
#pragma unroll
        for (int k = 0; k < NW; ++k) dst[k] = w[k];
      }
      wave_lds_sync();
    } else {
      // trit words (20 digits) do not line up with a lane's 64 elements: the digits go
      // through the buffer as bytes, then each lane packs words t, t + tr, ... of its row
      wave_lds_sync();
      u32x4_t* bw = reinterpret_cast<u32x4_t*>(buf + rl * K + 64 * t);
#pragma unroll
      for (int k = 0; k < 4; ++k) bw[k] = u32x4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
      wave_lds_sync();
      const uint32_t* rb = reinterpret_cast<const uint32_t*>(buf + rl * K);
      for (int wi = t; wi < p.wpr; wi += tr) {
        uint32_t d[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) d[k] = rb[5 * wi + k];
        uint32_t word = 0;
#pragma unroll
        for (int k = 19; k >= 0; --k) {
          const uint32_t digit = (d[k >> 2] >> (8 * (k & 3))) & 0xffu;
          word = word * 3u + (20 * wi + k < K ? digit : 0u);
        }
        if (live) p.codes[row * p.wpr + wi] = word;
      }
      wave_lds_sync();
    }
  }
}

template <int WDT, int LEVELS, bool BP>
hipError_t launch_p2_l(const EncP2Params& p, int group, int grid, hipStream_t s) {
  void (*kern)(EncP2Params) = nullptr;
  switch (group) {
    case 16: kern = k_encode_p2<WDT, LEVELS, 4, BP>; break;
    case 32: kern = k_encode_p2<WDT, LEVELS, 5, BP>; break;
    case 64: kern = k_encode_p2<WDT, LEVELS, 6, BP>; break;
    default: kern = k_encode_p2<WDT, LEVELS, 7, BP>; break;
  }
  const size_t lds = static_cast<size_t>(kP2Waves) * kP2BufBytes;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kP2Threads), lds, s, p);
  return hipGetLastError();
}

template <int WDT, bool BP>
hipError_t launch_p2_w(const EncP2Params& p, int levels, int group, int grid, hipStream_t s) {
  switch (levels) {
    case 3: return launch_p2_l<WDT, 3, BP>(p, group, grid, s);
    case 4: return launch_p2_l<WDT, 4, BP>(p, group, grid, s);
    case 8: return launch_p2_l<WDT, 8, BP>(p, group, grid, s);
    case 256: return launch_p2_l<WDT, 256, BP>(p, group, grid, s);
    default: return launch_p2_l<WDT, 16, BP>(p, group, grid, s);
  }
}

}  // namespace

bool encode_p2_supported(int K, int m) { return m == 1 && K >= 64 && K <= kP2Batch; }

hipError_t launch_encode_p2(const void* W, int wdt, int64_t rows, int K, int levels, int group,
                            uint64_t seed, uint32_t* codes, uint16_t* scales, hipStream_t s) {
  EncP2Params p{};
  p.W = W; p.rows = rows; p.seed = seed; p.codes = codes; p.scales = scales;
  int lg = 0;
  while ((1 << lg) < K) ++lg;
  p.lg_k = lg;
  p.inv_sqrt_k = 1.0 / __builtin_sqrt(static_cast<double>(K));
  p.wpr = levels == 3 ? (K + 19) / 20
                      : (K * (levels == 4 ? 2 : levels == 8 ? 3 : levels == 16 ? 4 : 8)) / 32;
  // positive thresholds of the symmetric codebook (the negative ones are their negations)
  const float* t = levels == 256 ? codebook256()->t : codebook_for(levels)->t;
  const int npos = levels == 3 ? 1 : levels / 2 - 1;
  uint32_t* dst = levels == 256 ? p.tbig : p.tbits;
  for (int q = 0; q < npos; ++q) {
    const float tq = t[levels - 1 - npos + q];
    const float tn = t[npos - 1 - q];
    if (!(tq > 0.f) || tn != -tq) return hipErrorInvalidValue;  // not symmetric: never
    dst[q] = __builtin_bit_cast(uint32_t, tq);
  }
  if (levels != 3 && t[levels / 2 - 1] != 0.f) return hipErrorInvalidValue;
  const int rpb = kP2Batch / K;
  const int64_t nbatch = (rows + rpb - 1) / rpb;
  const int64_t want = (nbatch + kP2Waves - 1) / kP2Waves;
  const int grid = static_cast<int>(want < 256 ? want : 256);  // one workgroup per CU
  const bool bp = lg >= 10;
  switch (wdt) {
    case 0: return bp ? launch_p2_w<0, true>(p, levels, group, grid, s) : launch_p2_w<0, false>(p, levels, group, grid, s);
    case 1: return bp ? launch_p2_w<1, true>(p, levels, group, grid, s) : launch_p2_w<1, false>(p, levels, group, grid, s);
    default: return bp ? launch_p2_w<2, true>(p, levels, group, grid, s) : launch_p2_w<2, false>(p, levels, group, grid, s);
  }
}

}  // namespace tq
