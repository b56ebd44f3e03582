// Encode of weight rows whose length is a power of two, K = 2^p with 6 <= p <= 12:
// rotate -> group RMS -> fp16 scale -> snap -> pack, with the row held in registers.
//
// Steps (turboquant-mlx "How it works", "Quantizing a weight, with no data"; "The ternary
// tier (1.58 bits)"): v = H_K (s * w) (unnormalized: the 1/sqrt(K) of R cancels in v / r
// and is applied to the stored scale only), r = sqrt(mean_g v^2), scale = fp16(r / sqrt(K)),
// u = v / r (0 when r = 0), idx = #{k : u > t_k} decided in binary32, then bit or trit
// packing. Rotation and RMS are computed in double precision, as in k_encode.
//
// Work layout. Each wave works alone on batches of 2048 elements, 32 values per lane (64
// registers of fp64), so that two waves share a SIMD (16 KB of LDS each, two 4-wave
// workgroups per CU). The Sylvester transform of a row is the product of one butterfly
// stage per bit of the element index, in any order. A batch holds 2048 / K whole rows
// when K <= 2048. A row of 4096 is two batches: the stage of the top element bit runs on
// load, v_h = s0 x0 + (-1)^h s1 x1 for the row's halves x0, x1, and the 2048-point
// transform of v_h gives elements 2048 h .. 2048 h + 2047 of the row; the two halves go to
// two waves of one workgroup, each reading the whole row. With Kv = 2^q = min(K, 2048)
// (the "virtual row"), the remaining stages run in register phases with LDS exchanges
// between them:
//   A (as loaded): lane t of a virtual row holds the 8-element chunks t + c Kv/32 (c < 4):
//       element bits 0-2 and q-2, q-1 in registers: 5 stages;
//   B (q >= 8): lane e + 8 h holds batch elements e + 8 j + 256 h (j < 32): bits 3-7 in
//       registers, the stages of bits 3..min(7, q-3); for q = 11 also the stage of bit 8,
//       a butterfly with lane ^ 8 (a DPP row rotation);
//   C (final): lane t holds batch elements 32 t .. 32 t + 31; for q <= 7 the stages of
//       bits 3..q-3 run here; then group sums (a group of 64 or 128 spans 2 or 4 lanes),
//       scales, snap and packing.
// The exchanges go through the wave's own 16 KB buffer, addressed so that none has bank
// conflicts (pair_slot), and need no workgroup barrier.
#include "device_common.hpp"
#include "encode_lane.hpp"
#include "internal.hpp"

namespace tq {
namespace {

constexpr int kP2Waves = 4;                        // waves per workgroup
constexpr int kP2Threads = 64 * kP2Waves;
constexpr int kP2Batch = 2048;                     // elements per wave batch
constexpr int kP2BufBytes = kP2Batch * 8;          // fp64 exchange buffer per wave
constexpr int kP2MaxK = 4096;

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

// Bank group of the 16-byte slot of element pair P (elements 2P, 2P + 1) of a batch: eight
// slots span the 32 banks, and the slot's low three bits are XORed with
//   g(y) = (y0 ^ y2) | (y1 ^ y3) << 1 | (y1 ^ y4) << 2,   y = P >> 3,
// which spreads the lanes of every pass of the three exchanges over distinct banks (found
// by an exhaustive search over the linear maps of this form, for every row length):
//   A writes  (16 B, 8 lanes a pass):  P = rl Kv/2 + 4 (t + c Kv/32) + s
//   B accesses (8 B, 16 lanes a pass): P = (e >> 1) + 4 j + 128 h, half e & 1
//   C reads   (16 B, 8 lanes a pass):  P = 16 t + i
// g is linear over GF(2): the term of a sum of parts with disjoint bits is the XOR of
// the parts' terms.
__device__ __forceinline__ constexpr int slot_mix(int P) {
  const int y = P >> 3;
  return ((y ^ (y >> 2)) & 1) | ((((y >> 1) ^ (y >> 3)) & 1) << 1) |
         ((((y >> 1) ^ (y >> 4)) & 1) << 2);
}

// WDT: 0 fp32, 1 bf16, 2 fp16 source rows; NH source halves (2 for a row of 4096).
template <int WDT, int NH>
struct P2Raw {
  static constexpr int kW = WDT == 0 ? 8 : 4;  // words per 8-element chunk
  uint32_t w[NH][4][kW];
};

// The lane's four chunks t + tr c of the virtual row (of both halves of the row for NH = 2).
template <int WDT, int NH>
__device__ __forceinline__ void p2_load(P2Raw<WDT, NH>& raw, const char* row_base, int t, int tr) {
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t off = static_cast<uint32_t>(8 * (t + tr * c) + 2048 * h) * (WDT == 0 ? 4u : 2u);
      const u32x4_t a = ld_at<u32x4_t>(row_base, off);
      raw.w[h][c][0] = a.x; raw.w[h][c][1] = a.y; raw.w[h][c][2] = a.z; raw.w[h][c][3] = a.w;
      if constexpr (WDT == 0) {
        const u32x4_t b = ld_at<u32x4_t>(row_base, off + 16u);
        raw.w[h][c][4] = b.x; raw.w[h][c][5] = b.y; raw.w[h][c][6] = b.z; raw.w[h][c][7] = b.w;
      }
    }
}

// Sign masks of one chunk's source words: the sign s_e (bit e of `sbits`) as the sign bit
// of element e in its word (flipping it in the source format is exact).
template <int WDT>
__device__ __forceinline__ uint32_t sign_word(uint32_t sbits, int k) {
  if constexpr (WDT == 0) return ((sbits >> k) & 1u) << 31;
  else return (((sbits >> (2 * k)) & 1u) << 15) | (((sbits >> (2 * k + 1)) & 1u) << 31);
}

// Element e of a chunk as fp64, from its source words with the signs already applied.
template <int WDT>
__device__ __forceinline__ double p2_elem(const uint32_t* wd, int e) {
  if constexpr (WDT == 0) {
    return static_cast<double>(__uint_as_float(wd[e]));
  } else {
    const uint32_t x = wd[e >> 1];
    if constexpr (WDT == 1) {
      return static_cast<double>(__uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16)));
    } else {
      const uint16_t hb = static_cast<uint16_t>((e & 1) ? (x >> 16) : (x & 0xffffu));
      return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, hb)));
    }
  }
}

// SPLIT: rows of 4096, one half per batch. At most 256 registers: two waves per SIMD.
template <int WDT, int LEVELS, int LG_G, bool SPLIT>
__global__ __launch_bounds__(kP2Threads, 2) void k_encode_p2(EncP2Params p) {
  constexpr int NH = SPLIT ? 2 : 1;
  extern __shared__ u32x4_t p2_smem[];
  __shared__ uint32_t sw[kP2MaxK / 32];
  __shared__ uint32_t tk[LEVELS == 256 ? 128 : 1];  // 8-bit codebook: searched thresholds
  if constexpr (LEVELS == 256)
    if (threadIdx.x < 128) tk[threadIdx.x] = p.tbig[threadIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lg = p.lg_k, K = 1 << lg;
  const int q = SPLIT ? 11 : lg;             // log2 of the virtual row length Kv
  const int Kv = 1 << q;
  const int lg_tr = q - 5, tr = 1 << lg_tr;  // lanes per virtual row
  const int rpb = kP2Batch >> q;             // virtual rows per batch
  const int rl = lane >> lg_tr, t = lane & (tr - 1);
  char* buf = reinterpret_cast<char*>(p2_smem) + wave * kP2BufBytes;

  const int64_t nbatch = SPLIT ? 2 * p.rows : (p.rows + rpb - 1) / rpb;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kP2Waves;
  int64_t b = static_cast<int64_t>(blockIdx.x) * kP2Waves + wave;
  const size_t esz = WDT == 0 ? 4 : 2;
  // the source row of this lane in batch bb (clamped: a partial last batch reads real rows)
  auto src_row = [&](int64_t bb) {
    const int64_t r = SPLIT ? (bb >> 1) : bb * rpb + rl;
    return r < p.rows ? r : p.rows - 1;
  };
  // the first batch's rows are requested before the signs are made
  P2Raw<WDT, NH> raw;
  if (b < nbatch) p2_load<WDT, NH>(raw, static_cast<const char*>(p.W) + src_row(b) * K * esz, t, tr);

  // the rotation's sign bits, once per workgroup: lane l of a wave makes the sign of
  // element 64 n + l, and a ballot packs the wave's 64 into words 2 n, 2 n + 1
  for (int n = wave; n < (K >> 6); n += kP2Waves) {
    const uint64_t bits = __ballot(static_cast<int>(splitmix64_at(p.seed, static_cast<uint64_t>(64 * n + lane)) >> 63));
    if (lane == 0) {
      sw[2 * n] = static_cast<uint32_t>(bits);
      sw[2 * n + 1] = static_cast<uint32_t>(bits >> 32);
    }
  }
  __syncthreads();
  // the signs of this lane's chunks t + c tr (of half h of the row) as masks of their
  // source words (the same in every batch)
  constexpr int KW = P2Raw<WDT, NH>::kW;
  uint32_t smask[NH][4][KW];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int u = t + tr * c + 256 * h;
      const uint32_t sb = (sw[u >> 2] >> (8 * (u & 3))) & 0xffu;
#pragma unroll
      for (int k = 0; k < KW; ++k) smask[h][c][k] = sign_word<WDT>(sb, k);
    }

  // LDS byte addresses (see slot_mix), as lane bases plus compile-time offsets:
  // A writes: pair rl Kv/2 + 4 t + (4 tr c + s); the XOR term of the uniform part is
  // computed per chunk
  const int pa = rl * (Kv >> 1) + 4 * t;
  const int amix = (pa & 4) ^ slot_mix(pa);
  const int abase = 16 * (pa & ~7);
  // B: pair (e >> 1) + 128 h + 4 j, half e & 1 -> bbase[k] + 128 (j >> 1), k the
  // compile-time part 4 (j & 1) ^ mix(4 j) of the slot's low bits
  const int be = lane & 7, bh = lane >> 3;
  int bbase[8];
  {
    const int pb = (be >> 1) + 128 * bh, F = (pb & 7) ^ slot_mix(pb);
#pragma unroll
    for (int k = 0; k < 8; ++k) bbase[k] = 16 * ((pb & ~7) + (F ^ k)) + 8 * (be & 1);
  }
  // C reads: pair 16 lane + i (i < 16) -> cbase[k] + 128 (i >> 3), k = (i & 7) ^ mix(i)
  int cbase[8];
  {
    const int pc = 16 * lane, F = slot_mix(pc);
#pragma unroll
    for (int k = 0; k < 8; ++k) cbase[k] = 16 * (pc + (F ^ k));
  }

  if (b >= nbatch) return;

  // C lanes: virtual row and first element of the lane's 32
  const int crl = lane >> lg_tr, ci0 = 32 * (lane & (tr - 1));

  for (; b < nbatch; b += stride) {
    // the half of the row this batch produces (SPLIT), as a sign flip of the second half
    const uint32_t hflip = SPLIT && (b & 1) ? (WDT == 0 ? 0x80000000u : 0x80008000u) : 0u;
    double v[32];
    // layout A: v[8 c + e] = element 8 (t + c tr) + e of the virtual row
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t x0[KW], x1[KW];
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        x0[k] = raw.w[0][c][k] ^ smask[0][c][k];
        if constexpr (SPLIT) x1[k] = raw.w[1][c][k] ^ smask[1][c][k] ^ hflip;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[8 * c + e] = p2_elem<WDT>(x0, e);
        if constexpr (SPLIT) v[8 * c + e] += p2_elem<WDT>(x1, e);
      }
    }
    if (b + stride < nbatch)
      p2_load<WDT, NH>(raw, static_cast<const char*>(p.W) + src_row(b + stride) * K * esz, t, tr);

    // phase A: element bits 0-2 and q-2, q-1
    bfly<0>(v); bfly<1>(v); bfly<2>(v); bfly<3>(v); bfly<4>(v);

#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int U = 4 * tr * c;  // uniform part of the pair index (bits >= 3)
      const int m = amix ^ slot_mix(U);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int addr = abase + 16 * U + 16 * (m ^ s2);
        *reinterpret_cast<double2*>(buf + addr) = make_double2(v[8 * c + 2 * s2], v[8 * c + 2 * s2 + 1]);
      }
    }
    wave_lds_sync();
    if (q >= 8) {
      // phase B: lane (e, h) holds batch elements e + 8 j + 256 h: bits 3-7 in registers
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int k = (4 * (j & 1)) ^ slot_mix(4 * j);
        v[j] = *reinterpret_cast<const double*>(buf + bbase[k] + 128 * (j >> 1));
      }
      bfly<0>(v); bfly<1>(v); bfly<2>(v);
      if (q >= 9) bfly<3>(v);
      if (q >= 10) bfly<4>(v);
      if (q >= 11) {
        // bit 8 is bit 0 of h, lane bit 3: the lower lane of a pair gets v + o, the upper
        // one o - v, as o + (-v) with the sign flipped in the high word (exact)
        const int flip = (lane & 8) ? static_cast<int>(0x80000000u) : 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const double o = lane_xor<8>(v[j]);
          v[j] = __hiloint2double(__double2hiint(v[j]) ^ flip, __double2loint(v[j])) + o;
        }
      }
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int k = (4 * (j & 1)) ^ slot_mix(4 * j);
        *reinterpret_cast<double*>(buf + bbase[k] + 128 * (j >> 1)) = v[j];
      }
      wave_lds_sync();
    }
    // layout C: lane holds batch elements 32 lane + j
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = (i & 7) ^ slot_mix(i);
      const double2 d = *reinterpret_cast<const double2*>(buf + cbase[k] + 128 * (i >> 3));
      v[2 * i] = d.x;
      v[2 * i + 1] = d.y;
    }
    if (q <= 7) {
      bfly<3>(v);
      if (q == 7) bfly<4>(v);
    }

    // this lane's row and the position of its 32 elements in it
    const int64_t row = SPLIT ? (b >> 1) : b * rpb + crl;
    const int off = SPLIT ? 2048 * static_cast<int>(b & 1) + ci0 : ci0;
    const bool live = row < p.rows;

    constexpr int NW = lane_code_bits<LEVELS>();  // words of the lane's 32 codes
    uint32_t w[NW];
    lane_encode<LEVELS, LG_G>(v, p.tbits, tk, p.inv_sqrt_k, lane, row, off, live, K, p.scales, w);

    if constexpr (LEVELS != 3) {
      if (live) {
        uint32_t* dst = p.codes + row * p.wpr + (off >> 5) * NW;
#pragma unroll
        for (int k = 0; k < NW; ++k) dst[k] = w[k];
      }
      wave_lds_sync();
    } else {
      // trit words (20 digits) do not line up with a lane's 32 elements: the digits go
      // through the buffer as bytes, then each lane packs words t, t + tr, ... of its row
      // (rows of 4096 never take this kernel with trits)
      wave_lds_sync();
      u32x4_t* bw = reinterpret_cast<u32x4_t*>(buf + 32 * lane);
      bw[0] = u32x4_t{w[0], w[1], w[2], w[3]};
      bw[1] = u32x4_t{w[4], w[5], w[6], w[7]};
      wave_lds_sync();
      const int64_t prow = b * rpb + rl;
      const uint32_t* rb = reinterpret_cast<const uint32_t*>(buf + rl * Kv);
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
        if (prow < p.rows) p.codes[prow * p.wpr + wi] = word;
      }
      wave_lds_sync();
    }
  }
}

template <int WDT, int LEVELS, bool SPLIT>
hipError_t launch_p2_l(const EncP2Params& p, int group, int grid, hipStream_t s) {
  void (*kern)(EncP2Params) = nullptr;
  switch (group) {
    case 16: kern = k_encode_p2<WDT, LEVELS, 4, SPLIT>; break;
    case 32: kern = k_encode_p2<WDT, LEVELS, 5, SPLIT>; break;
    case 64: kern = k_encode_p2<WDT, LEVELS, 6, SPLIT>; break;
    default: kern = k_encode_p2<WDT, LEVELS, 7, SPLIT>; break;
  }
  const size_t lds = static_cast<size_t>(kP2Waves) * kP2BufBytes;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kP2Threads), lds, s, p);
  return hipGetLastError();
}

template <int WDT, bool SPLIT>
hipError_t launch_p2_w(const EncP2Params& p, int levels, int group, int grid, hipStream_t s) {
  switch (levels) {
    case 3:
      if constexpr (!SPLIT) return launch_p2_l<WDT, 3, SPLIT>(p, group, grid, s);
      return hipErrorInvalidValue;  // never: trit rows of 4096 take k_encode
    case 4: return launch_p2_l<WDT, 4, SPLIT>(p, group, grid, s);
    case 8: return launch_p2_l<WDT, 8, SPLIT>(p, group, grid, s);
    case 256: return launch_p2_l<WDT, 256, SPLIT>(p, group, grid, s);
    default: return launch_p2_l<WDT, 16, SPLIT>(p, group, grid, s);
  }
}

}  // namespace

bool positive_threshold_bits(int levels, uint32_t* dst) {
  // the negative thresholds of a symmetric codebook are the negations of the positive ones
  const float* t = levels == 256 ? codebook256()->t : codebook_for(levels)->t;
  const int npos = levels == 3 ? 1 : levels / 2 - 1;
  for (int q = 0; q < npos; ++q) {
    const float tq = t[levels - 1 - npos + q];
    const float tn = t[npos - 1 - q];
    if (!(tq > 0.f) || tn != -tq) return false;
    dst[q] = __builtin_bit_cast(uint32_t, tq);
  }
  return levels == 3 || t[levels / 2 - 1] == 0.f;
}

// Trit words of a row of 4096 would straddle the two halves' batches: that case takes
// k_encode.
bool encode_p2_supported(int K, int m, int levels) {
  return m == 1 && K >= 64 && K <= kP2MaxK && !(levels == 3 && K > kP2Batch);
}

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
  if (!positive_threshold_bits(levels, levels == 256 ? p.tbig : p.tbits)) return hipErrorInvalidValue;
  const bool split = K > kP2Batch;
  const int64_t nbatch = split ? 2 * rows : (rows + kP2Batch / K - 1) / (kP2Batch / K);
  const int64_t want = (nbatch + kP2Waves - 1) / kP2Waves;
  const int grid = static_cast<int>(want < 512 ? want : 512);  // two workgroups per CU
  switch (wdt) {
    case 0: return split ? launch_p2_w<0, true>(p, levels, group, grid, s) : launch_p2_w<0, false>(p, levels, group, grid, s);
    case 1: return split ? launch_p2_w<1, true>(p, levels, group, grid, s) : launch_p2_w<1, false>(p, levels, group, grid, s);
    default: return split ? launch_p2_w<2, true>(p, levels, group, grid, s) : launch_p2_w<2, false>(p, levels, group, grid, s);
  }
}

}  // namespace tq
