// Encode of weight rows of length K = m * 2^k (m = 12, 20, 28; 32 <= 2^k <= 256) with the
// rotation in registers: rotate -> group RMS -> fp16 scale -> snap -> pack.
//
// Steps (turboquant-mlx "How it works", "Quantizing a weight, with no data"; "The ternary
// tier (1.58 bits)"): v = H_K (s * w) with H_K = H_m (x) H_P, P = 2^k, element (a, b) of a
// row at a P + b (unnormalized: the 1/sqrt(K) of R cancels in v / r and is applied to the
// stored scale only), r = sqrt(mean_g v^2), scale = fp16(r / sqrt(K)), u = v / r (0 when
// r = 0), idx = #{k : u > t_k} decided in binary32, then bit or trit packing. Rotation and
// RMS in double precision, as in k_encode and k_encode_p2.
//
// Work layout. A 4-wave workgroup takes batches of R = floor(8192 / K) rows, transformed in
// 64 KB of LDS (fp64), in three phases separated by barriers; two workgroups share a CU,
// so one computes while the other waits at a barrier:
//   A: lane (row, b) loads column b of its row (m elements, P apart), applies the signs
//      and the m-point factor in registers (fast forms of fwht_block.hpp) and writes the m
//      outputs; 256 / P rows per pass;
//   B (P >= 64): lane (sub-row, l) holds 32 elements of one length-P sub-row whose index
//      bits 5..k-1 are in registers (with the 10 - k filler bits 1..10-k; bit 0 and the
//      rest come from l): the stages of bits 5..k-1;
//   C: lane t holds batch elements 32 t .. 32 t + 31: the stages of bits 0-4, then the
//      group sums, scales, snap and packing of encode_lane.hpp.
// LDS addresses: the 16-byte slot of element pair P2 = e / 2 has its low three bits XORed
// with g(P2 >> 3) = (y0 ^ y1 ^ y2) | (y2 ^ y4) << 1 | y3 << 2, which keeps every B and C
// pass free of bank conflicts for all twelve (m, k) (checked exhaustively); an A pass
// of 16 lanes covers one aligned run of 16 elements, which any such XOR keeps
// conflict-free.
#include <utility>

#include "device_common.hpp"
#include "encode_lane.hpp"
#include "fwht_block.hpp"
#include "internal.hpp"

namespace tq {
namespace {

constexpr int kMWaves = 4;
constexpr int kMThreads = 64 * kMWaves;
constexpr int kMBatch = 8192;  // elements of a workgroup's batch of rows
constexpr int kMMaxK = 28 * 256;

struct EncMParams {
  const void* W;
  int64_t rows;
  uint64_t seed;
  uint32_t* codes;
  uint16_t* scales;
  double inv_sqrt_k;
  uint32_t tbits[8];   // positive decision thresholds (binary32 bits), ascending
  uint32_t tbig[128];  // the same for the 256-level codebook (127 used)
  int K, lg_p, R, wpr, wdt;
  uint32_t inv_k;  // ceil(2^32 / K): t / K = mulhi(t, inv_k) for t < 2^13
};

__device__ __forceinline__ constexpr int mslot_mix(int P2) {
  const int y = P2 >> 3;
  return ((y ^ (y >> 1) ^ (y >> 2)) & 1) | ((((y >> 2) ^ (y >> 4)) & 1) << 1) |
         (((y >> 3) & 1) << 2);
}

// byte address of batch element e
__device__ __forceinline__ int melem_addr(int e) {
  const int P2 = e >> 1;
  return 16 * (P2 ^ mslot_mix(P2)) + 8 * (e & 1);
}

// Source element bits (zero-extended 16-bit types) with the sign bit flipped if s, as fp64.
__device__ __forceinline__ double m_elem(uint32_t bits, uint32_t s, int wdt) {
  if (wdt == 0) return static_cast<double>(__uint_as_float(bits ^ (s << 31)));
  bits ^= s << 15;
  if (wdt == 1) return static_cast<double>(__uint_as_float(bits << 16));
  return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits))));
}

// Phase B for P = 2^(10 - F): lane (sr, ls), register j -> element
// sr P + (ls & 1) + (j & (2^F - 1)) * 2 + (ls >> 1) * 2^(F + 1) + (j >> F) * 32.
template <int F>
__device__ __forceinline__ void m_phase_b(char* buf, int tid, int nsub) {
  constexpr int KK = 5 - F;  // lane bits per sub-row: P / 32 lanes
  constexpr int P = 1 << (10 - F);
  const int sr = tid >> KK, ls = tid & ((1 << KK) - 1);
  if (sr >= nsub) return;
  const int El = sr * P + (ls & 1) + ((ls >> 1) << (F + 1));
  // El and the register part J have disjoint bits, so the slot of El | J is
  // ((El >> 1) & ~7) + ((J >> 1) & ~7) + (lam ^ kap(J)) with the XOR terms split likewise
  const int lam = ((El >> 1) & 7) ^ mslot_mix(El >> 1);
  int base[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) base[k] = 16 * ((El >> 1) & ~7) + 8 * (El & 1) + 16 * (lam ^ k);
  auto joff = [](int j) { return ((j & ((1 << F) - 1)) << 1) | ((j >> F) << 5); };
  double v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int J = joff(j);
    const int kap = ((J >> 1) & 7) ^ mslot_mix(J >> 1);
    v[j] = *reinterpret_cast<const double*>(buf + base[kap] + 16 * ((J >> 1) & ~7));
  }
  // register bits F..4 are element bits 5..k-1
  if constexpr (F <= 4) bfly<4>(v);
  if constexpr (F <= 3) bfly<3>(v);
  if constexpr (F <= 2) bfly<2>(v);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int J = joff(j);
    const int kap = ((J >> 1) & 7) ^ mslot_mix(J >> 1);
    *reinterpret_cast<double*>(buf + base[kap] + 16 * ((J >> 1) & ~7)) = v[j];
  }
}

// Passes of phase A (256 / P rows each, floor(8192 / K) rows per batch): at most 3 for
// m = 12 and 2 otherwise. The loads of the first NP passes of a batch are requested one
// batch ahead (all of them for m = 12; the registers of more m = 20 or 28 columns would
// spill), later passes' loads at their start.
template <int M>
constexpr int prefetch_passes() {
  return M == 12 ? 3 : 1;
}

template <int M, int LEVELS, int LG_G, bool FAST_A>
__global__ __launch_bounds__(kMThreads, 2) void k_encode_m(EncMParams p) {
  constexpr int NP = prefetch_passes<M>();
  constexpr int MAXP = M == 12 ? 3 : 2;
  constexpr bool UNROLL = M == 12;  // passes unrolled (prefetched registers of every pass)
  extern __shared__ double mbuf[];  // R K fp64 elements of the batch (swizzled)
  __shared__ uint32_t sw[kMMaxK / 32];
  __shared__ uint32_t tk[LEVELS == 256 ? 128 : 1];
  char* buf = reinterpret_cast<char*>(mbuf);
  if constexpr (LEVELS == 256)
    if (threadIdx.x < 128) tk[threadIdx.x] = p.tbig[threadIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K, lgp = p.lg_p, P = 1 << lgp, R = p.R, wdt = p.wdt;
  const int rpp = kMThreads >> lgp;  // rows per A pass
  const int npass = (R + rpp - 1) / rpp;
  const int ar = tid >> lgp, ab = tid & (P - 1);  // A lane: row in the pass, column
  const int64_t nbatch = (p.rows + R - 1) / R;
  int64_t bt = blockIdx.x;
  const size_t esz = wdt == 0 ? 4 : 2;

  // column ab of row ar of pass ps of batch b (clamped to the last row), addressed from
  // the batch's first row (uniform) by 32-bit offsets
  auto load_col = [&](uint32_t (&raw)[M], int64_t b, int ps) {
    const int64_t r0 = b * R;
    int64_t row = r0 + ps * rpp + ar;
    row = row < p.rows ? row : p.rows - 1;
    const char* src = static_cast<const char*>(p.W) + r0 * K * static_cast<int64_t>(esz);
    const uint32_t lo = static_cast<uint32_t>((row - r0) * K + ab);
    if (wdt == 0) {
#pragma unroll
      for (int a = 0; a < M; ++a) raw[a] = ld_at<uint32_t>(src, (lo + static_cast<uint32_t>(a * P)) * 4u);
    } else {
#pragma unroll
      for (int a = 0; a < M; ++a) raw[a] = ld_at<uint16_t>(src, (lo + static_cast<uint32_t>(a * P)) * 2u);
    }
  };
  uint32_t raw[NP][M];
  auto load_batch = [&](int64_t b) {
#pragma unroll
    for (int ps = 0; ps < NP; ++ps)
      if (ps < npass) load_col(raw[ps], b, ps);
  };
  if (bt < nbatch) load_batch(bt);

  // the rotation's sign bits, once per workgroup (lane l of a wave: element 64 n + l)
  for (int n = wave; n < (K >> 6); n += kMWaves) {
    const uint64_t bits = __ballot(static_cast<int>(splitmix64_at(p.seed, static_cast<uint64_t>(64 * n + lane)) >> 63));
    if (lane == 0) {
      sw[2 * n] = static_cast<uint32_t>(bits);
      sw[2 * n + 1] = static_cast<uint32_t>(bits >> 32);
    }
  }
  __syncthreads();
  // the signs of this lane's column: bit a = sign of element a P + ab
  uint32_t smask = 0;
#pragma unroll
  for (int a = 0; a < M; ++a) {
    const int e = a * P + ab;
    smask |= ((sw[e >> 5] >> (e & 31)) & 1u) << a;
  }

  // Addresses of the m-point outputs (FAST_A: P >= 128). The slot swizzle is linear over
  // the bits of the element index and reads only bits 4..8, so with P >= 128 and m a
  // multiple of 4 element (row r, a, column b) lies at 8 P (r m + a - a % 4) + tA[a % 4],
  // tA[k] the address of element k P + b: one add per output instead of the swizzle.
  static_assert(M % 4 == 0, "the address split needs m = 0 mod 4");
  int tA[4];
  if constexpr (FAST_A) {
#pragma unroll
    for (int k = 0; k < 4; ++k) tA[k] = melem_addr(k * P + ab);
  }

  // C lanes: 32 consecutive elements of the batch
  const int nC = (R * K) >> 5;
  const int crr = static_cast<int>(__umulhi(static_cast<uint32_t>(32 * tid), p.inv_k));  // row in batch
  const int coff = 32 * tid - crr * K;
  int cbase[8];
  {
    const int pc = 16 * tid, F = mslot_mix(pc);
#pragma unroll
    for (int k = 0; k < 8; ++k) cbase[k] = 16 * (pc + (F ^ k));
  }

  for (; bt < nbatch; bt += gridDim.x) {
    const int64_t row0 = bt * R;
    // phase A: signs and the m-point factor on each column
#pragma unroll
    for (int ps = 0; ps < (UNROLL ? MAXP : npass); ++ps) {
      if (ps >= npass) break;
      uint32_t(&rw)[M] = raw[UNROLL ? (ps < NP ? ps : NP - 1) : 0];
      if (ps >= NP) load_col(rw, bt, ps);
      double x[M];
      if (wdt == 0) {
#pragma unroll
        for (int a = 0; a < M; ++a) x[a] = m_elem(rw[a], (smask >> a) & 1u, 0);
      } else if (wdt == 1) {
#pragma unroll
        for (int a = 0; a < M; ++a) x[a] = m_elem(rw[a], (smask >> a) & 1u, 1);
      } else {
#pragma unroll
        for (int a = 0; a < M; ++a) x[a] = m_elem(rw[a], (smask >> a) & 1u, 2);
      }
      // the next batch is requested as soon as the last pass's registers are free
      if (ps == npass - 1 && bt + gridDim.x < nbatch) load_batch(bt + gridDim.x);
      const int r = ps * rpp + ar;
      if (r < R) {  // rows past the end of the data are transformed but never stored
        auto factor = [&](auto put) __attribute__((always_inline)) {
          if constexpr (M == 28) {
            hadamard28_side<double, 0>(x, [&](int Rr, double y) { put(2 * Rr, y); });
            hadamard28_side<double, 1>(x, [&](int Rr, double y) { put(2 * Rr + 1, y); });
          } else {
            [&]<int... A>(std::integer_sequence<int, A...>) {
              (put(A, hadamard_row<double, M, A>(x, std::make_integer_sequence<int, M>{})), ...);
            }(std::make_integer_sequence<int, M>{});
          }
        };
        if constexpr (FAST_A) {
          const int bq = (r * M) << (lgp + 3);
          factor([&](int a, double y) {
            *reinterpret_cast<double*>(buf + bq + ((a & ~3) << (lgp + 3)) + tA[a & 3]) = y;
          });
        } else {
          const int e0 = r * K + ab;
          factor([&](int a, double y) {
            *reinterpret_cast<double*>(buf + melem_addr(e0 + a * P)) = y;
          });
        }
      }
    }
    __syncthreads();
    // phase B: element bits 5..k-1 of every sub-row
    switch (lgp) {
      case 6: m_phase_b<4>(buf, tid, R * M); break;
      case 7: m_phase_b<3>(buf, tid, R * M); break;
      case 8: m_phase_b<2>(buf, tid, R * M); break;
      default: break;
    }
    __syncthreads();
    // phase C: bits 0-4, then the encode of the lane's 32 elements (every barrier below is
    // reached by every thread)
    constexpr int NW = lane_code_bits<LEVELS>();
    uint32_t w[NW];
    if (tid < nC) {
      double v[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = (i & 7) ^ mslot_mix(i);
        const double2 d = *reinterpret_cast<const double2*>(buf + cbase[k] + 128 * (i >> 3));
        v[2 * i] = d.x;
        v[2 * i + 1] = d.y;
      }
      bfly<0>(v); bfly<1>(v); bfly<2>(v); bfly<3>(v); bfly<4>(v);
      const int64_t row = row0 + crr;
      const bool live = row < p.rows;
      lane_encode<LEVELS, LG_G>(v, p.tbits, tk, p.inv_sqrt_k, lane, row, coff, live, K, p.scales, w);
      if constexpr (LEVELS != 3) {
        if (live) {
          uint32_t* dst = p.codes + row * p.wpr + (coff >> 5) * NW;
#pragma unroll
          for (int k = 0; k < NW; ++k) dst[k] = w[k];
        }
      }
    }
    if constexpr (LEVELS == 3) {
      // trit words (20 digits) do not line up with the lanes' 32 elements: the digits go
      // through LDS as bytes, once every lane has read its elements
      __syncthreads();
      if (tid < nC) {
        u32x4_t* bw = reinterpret_cast<u32x4_t*>(buf + 32 * tid);
        bw[0] = u32x4_t{w[0], w[1], w[2], w[3]};
        bw[1] = u32x4_t{w[4], w[5], w[6], w[7]};
      }
      __syncthreads();
      const int64_t left = p.rows - row0;
      const int nr = left < R ? static_cast<int>(left) : R;
      for (int idx = tid; idx < nr * p.wpr; idx += kMThreads) {
        const int rr = idx / p.wpr, wi = idx - rr * p.wpr;
        const uint32_t* rb = reinterpret_cast<const uint32_t*>(buf + rr * K + 20 * wi);
        uint32_t d[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) d[k] = rb[k];
        uint32_t word = 0;
#pragma unroll
        for (int k = 19; k >= 0; --k) {
          const uint32_t digit = (d[k >> 2] >> (8 * (k & 3))) & 0xffu;
          word = word * 3u + (20 * wi + k < K ? digit : 0u);
        }
        p.codes[(row0 + rr) * p.wpr + wi] = word;
      }
    }
    __syncthreads();  // the next batch's phase A overwrites the buffer
  }
}

template <int M, int LEVELS, bool FAST_A>
hipError_t launch_m_f(const EncMParams& p, int group, int grid, size_t lds, hipStream_t s) {
  void (*kern)(EncMParams) = nullptr;
  switch (group) {
    case 16: kern = k_encode_m<M, LEVELS, 4, FAST_A>; break;
    case 32: kern = k_encode_m<M, LEVELS, 5, FAST_A>; break;
    case 64: kern = k_encode_m<M, LEVELS, 6, FAST_A>; break;
    default: kern = k_encode_m<M, LEVELS, 7, FAST_A>; break;
  }
  // lds <= 64 KB, the default limit of dynamic LDS
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kMThreads), lds, s, p);
  return hipGetLastError();
}

template <int M, int LEVELS>
hipError_t launch_m_l(const EncMParams& p, int group, int grid, size_t lds, hipStream_t s) {
  // the one-add output addresses of phase A hold for rows of P >= 128
  return p.lg_p >= 7 ? launch_m_f<M, LEVELS, true>(p, group, grid, lds, s)
                     : launch_m_f<M, LEVELS, false>(p, group, grid, lds, s);
}

template <int M>
hipError_t launch_m_m(const EncMParams& p, int levels, int group, int grid, size_t lds, hipStream_t s) {
  switch (levels) {
    case 3: return launch_m_l<M, 3>(p, group, grid, lds, s);
    case 4: return launch_m_l<M, 4>(p, group, grid, lds, s);
    case 8: return launch_m_l<M, 8>(p, group, grid, lds, s);
    case 256: return launch_m_l<M, 256>(p, group, grid, lds, s);
    default: return launch_m_l<M, 16>(p, group, grid, lds, s);
  }
}

}  // namespace

bool encode_m_supported(int K, int m) {
  if (m != 12 && m != 20 && m != 28) return false;
  const int P = K / m;
  return P * m == K && P >= 32 && P <= 256 && (P & (P - 1)) == 0;
}

hipError_t launch_encode_m(const void* W, int wdt, int64_t rows, int K, int m, int levels,
                           int group, uint64_t seed, uint32_t* codes, uint16_t* scales,
                           hipStream_t s) {
  EncMParams p{};
  p.W = W; p.rows = rows; p.seed = seed; p.codes = codes; p.scales = scales;
  p.K = K; p.wdt = wdt;
  const int P = K / m;
  int lg = 0;
  while ((1 << lg) < P) ++lg;
  p.lg_p = lg;
  p.R = kMBatch / K;  // >= 1: K <= 7168
  p.inv_k = static_cast<uint32_t>(((1ull << 32) + K - 1) / K);
  p.inv_sqrt_k = 1.0 / __builtin_sqrt(static_cast<double>(K));
  p.wpr = levels == 3 ? (K + 19) / 20
                      : (K * (levels == 4 ? 2 : levels == 8 ? 3 : levels == 16 ? 4 : 8)) / 32;
  if (!positive_threshold_bits(levels, levels == 256 ? p.tbig : p.tbits)) return hipErrorInvalidValue;
  const int64_t nbatch = (rows + p.R - 1) / p.R;
  const int grid = static_cast<int>(nbatch < 512 ? nbatch : 512);  // two workgroups per CU
  const size_t lds = static_cast<size_t>(p.R) * K * 8;
  switch (m) {
    case 12: return launch_m_m<12>(p, levels, group, grid, lds, s);
    case 20: return launch_m_m<20>(p, levels, group, grid, lds, s);
    default: return launch_m_m<28>(p, levels, group, grid, lds, s);
  }
}

}  // namespace tq
