// gather_qmm: batched gather-GEMM over rows sorted by expert,
//   y[m] = W_e R x[row_token[m]]   for offsets[e] <= m < offsets[e+1].
//
// turboquant-mlx "How it works", "Running a quantized layer", kernel table, third row (a
// large batch sorted by expert). Three launches on the caller's stream:
//   1. k_rot16: the T input rows rotated once into an fp16 workspace with a power-of-two
//      scale per row (rot16.hpp), plus one zero row;
//   2. k_schedule: the table of (expert, 128-row tile) pairs;
//   3. k_gqmm: one workgroup per (tile of 128 rows of one expert, 512 output columns).
//
// k_gqmm. The 8 waves of a workgroup share the tile's 128 gathered input rows, staged
// through LDS one K step at a time (double-buffered, loaded a step ahead with coalesced
// 16-byte loads). Each wave owns 64 output columns: its lanes load and decode their own
// packed codes straight into matrix-core operands (mfma_decode.hpp, the same decoder as
// multi_gather_qmv) and multiply them with v_mfma_f32_32x32x16_f16, so a weight element
// is decoded once per tile and never goes through LDS. Experts with fewer rows than a
// tile run only the 32-row sub-tiles that hold rows.
//
// For v_mfma_f32_32x32x16_f16 lane l holds A[l % 32][8 (l / 32) + j], B[8 (l / 32) + j][l % 32]
// (j < 8) and gets D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] (r < 16). As in multi_gather,
// the K order inside an instruction is free: lane group g = l / 32 takes a contiguous span
// of SPAN elements of the step (Span<L>), fed to MF consecutive instructions 8 at a time.
#include <type_traits>
#include <utility>

#include "internal.hpp"
#include "mfma_decode.hpp"
#include "rot16.hpp"

namespace tq {

constexpr int kQmmWaves = 8;
constexpr int kQmmThreads = 64 * kQmmWaves;
constexpr int kQmmBM = 128;                      // rows per tile: 4 sub-tiles of 32
constexpr int kQmmWN = 64;                       // output columns per wave: 2 tiles of 32
constexpr int kQmmBN = kQmmWN * kQmmWaves;       // output columns per workgroup
// Scales of a tile's rows are staged in LDS (except for the bit formats with groups of
// 16), a window of this many consecutive groups of every row at a time: what the LDS holds
// beside the format's table and the double-buffered input tile.
template <int L>
constexpr int qmm_lds_groups() {
  return L == 3 ? 88 : 32;
}

template <int L>
struct QmmStep {
  static constexpr int BK = 2 * Span<L>::elems;                 // elements per K step
  static constexpr int AST = BK + 8;                            // LDS halves per input row
  static constexpr int UPR = BK / 8;                            // 16-byte units per row
  static constexpr int AU = (kQmmBM * UPR + kQmmThreads - 1) / kQmmThreads;
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

constexpr int kMaxExpertsQmm = 8192;
__device__ __forceinline__ int64_t max_tiles_dev(int64_t M, int E) { return (M + kQmmBM - 1) / kQmmBM + E; }

// Workspace: rotated rows [T+1][K] fp16 (row T all zero) | row scales [T+1] float |
// tile count int32 | tile table int4 [M / 128 + E] ({expert, first row, rows, 0});
// 256-byte aligned sections.
struct QmmLayout {
  size_t rows, scale, count, tiles, total;
};
static int64_t max_tiles(int64_t M, int E) { return (M + kQmmBM - 1) / kQmmBM + E; }
static QmmLayout qmm_layout(const WeightArgs& w, int64_t M, int64_t T) {
  QmmLayout l{};
  l.rows = 0;
  l.scale = align256(static_cast<size_t>(T + 1) * rot16_row_halves(w.K) * 2);
  l.count = l.scale + align256(static_cast<size_t>(T + 1) * 4);
  l.tiles = l.count + 256;
  l.total = l.tiles + align256(static_cast<size_t>(max_tiles(M, w.E)) * 16);
  return l;
}

size_t gather_qmm_workspace(const WeightArgs& w, int64_t M, int64_t T) {
  return qmm_layout(w, M, T).total;
}

constexpr int kSchedThreads = 1024;

// The tile table: expert e's rows offsets[e] .. offsets[e+1] - 1 are cut into tiles of
// 128. Full tiles come first (expert by expert), then the experts' last, partial tiles from
// the largest to the smallest, so that the short tiles fill the end of the launch (longest
// first). Experts with no rows (or inconsistent offsets) get no tile; the table never holds
// more than max_tiles entries. Each thread takes a block of consecutive experts: a
// block-wide scan places the full tiles, a histogram over the partial sizes the rest.
__global__ __launch_bounds__(kSchedThreads) void k_schedule(const int32_t* offsets, int E,
                                                           int64_t M, int32_t* count,
                                                           int4* tiles) {
  constexpr int PER = (kMaxExpertsQmm + kSchedThreads - 1) / kSchedThreads;
  __shared__ int32_t wsum[kSchedThreads / 64];
  __shared__ int32_t pos[kQmmBM];  // next table index for partial tiles of each size
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = threadIdx.x * PER;
  if (threadIdx.x < kQmmBM) pos[threadIdx.x] = 0;
  __syncthreads();
  int nfull[PER], part[PER];
  int local = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = e0 + k;
    const int rows = e < E ? offsets[e + 1] - offsets[e] : 0;
    nfull[k] = rows > 0 ? rows / kQmmBM : 0;
    part[k] = rows > 0 ? rows % kQmmBM : 0;
    local += nfull[k];
    if (part[k] > 0) atomicAdd(&pos[part[k]], 1);
  }
  // inclusive scan of the full-tile counts within the wave, then across the waves
  int v = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0, full = 0;
#pragma unroll
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    full += x;
  }
  if (wave == 0) {
    // partial sizes from 127 rows down to 1: histogram counts -> first table indices, by a
    // wave scan (lane l takes the sizes 127 - 2l and 126 - 2l; size 0 holds no tile)
    const int r0 = kQmmBM - 1 - 2 * lane, r1 = r0 - 1;
    const int c0 = pos[r0], c1 = r1 >= 1 ? pos[r1] : 0;
    int sc = c0 + c1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(sc, off, 64);
      if (lane >= off) sc += t;
    }
    const int at = full + sc - c0 - c1;
    pos[r0] = at;
    if (r1 >= 1) pos[r1] = at + c0;
    if (lane == 63) {
      const int64_t cap = max_tiles_dev(M, E);
      *count = static_cast<int>(full + sc < cap ? full + sc : cap);
    }
  }
  __syncthreads();
  const int64_t cap = max_tiles_dev(M, E);
  int idx = before + v - local;  // first table index of this thread's full tiles
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = e0 + k;
    if (nfull[k] + part[k] == 0) continue;
    const int o0 = offsets[e];
    for (int t = 0; t < nfull[k]; ++t, ++idx)
      if (idx < cap) tiles[idx] = make_int4(e, o0 + t * kQmmBM, kQmmBM, 0);
    if (part[k] > 0) {
      const int at = atomicAdd(&pos[part[k]], 1);
      if (at < cap) tiles[at] = make_int4(e, o0 + nfull[k] * kQmmBM, part[k], 0);
    }
  }
}

struct QmmParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const _Float16* xh;     // rotated rows [T+1][K]
  const float* xs;        // their scales
  const int32_t* row_token;
  const int32_t* count;
  const int4* tiles;
  void* y;
  int64_t T, M;
  int K, N, E, wpr, lg_group, ngk, ydt;
  CodebookArgs cb;
};

__device__ __forceinline__ f32x16_t mfma32_f16(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Scales a lane needs per span: one for the bit formats with groups of 32 or more (a
// 32-element span lies in one group), two with groups of 16, one per fragment for trits
// (40-element spans are not aligned to groups).
template <int L, bool G16>
constexpr int span_scales() {
  return L == 3 ? Span<L>::mf : (G16 ? 2 : 1);
}

// Pipeline registers: the codes and scales of both column tiles of a lane for one K step
// (a ring of qmm_code_ring steps), and the thread's share of one step's input tile (a ring of
// two). Three steps of codes in flight for the bit formats whose scales are staged in LDS;
// the other kernels have no registers for the third.
template <int L, bool SL>
constexpr int qmm_code_ring() {
  return SL && L != 3 ? 3 : 2;
}
template <int L, bool G16>
struct QmmCodes {
  uint32_t w[2][Span<L>::words];
  uint16_t s[2][span_scales<L, G16>()];
};
template <int L>
struct QmmA {
  u32x4_t a[QmmStep<L>::AU];
};

template <typename T>
__device__ __forceinline__ T to_out(float v) {
  return static_cast<T>(v);  // bf16: v_cvt_pk_bf16_f32 (round to nearest even)
}

// Stores of one wave's results: column n (and n + 32) of rows m0 + 32 mt + 8 q + 4 g + i.
template <typename T, int MT>
__device__ __forceinline__ void qmm_store(const QmmParams& p, const f32x16_t (&acc)[MT][2], int m0,
                                          int mrows, int n, int g, const float* txs) {
  T* y = static_cast<T*>(p.y);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float sc[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(txs + 32 * mt + 8 * q + 4 * g);
      sc[4 * q] = v.x; sc[4 * q + 1] = v.y; sc[4 * q + 2] = v.z; sc[4 * q + 3] = v.w;
    }
    const bool full = 32 * mt + 32 <= mrows;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n + 32 * j;
      if (col >= p.N) continue;
      T* base = y + static_cast<int64_t>(m0 + 32 * mt + 4 * g) * p.N + col;
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          base[(8 * (r >> 2) + (r & 3)) * p.N] = to_out<T>(acc[mt][j][r] * sc[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + (r & 3);
          if (32 * mt + 4 * g + row < mrows) base[row * p.N] = to_out<T>(acc[mt][j][r] * sc[r]);
        }
      }
    }
  }
}

template <int L, int MT, bool G16, bool SL>
__device__ __forceinline__ void qmm_tile(const QmmParams& p, int e, int m0, int mrows, int n0,
                                         const uint32_t* lut, _Float16* la, const int32_t* tok,
                                         const float* txs, uint16_t* ls) {
  using S = Span<L>;
  using Q = QmmStep<L>;
  constexpr int NSC = span_scales<L, G16>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, c32 = lane & 31;
  const uint32_t slot = mlut_slot<L>(lane);

  // this lane's two packed rows (output columns), clamped to the last row, as 32-bit offsets
  // from the expert's codes and scales
  const uint32_t* cexp = p.codes + static_cast<int64_t>(e) * p.N * p.wpr;
  const uint16_t* sexp = p.scales + static_cast<int64_t>(e) * p.N * p.ngk;
  uint32_t coff[2], soff[2];
  constexpr int WG = qmm_lds_groups<L>();
  constexpr int sst = WG + 1;  // LDS halves per row of staged scales (odd: no bank conflicts)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int n = n0 + wave * kQmmWN + 32 * j + c32;
    n = n < p.N ? n : p.N - 1;
    coff[j] = static_cast<uint32_t>(n) * p.wpr * 4u;
    soff[j] = SL ? static_cast<uint32_t>((n - n0) * sst) : static_cast<uint32_t>(n) * p.ngk * 2u;
  }
  // groups wbase .. wbase + WG - 1 of the tile's rows are in LDS; the window moves forward
  // when a step needs a group past it (only trits: the bit formats stage their scales only
  // when a row has at most WG groups)
  constexpr bool MOVES = L == 3;
  int wbase = 0;
  auto stage_scales = [&](int gb) {
    const int rows = p.N - n0 < kQmmBN ? p.N - n0 : kQmmBN;
    const int ng = p.ngk - gb < WG ? p.ngk - gb : WG;
    const int total = rows * ng;
    const uint16_t* src = sexp + static_cast<int64_t>(n0) * p.ngk + gb;
    for (int i = threadIdx.x; i < total; i += kQmmThreads) {
      const int r = i / ng, c = i - r * ng;
      ls[r * sst + c] = src[r * p.ngk + c];
    }
  };
  if constexpr (SL) stage_scales(0);
  // this thread's 16-byte units of the input tile (a unit past the tile, which only the
  // trit format has, loads the tile's first unit and is not stored)
  const _Float16* asrc[Q::AU];
  int aoff[Q::AU], ak[Q::AU];
  bool aon[Q::AU];
#pragma unroll
  for (int j = 0; j < Q::AU; ++j) {
    const int i = threadIdx.x + j * kQmmThreads;
    aon[j] = i < kQmmBM * Q::UPR;
    const int ic = aon[j] ? i : 0;
    const int r = ic / Q::UPR, u = ic - r * Q::UPR;
    asrc[j] = p.xh + static_cast<int64_t>(tok[r]) * rot16_row_halves(p.K) + 8 * u;
    aoff[j] = r * Q::AST + 8 * u;
    ak[j] = 8 * u;
  }
  const int last = (p.K - 1) / Q::BK;  // last step holding elements
  const int nsteps = last + 1;

  // Loads are issued unconditionally (indices clamped) so that every loop iteration has the
  // same memory operations and the compiler's count of outstanding loads stays exact.
  auto load_codes = [&](QmmCodes<L, G16>& st, int step) {
    step = step < last ? step : last;
    const int e0 = step * Q::BK + g * S::elems;
    // With K an odd multiple of 32, the second lane group's span of the last step starts at
    // K: its vector loads read the row's last span instead of the words past the row (its
    // inputs are zero, so the values do not matter, but the last row of the last expert
    // ends the buffer).
    const int fw = span_first_word<L>(L == 3 || e0 < p.K ? e0 : p.K - S::elems);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (L == 16) {
        const u32x4_t v = ld_at<u32x4_t>(cexp, coff[j] + fw * 4u);
        st.w[j][0] = v[0]; st.w[j][1] = v[1]; st.w[j][2] = v[2]; st.w[j][3] = v[3];
      } else if constexpr (L == 4) {
        const uint2 v = ld_at<uint2>(cexp, coff[j] + fw * 4u);
        st.w[j][0] = v.x; st.w[j][1] = v.y;
      } else {
#pragma unroll
        for (int i = 0; i < S::words; ++i) {
          const int wi = fw + i < p.wpr ? fw + i : p.wpr - 1;  // spans may run past the row
          st.w[j][i] = ld_at<uint32_t>(cexp, coff[j] + wi * 4u);
        }
      }
      if constexpr (!SL) {
#pragma unroll
        for (int k = 0; k < NSC; ++k) {
          // first element of the k-th scale's fragment(s): fragment k (trits), 16 k (g16)
          const int ek = L == 3 ? e0 + 8 * k : e0 + 16 * k;
          int gi = ek >> p.lg_group;
          gi = gi < p.ngk ? gi : p.ngk - 1;
          st.s[j][k] = ld_at<uint16_t>(sexp, soff[j] + gi * 2u);
        }
      }
    }
  };
  auto fetch_a = [&](QmmA<L>& st, int step) {
    const int k0 = step * Q::BK;
#pragma unroll
    for (int j = 0; j < Q::AU; ++j) {
      const int kc = k0 + ak[j] < p.K ? k0 : 0;
      st.a[j] = *reinterpret_cast<const u32x4_t*>(asrc[j] + kc);
    }
  };
  auto stash_a = [&](const QmmA<L>& st, int buf, int step) {
    const int k0 = step * Q::BK;
#pragma unroll
    for (int j = 0; j < Q::AU; ++j) {
      const u32x4_t v = k0 + ak[j] < p.K ? st.a[j] : u32x4_t{0u, 0u, 0u, 0u};
      if (aon[j]) *reinterpret_cast<u32x4_t*>(la + buf * (kQmmBM * Q::AST) + aoff[j]) = v;
    }
  };

  f32x16_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][j][r] = 0.f;

  // Step t's codes live in ring slot t % CR, loaded CR steps ahead (the table indices of
  // step t + 1 are formed during step t, so a code load has CR - 1 steps to arrive); its
  // inputs live in slot t % 2, loaded three steps ahead and copied to LDS buffer t % 2 at the
  // end of step t - 1. Loads past the last step are clamped to it.
  constexpr int CR = qmm_code_ring<L, SL>();
  QmmCodes<L, G16> cr[CR];
  QmmA<L> ar[2];
  fetch_a(ar[0], 0);
#pragma unroll
  for (int c = 0; c < CR; ++c) load_codes(cr[c], c);
  fetch_a(ar[1], 1);
  stash_a(ar[0], 0, 0);
  fetch_a(ar[0], 2);
  __syncthreads();

  // Table lookups run LA fragments ahead of the multiplies that use them, across step
  // boundaries: slot f of `raw` holds fragment f of the current step, refilled with fragment
  // f of the next step once consumed. Deeper look-ahead where registers allow it.
  constexpr int MF = S::mf;
  constexpr int LA = SL ? 2 : 1;
  SpanIdx<L> xc[2], xn[2];  // table indices of this step and of the next one
  u32x4_t raw[MF][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    span_index<L>(cr[0].w[j], xc[j]);
#pragma unroll
    for (int q = 0; q < LA; ++q) raw[q][j] = span_lookup<L>(xc[j], q, lut, slot);
  }

  auto body = [&](auto slot_of_step, int step) {
    constexpr int P = decltype(slot_of_step)::value & 1;  // input slot and LDS buffer
    constexpr int C = decltype(slot_of_step)::value >> 1;  // code slot
    QmmCodes<L, G16>& cur = cr[C];
    const int e0 = (step < last ? step : last) * Q::BK + g * S::elems;
    uint32_t s2[2][MF];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        const int k = L == 3 ? f : (G16 ? f >> 1 : 0);
        uint32_t sv;
        if constexpr (SL) {
          const int ek = L == 3 ? e0 + 8 * k : e0 + 16 * k;
          int gi = ek >> p.lg_group;
          gi = gi < p.ngk ? gi : p.ngk - 1;
          sv = ls[soff[j] + gi - (MOVES ? wbase : 0)];
        } else {
          sv = cur.s[j][k];
        }
        s2[j][f] = __umul24(sv, 0x10001u);
      }
    }
    // Per fragment f: read its inputs from LDS, issue the lookups of fragment f + LA (of
    // this step or the next), scale fragment f's entries, then the matrix multiplies.
    const _Float16* abuf = la + P * (kQmmBM * Q::AST);
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      u32x4_t a[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        a[mt] = *reinterpret_cast<const u32x4_t*>(abuf + (32 * mt + c32) * Q::AST + g * S::elems + 8 * f);
      const int q = f + LA;
      if (q < MF) {
#pragma unroll
        for (int j = 0; j < 2; ++j) raw[q][j] = span_lookup<L>(xc[j], q, lut, slot);
      } else {
        if (q == MF) {
          // the next step's codes (loaded two steps ago) become table indices
#pragma unroll
          for (int j = 0; j < 2; ++j) span_index<L>(cr[(C + 1) % CR].w[j], xn[j]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) raw[q - MF][j] = span_lookup<L>(xn[j], q - MF, lut, slot);
      }
      u32x4_t b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = scale_pairs(raw[f][j], s2[j][f]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[mt][j] = mfma32_f16(a[mt], b[j], acc[mt][j]);
    }
    // this step's indices are consumed: its code registers take step + CR
    load_codes(cur, step + CR);
#pragma unroll
    for (int j = 0; j < 2; ++j) xc[j] = xn[j];
    stash_a(ar[P ^ 1], P ^ 1, step + 1);
    fetch_a(ar[P ^ 1], step + 3);
    __syncthreads();
  };
  // Before a step whose groups run past the window, the window restarts at the step's first
  // group (the barrier that ends every step has retired the reads of the old window; a
  // window of WG groups covers any step, as WG * group >= BK + group).
  auto advance_window = [&](int step) {
    if constexpr (SL && MOVES) {
      const int sc = step < last ? step : last;
      int hi = (sc * Q::BK + Q::BK - 1) >> p.lg_group;
      hi = hi < p.ngk ? hi : p.ngk - 1;
      if (hi >= wbase + WG) {  // uniform per workgroup
        wbase = (sc * Q::BK) >> p.lg_group;
        stage_scales(wbase);
        __syncthreads();
      }
    }
  };
  // The loop body runs PER steps, the period of the two rings (slot value (t % CR) * 2 + t % 2),
  // and stops after step nsteps - 1.
  constexpr int PER = CR == 3 ? 6 : 2;
  auto run = [&]<int... U>(std::integer_sequence<int, U...>, int step) {
    bool more = true;
    ((more = more && (advance_window(step + U),
                      body(std::integral_constant<int, (U % CR) * 2 + U % 2>{}, step + U),
                      step + U + 1 < nsteps)),
     ...);
    return more;
  };
  for (int step = 0; run(std::make_integer_sequence<int, PER>{}, step); step += PER) {
  }

  // D[8 (r / 4) + 4 g + r % 4][c32] of sub-tile (mt, j), times the row's input scale
  switch (p.ydt) {
    case 0: qmm_store<float, MT>(p, acc, m0, mrows, n0 + wave * kQmmWN + c32, g, txs); break;
    case 1: qmm_store<__bf16, MT>(p, acc, m0, mrows, n0 + wave * kQmmWN + c32, g, txs); break;
    default: qmm_store<_Float16, MT>(p, acc, m0, mrows, n0 + wave * kQmmWN + c32, g, txs); break;
  }
}

template <int L, bool G16, bool SL>
__global__ __launch_bounds__(kQmmThreads) void k_gqmm(QmmParams p) {
  using Q = QmmStep<L>;
  // the table is the first static LDS array: it starts at address 0
  __shared__ __attribute__((aligned(16))) uint32_t lut[mlut_bytes<L>() / 4];
  __shared__ __attribute__((aligned(16))) _Float16 la[2 * kQmmBM * Q::AST];
  __shared__ int32_t tok[kQmmBM];
  __shared__ __attribute__((aligned(16))) float txs[kQmmBM];
  __shared__ uint16_t hs[16];
  __shared__ uint16_t ls[SL ? kQmmBN * (qmm_lds_groups<L>() + 1) : 1];

  // Workgroups are dealt to the 8 XCDs in turn (XCD b % 8). Row tile t goes to XCD t % 8,
  // all its column tiles in a row there, so they share the tile's inputs in that XCD's L2;
  // each XCD takes its row tiles in table order (longest first).
  const int total_mt = *p.count;
  const int nt = (p.N + kQmmBN - 1) / kQmmBN;
  const int b = blockIdx.x;
  const int i = b >> 3;
  const int tl = i / nt, ntile = i - tl * nt;
  const int t = tl * 8 + (b & 7);
  if (t >= total_mt) return;  // uniform per workgroup
  const int4 te = p.tiles[t];
  const int e = te.x, m0 = te.y;
  if (e < 0 || e >= p.E || m0 < 0 || m0 >= p.M) return;  // never touch memory past y
  int mrows = te.z;
  mrows = mrows < p.M - m0 ? mrows : static_cast<int>(p.M - m0);
  if (mrows <= 0) return;
  const int n0 = ntile * kQmmBN;

  if (threadIdx.x < kQmmBM) {
    // padding rows read the zero row T; an out-of-range token reads it too and gives NaN
    int tk = static_cast<int>(p.T);
    float sc = 0.f;
    if (static_cast<int>(threadIdx.x) < mrows) {
      const int v2 = p.row_token[m0 + threadIdx.x];
      if (v2 >= 0 && v2 < p.T) {
        tk = v2;
        sc = p.xs[v2];
      } else {
        sc = __builtin_nanf("");
      }
    }
    tok[threadIdx.x] = tk;
    txs[threadIdx.x] = sc;
  }
  if (threadIdx.x < 16) hs[threadIdx.x] = p.cb.h[threadIdx.x];
  __syncthreads();
  build_mlut<L, kQmmThreads>(lut, hs);
  // (the first barrier inside qmm_tile orders the table writes before any lookup)
  switch ((mrows + 31) >> 5) {
    case 1: qmm_tile<L, 1, G16, SL>(p, e, m0, mrows, n0, lut, la, tok, txs, ls); break;
    case 2: qmm_tile<L, 2, G16, SL>(p, e, m0, mrows, n0, lut, la, tok, txs, ls); break;
    case 3: qmm_tile<L, 3, G16, SL>(p, e, m0, mrows, n0, lut, la, tok, txs, ls); break;
    default: qmm_tile<L, 4, G16, SL>(p, e, m0, mrows, n0, lut, la, tok, txs, ls); break;
  }
}

hipError_t launch_gather_qmm(const WeightArgs& w, const void* x, int xdt, int64_t T,
                             const int32_t* row_token, const int32_t* offsets, int64_t M,
                             bool x_rotated, void* y, int ydt, void* ws, hipStream_t s,
                             const WeightArgs* w2) {
  if (M == 0 || w.N == 0) return hipSuccess;
  if (w.E > kMaxExpertsQmm) return hipErrorInvalidValue;
  // one expert's codes and scales are addressed with 32-bit byte offsets
  if (static_cast<uint64_t>(w.N) * w.wpr * 4 > 0xffffffffull) return hipErrorInvalidValue;
  const QmmLayout lay = qmm_layout(w, M, T);
  char* base = static_cast<char*>(ws);
  _Float16* xh = reinterpret_cast<_Float16*>(base + lay.rows);
  float* xs = reinterpret_cast<float*>(base + lay.scale);
  int32_t* count = reinterpret_cast<int32_t*>(base + lay.count);
  int4* tiles = reinterpret_cast<int4*>(base + lay.tiles);

  hipError_t err = launch_rot16(x, xdt, nullptr, T, /*zero_rows=*/1, w, x_rotated, xh, xs, nullptr, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, s, offsets, w.E, M, count, tiles);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  QmmParams p{};
  p.codes = w.codes; p.scales = w.scales; p.xh = xh; p.xs = xs; p.row_token = row_token;
  p.count = count; p.tiles = tiles; p.y = y;
  p.T = T; p.M = M;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.ydt = ydt;
  p.ngk = w.K / w.group;
  p.lg_group = __builtin_ctz(w.group);
  p.cb = *codebook_for(w.levels);
  // enough workgroups for any schedule: 8 XCDs x ceil(tiles / 8) row tiles x column tiles
  const int64_t nt = (w.N + kQmmBN - 1) / kQmmBN;
  const int64_t gx = 8 * ((max_tiles(M, w.E) + 7) / 8) * nt;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx));
  const bool g16 = w.group == 16;
  // Scales staged in LDS: always for trits (kept in registers, their five scales per span
  // and stage make the kernel spill, at half the speed); for the bit formats when a row's
  // groups fit one window (never with groups of 16, whose scales are per half fragment).
  const bool sl = !g16 && p.ngk <= qmm_lds_groups<16>();
  const dim3 blk(kQmmThreads);
  // with a second weight: a second matrix launch over the same rotated rows and tiles,
  // writing rows M .. 2M - 1
  for (int h = 0; h < (w2 ? 2 : 1); ++h) {
    if (h == 1) {
      p.codes = w2->codes;
      p.scales = w2->scales;
      p.y = static_cast<char*>(y) + M * w.N * (ydt == 0 ? 4 : 2);
    }
    switch (w.levels) {
      case 16:
        if (g16) hipLaunchKernelGGL((k_gqmm<16, true, false>), grid, blk, 0, s, p);
        else if (sl) hipLaunchKernelGGL((k_gqmm<16, false, true>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((k_gqmm<16, false, false>), grid, blk, 0, s, p);
        break;
      case 8:
        if (g16) hipLaunchKernelGGL((k_gqmm<8, true, false>), grid, blk, 0, s, p);
        else if (sl) hipLaunchKernelGGL((k_gqmm<8, false, true>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((k_gqmm<8, false, false>), grid, blk, 0, s, p);
        break;
      case 4:
        if (g16) hipLaunchKernelGGL((k_gqmm<4, true, false>), grid, blk, 0, s, p);
        else if (sl) hipLaunchKernelGGL((k_gqmm<4, false, true>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((k_gqmm<4, false, false>), grid, blk, 0, s, p);
        break;
      default:
        hipLaunchKernelGGL((k_gqmm<3, false, true>), grid, blk, 0, s, p);
        break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
