// k_qmv: the qmv / gather_qmv kernel template and its launcher (one instantiation per
// code format, each in its own translation unit qmv_<levels>.hip).
//
// turboquant-mlx "How it works", "Running a quantized layer": the layer rotates its input
// and multiplies by the packed weights, decoding them inline, so full-precision weights
// never exist in memory: y_i = sum_g scale_{i,g} sum_{j in g} c[idx_ij] x'_j. The kernel
// table of that section has gather_qmv for one token, each routed expert reading the
// same (shared) input.
//
// Work split. One 16-wave workgroup per compute unit rotates the input once in LDS and
// then streams rows. A row is cut into chunks (32 elements, or one 20-trit word); the
// chunks of a row are split into KS contiguous K-slices, each taken by one wave of a
// "row set" of KS waves, and the lanes of a wave take fixed chunk positions of their
// slice (at most two per lane), so every lane keeps the rotated input of its chunks in
// registers for all rows. Grid row y = routed slot (its expert id is uniform in the
// workgroup), grid layer z = the weight (two for gate and up in one launch); grid columns
// loop over groups of rows, keeping D groups of code and scale loads in flight per wave (a
// ring of register sets), the first D - 1 of them issued before the input rotation.
//
// Codes are decoded through LDS tables into fp16 centroid pairs (qmv_decode.hpp) and
// multiplied with v_dot2 (fp32 accumulate); each group's partial sum is multiplied by its
// fp16 scale; lanes of a slice are summed with DPP moves. The slice sums of every row go
// to LDS and are added in slice order and stored after the loop: no store is mixed into
// the stream of loads (which would make the wait for a group's loads wait for all of
// them), and results do not depend on timing.
#pragma once

#include "internal.hpp"
#include "prologue.hpp"
#include "qmv_decode.hpp"
#include "rot_mfma.hpp"

namespace tq {

constexpr int kQmvThreads = 1024;
constexpr int kQmvWaves = kQmvThreads / 64;
constexpr int kMaxRowPartBytes = 32768;
// Row groups whose loads are issued before the input rotation (the rest of the ring after
// it). Fewer (2, which also removes the 8 registers the 2-bit gate kernel spills) measured
// slower on the MoE decode layer: the loads in flight during the rotation matter more.
constexpr int kQmvPreGroups = 3;

struct QmvParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  const int32_t* ids;  // routed expert per slot, or nullptr for a dense layer
  const void* x;
  void* y;
  int K, N, E, wpr, group, m, P;
  int xdt, ydt, rotated;
  int Q;          // chunks per row
  int Qh;         // chunks per K-slice
  int ks_log;     // log2(KS), K-slices (waves) per row
  int lpr_log;    // log2(lanes per row within a slice)
  int lk;         // ceil(log2(K))
  int ngroups;    // row groups per slot
  int max_iters;  // row groups per workgroup at most (sizes the slice-sum buffer)
  int mrot;       // rotate on the matrix cores (K = 4096, 16-bit input, bit formats)
  float inv_sqrt_k;
  CodebookArgs cb;
  // the second weight of a two-weight launch (grid.z = 2; same format, shape and experts):
  // a MoE layer's gate and up projections, read by the workgroups with blockIdx.z = 1
  const uint32_t* codes2;
  const uint16_t* scales2;
};

// fp32 words of the kernel's row buffer: the padded row, or (rotation on the matrix cores)
// the two bf16 terms of the transposed intermediate if they are larger.
__host__ __device__ inline int qmv_xf_words(int K, int mrot) {
  const int w = padded_len(K);
  return mrot && w < 2 * kZtBytes / 4 ? 2 * kZtBytes / 4 : w;
}

// The codes and scales of one group of rows for one lane.
template <int L, int CPL>
struct GroupRegs {
  uint32_t w[CPL][Fmt<L>::cw];
  half2_t s[CPL];
};

// Per-lane constants of the work split.
struct Lane {
  int ks;       // K-slice of this wave
  int rset;     // row set of this wave
  int sub;      // row within the wave's rows
  int c0;       // first chunk position within the slice
  int lpr;      // lanes per row
  int rpw;      // rows per wave
  int rows_per_group;
  int slice_q;  // chunks in this wave's slice
};

template <int L, int CPL, bool G16>
__device__ __forceinline__ void qmv_load_group(GroupRegs<L, CPL>& g, const QmvParams& p,
                                               const Lane& ln, int grp, const uint32_t* cexp,
                                               const uint16_t* sexp, int ngroups_k) {
  int n = grp * ln.rows_per_group + ln.rset * ln.rpw + ln.sub;
  n = n < p.N ? n : p.N - 1;
  // byte offsets inside the expert (its codes are below 4 GB, checked on the host)
  const uint32_t cbyte = __umul24(static_cast<uint32_t>(n), static_cast<uint32_t>(p.wpr)) * 4u;
  const uint32_t sbyte = __umul24(static_cast<uint32_t>(n), static_cast<uint32_t>(ngroups_k)) * 2u;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int c = ln.c0 + j * ln.lpr;
    c = c < ln.slice_q ? c : ln.slice_q - 1;
    c += ln.ks * p.Qh;
    load_chunk_words<L>(cexp, cbyte, c, g.w[j]);
    g.s[j] = load_chunk_scales<L, G16>(sexp, sbyte, c, p.group, ngroups_k);
  }
}

// Decode one group of rows; returns the sum of the lane's row over its slice (valid in
// the last lane of each row segment).
template <int L, int CPL, bool G16>
__device__ __forceinline__ float qmv_group_sum(const GroupRegs<L, CPL>& g, const QmvParams& p,
                                               const Lane& ln, uint32_t lslot, const uint32_t* lut,
                                               const uint32_t (&xr)[CPL][Fmt<L>::np]) {
  using F = Fmt<L>;
  constexpr bool TWO = (L == 3) || G16;  // a chunk may span two groups
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int cr = ln.c0 + j * ln.lpr;
    const int c = ln.ks * p.Qh + cr;
    int pb = F::np;
    if constexpr (L == 3) {
      const int e0 = c * F::ce;
      const int bound = ((e0 / p.group) + 1) * p.group - e0;
      pb = bound >= F::ce ? F::np : bound / 2;
    }
    float a0 = 0.f, a1 = 0.f;
    chunk_dot_v<L, G16>(g.w[j], lut, lslot, xr[j], pb, a0, a1);
    float v = a0 * static_cast<float>(g.s[j].x);
    if constexpr (TWO) v += a1 * static_cast<float>(g.s[j].y);
    acc += cr < ln.slice_q ? v : 0.f;
  }
  return p.lpr_log == 6 ? wave_sum_to_last(acc) : segment_sum_flat(acc, p.lpr_log);
}

// The same sum as qmv_group_sum from table entries looked up beforehand.
template <int L, int CPL, bool G16>
__device__ __forceinline__ float qmv_group_dot(const GroupRegs<L, CPL>& g, const QmvParams& p,
                                               const Lane& ln,
                                               const uint32_t (&cw)[CPL][Fmt<L>::np],
                                               const uint32_t (&xr)[CPL][Fmt<L>::np]) {
  using F = Fmt<L>;
  constexpr bool TWO = (L == 3) || G16;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int cr = ln.c0 + j * ln.lpr;
    const int c = ln.ks * p.Qh + cr;
    int pb = F::np;
    if constexpr (L == 3) {
      const int e0 = c * F::ce;
      const int bound = ((e0 / p.group) + 1) * p.group - e0;
      pb = bound >= F::ce ? F::np : bound / 2;
    }
    float a0 = 0.f, a1 = 0.f;
    chunk_dot_pairs<L, G16>(cw[j], xr[j], pb, a0, a1);
    float v = a0 * static_cast<float>(g.s[j].x);
    if constexpr (TWO) v += a1 * static_cast<float>(g.s[j].y);
    acc += cr < ln.slice_q ? v : 0.f;
  }
  return p.lpr_log == 6 ? wave_sum_to_last(acc) : segment_sum_flat(acc, p.lpr_log);
}

// The input row of a qmv workgroup: its loads (issued first) and its rotation into the fp16
// chunk layout xh, by the butterflies of prologue.hpp or, for K = 4096 and a 16-bit input,
// on the matrix cores (rot_mfma.hpp). The centroid table is built on the way: it is
// complete when rotate() returns.
template <int L, bool X32>
struct QmvInput {
  static constexpr bool HALF = L != 3;  // bit formats: the rotation writes xh directly
  InputLoad<X32, kQmvThreads> xin;
  Rot4096Mfma<kQmvThreads> mr;
  bool mrot;

  // three loads per lane at most
  __device__ __forceinline__ void issue(const QmvParams& p) {
    mrot = false;
    if constexpr (!X32 && HALF) mrot = p.mrot != 0;
    if (mrot) mr.issue(p.x, p.signs);
    else xin.issue(p.x, p.xdt, 0, p.K, p.rotated ? nullptr : p.signs);
  }

  // Returns sc (x' in xh is sc times the rotated input, rounded to fp16); *out_scale gets
  // 1 / (sc sqrt(K)) (1 / sc for a rotated input). Ends synchronized.
  __device__ __forceinline__ float rotate(const QmvParams& p, uint32_t* lut, uint32_t* xh,
                                         float* xf, float* red, uint16_t* hs, float* out_scale) {
    // the centroids reach LDS through the first barrier of the rotation
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) hs[k] = p.cb.h[k];  // uniform (scalar) loads
    }
    if (mrot) {
      // the table is built after the first barrier (the centroids reach LDS through it)
      auto side = [&](int, int) {};
      auto between = [&] { build_lut_v<L, kQmvThreads>(lut, hs); };
      char* zt = reinterpret_cast<char*>(xf);
      _Float16* xhh = reinterpret_cast<_Float16*>(xh);
      return p.xdt == 1 ? mr.template rotate<true>(zt, red, p.lk, p.inv_sqrt_k, xhh, out_scale,
                                                   side, between)
                        : mr.template rotate<false>(zt, red, p.lk, p.inv_sqrt_k, xhh, out_scale,
                                                    side, between);
    }
    const bool rotated = p.rotated != 0;
    const float sc = xin.template finish_a<HALF>(xf, red, p.K, p.lk, p.P, rotated,
                                                 p.inv_sqrt_k, out_scale);
    build_lut_v<L, kQmvThreads>(lut, hs);
    xin.template finish_b<HALF>(xf, xh, p.K, p.m, p.P, rotated, sc);
    if constexpr (!HALF) pairs_to_lds<L, kQmvThreads>(xf, xh, p.K, p.Q, sc);
    return sc;
  }
};

template <int L, int CPL, bool G16, bool X32, int D>
__global__ __launch_bounds__(kQmvThreads) void k_qmv(QmvParams p) {
  using F = Fmt<L>;
  // The table is the kernel's only static LDS array, so it starts at address 0 and every
  // lookup address (index << 8 | slot) is used as is.
  __shared__ __attribute__((aligned(16))) uint32_t lut[lut_bytes<L>() / 4];
  extern __shared__ uint32_t smem_u[];
  uint32_t* xh = smem_u;                                   // fp16 pairs of x', by chunk
  float* xf = reinterpret_cast<float*>(xh + p.Q * pair_stride<L>());  // padded fp32 row
  float* red = xf + qmv_xf_words(p.K, p.mrot);             // one float per wave
  uint16_t* hs = reinterpret_cast<uint16_t*>(red + kQmvWaves);  // 16 fp16 centroids
  float* rowpart = red + kQmvWaves + 8;                    // slice sums of the rows

  // the wave index is uniform: held in a scalar register, so are the per-wave constants
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const uint32_t lslot = lut_slot<L>(lane);  // this lane's copy inside every table entry
  const int KS = 1 << p.ks_log;
  Lane ln;
  ln.ks = wave & (KS - 1);
  ln.rset = wave >> p.ks_log;
  ln.lpr = 1 << p.lpr_log;
  ln.rpw = 64 >> p.lpr_log;
  ln.sub = lane >> p.lpr_log;
  ln.c0 = lane & (ln.lpr - 1);
  ln.rows_per_group = (kQmvWaves >> p.ks_log) * ln.rpw;
  {
    const int rest = p.Q - ln.ks * p.Qh;
    ln.slice_q = rest < p.Qh ? rest : p.Qh;
  }
  const int ngroups_k = p.K / p.group;
  const int slot = blockIdx.y;
  // the second weight (its outputs follow the first's); two-weight launches use the ring
  // kernels (D > 1), so the one-group kernel keeps its first loads free of the choice
  const bool second = D > 1 && blockIdx.z != 0;
  const int64_t orow = D > 1 ? static_cast<int64_t>(blockIdx.z) * gridDim.y + slot : slot;
  const bool last_lane = seg_sum_lane(ln.c0, p.lpr_log);

  // Loads, in this order: input row and sign words, expert id (a dense layer reads none),
  // then the first D - 1 groups' codes and scales. The rotation below waits only for the
  // first ones while the codes stream in.
  QmvInput<L, X32> in;
  in.issue(p);
  int e = 0;
  if (p.ids) e = p.ids[slot];
  const bool bad = e < 0 || e >= p.E;
  const int64_t ebase = static_cast<int64_t>(bad ? 0 : e) * p.N;
  const uint32_t* cexp = (second ? p.codes2 : p.codes) + ebase * p.wpr;
  const uint16_t* sexp = (second ? p.scales2 : p.scales) + ebase * ngroups_k;

  const int grp0 = blockIdx.x, stride = gridDim.x;
  GroupRegs<L, CPL> buf[D];
  // D == 1: the launch gives every workgroup exactly one row group (grp0 < ngroups)
  if constexpr (D == 1) qmv_load_group<L, CPL, G16>(buf[0], p, ln, grp0, cexp, sexp, ngroups_k);
  // PRE of the D - 1 groups ahead are requested before the rotation, the rest after it
  constexpr int PRE = D - 1 > kQmvPreGroups ? kQmvPreGroups : D - 1;
#pragma unroll
  for (int d = 0; d < PRE; ++d) {
    const int g = grp0 + d * stride;
    qmv_load_group<L, CPL, G16>(buf[d], p, ln, g < p.ngroups ? g : grp0, cexp, sexp, ngroups_k);
  }

  float out_scale;
  in.rotate(p, lut, xh, xf, red, hs, &out_scale);
#pragma unroll
  for (int d = PRE; d < D - 1; ++d) {
    const int g = grp0 + d * stride;
    qmv_load_group<L, CPL, G16>(buf[d], p, ln, g < p.ngroups ? g : grp0, cexp, sexp, ngroups_k);
  }
  const float nan = __builtin_nanf("");
  const int rloc = ln.rset * ln.rpw + ln.sub;
  int grp = grp0, it = 0;
  uint32_t xr[CPL][F::np];
  lane_pairs<L, CPL>(xh, ln.ks * p.Qh, ln.c0, ln.lpr, ln.slice_q, xr);
  if constexpr (D == 1) {
    // One row group per workgroup, its loads issued before the rotation.
    uint32_t cw[CPL][F::np];
#pragma unroll
    for (int j = 0; j < CPL; ++j) chunk_lookup<L>(buf[0].w[j], lut, lslot, cw[j]);
    const float v = qmv_group_dot<L, CPL, G16>(buf[0], p, ln, cw, xr);
    if (KS == 1) {
      // a whole row per lane segment and no loads left: its last lane stores the result
      const int n = grp0 * ln.rows_per_group + rloc;
      if (last_lane && n < p.N)
        store_any(p.y, p.ydt, orow * p.N + n, bad ? nan : v * out_scale);
      return;
    }
    if (last_lane) rowpart[rloc * KS + ln.ks] = v;
    it = 1;
  } else {
    // The loop body is unrolled over U groups (a multiple of D, so the ring positions
    // repeat): inside straight-line code the compiler waits for exactly the one group it
    // computes; only the rare back edge (workgroups with more than U groups) waits longer.
    constexpr int U = D >= 4 ? 8 : 4;
    while (true) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // refill the set computed last with the group D - 1 strides ahead (past the end:
        // this group again, lines just read, so the loads stay unconditional)
        const int gl = grp + (D - 1) * stride;
        qmv_load_group<L, CPL, G16>(buf[(u + D - 1) % D], p, ln, gl < p.ngroups ? gl : grp,
                                    cexp, sexp, ngroups_k);
        const float v = qmv_group_sum<L, CPL, G16>(buf[u % D], p, ln, lslot, lut, xr);
        if (last_lane) rowpart[(it * ln.rows_per_group + rloc) * KS + ln.ks] = v;
        ++it;
        grp += stride;
        if (grp >= p.ngroups) goto done;
      }
    }
  }
done:
  // add the slice sums of every row in slice order and store the rows
  __syncthreads();
  const int rows = it * ln.rows_per_group;
  for (int i = threadIdx.x; i < rows; i += kQmvThreads) {
    const int itr = i / ln.rows_per_group, r = i - itr * ln.rows_per_group;
    const int n = (grp0 + itr * stride) * ln.rows_per_group + r;
    float v = 0.f;
    for (int k = 0; k < KS; ++k) v += rowpart[i * KS + k];
    if (n < p.N)
      store_any(p.y, p.ydt, orow * p.N + n, bad ? nan : v * out_scale);
  }
}

inline int pow2_ceil_log(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Registers per row group and lane: the code words and the scale of each chunk.
template <int L, int CPL>
constexpr int group_regs() {
  return CPL * (Fmt<L>::cw + 1);
}
// The deepest ring. Eight groups in flight (most of a workgroup's rows requested before the
// input rotation) measured slower than four on every layer shape tried, so four it is.
template <int L, int CPL>
constexpr int max_depth() {
  return 4;
}

template <int L, int CPL, bool G16, bool X32>
static const void* pick_depth(int depth) {
  // 4-bit rows of one chunk per lane (K <= 2048; the MoE down projection, 14 row groups per
  // workgroup): a ring of two measured faster than four there (15.3-15.7 against
  // 15.7-16.1 us per call), one of eight slower; the other kernels keep four
  if constexpr (L == 16 && CPL == 1) {
    if (depth >= 2) return reinterpret_cast<const void*>(k_qmv<L, CPL, G16, X32, 2>);
  }
  if constexpr (max_depth<L, CPL>() >= 8) {
    if (depth >= 8) return reinterpret_cast<const void*>(k_qmv<L, CPL, G16, X32, 8>);
  }
  return depth >= 4 ? reinterpret_cast<const void*>(k_qmv<L, CPL, G16, X32, 4>)
         : depth >= 2 ? reinterpret_cast<const void*>(k_qmv<L, CPL, G16, X32, 2>)
                      : reinterpret_cast<const void*>(k_qmv<L, CPL, G16, X32, 1>);
}

template <int L, int CPL>
static const void* pick_kernel(bool g16, bool x32, int depth) {
  if constexpr (L == 3) {
    return x32 ? pick_depth<L, CPL, false, true>(depth) : pick_depth<L, CPL, false, false>(depth);
  } else {
    if (g16) return x32 ? pick_depth<L, CPL, true, true>(depth) : pick_depth<L, CPL, true, false>(depth);
    return x32 ? pick_depth<L, CPL, false, true>(depth) : pick_depth<L, CPL, false, false>(depth);
  }
}

template <int L>
hipError_t launch_qmv_l(QmvParams& p, int n_slots, int n_weights, hipStream_t s) {
  using F = Fmt<L>;
  p.Q = (p.wpr + F::cw - 1) / F::cw;
  p.lk = pow2_ceil_log(p.K);
  p.mrot = (L != 3 && p.K == 4096 && p.m == 1 && p.xdt != 0 && !p.rotated) ? 1 : 0;
  // K-slices: at most two chunks of each row per lane
  int ks_log = 0;
  while (((p.Q + (1 << ks_log) - 1) >> ks_log) > 128) ++ks_log;
  p.ks_log = ks_log;
  p.Qh = (p.Q + (1 << ks_log) - 1) >> ks_log;
  int lpr_log = pow2_ceil_log(p.Qh);
  if (lpr_log > 6) lpr_log = 6;
  p.lpr_log = lpr_log;
  const int cpl = (p.Qh + (1 << lpr_log) - 1) >> lpr_log;  // 1 or 2
  const int rows_per_group = (kQmvWaves >> ks_log) * (64 >> lpr_log);
  p.ngroups = (p.N + rows_per_group - 1) / rows_per_group;

  // one workgroup per compute unit in total, each looping over its row groups
  const int jobs = n_slots * n_weights;
  int per_slot = (256 + jobs - 1) / jobs;
  if (per_slot > p.ngroups) per_slot = p.ngroups;
  if (per_slot < 1) per_slot = 1;
  int iters = (p.ngroups + per_slot - 1) / per_slot;
  {
    // the slice sums of a workgroup's rows must fit their LDS buffer
    const int per_iter = rows_per_group * (1 << ks_log) * 4;
    const int max_iters = kMaxRowPartBytes / per_iter;
    if (iters > max_iters) {
      per_slot = (p.ngroups + max_iters - 1) / max_iters;
      iters = (p.ngroups + per_slot - 1) / per_slot;
    }
  }
  p.max_iters = iters;
  // one group per workgroup: no ring (depth 1, lookups overlap the rotation); a two-weight
  // launch always takes a ring kernel
  const int depth = iters <= 1 && n_weights == 1 ? 1 : iters <= 2 ? 2 : iters <= 4 ? 4 : 8;
  const bool g16 = (L != 3) && p.group == 16;
  const bool x32 = p.xdt == 0;
  const void* kern = cpl <= 1 ? pick_kernel<L, 1>(g16, x32, depth)
                              : pick_kernel<L, 2>(g16, x32, depth);

  const size_t rowpart = static_cast<size_t>(iters) * rows_per_group * (1 << ks_log) * 4;
  // dynamic LDS (the table is static)
  const size_t lds = static_cast<size_t>(p.Q) * pair_stride<L>() * 4 + qmv_xf_words(p.K, p.mrot) * 4 +
                     (kQmvWaves + 8) * 4 + rowpart;
  if (lds + lut_bytes<L>() > 65536) {
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(reinterpret_cast<void (*)(QmvParams)>(const_cast<void*>(kern)),
                     dim3(per_slot, n_slots, n_weights), dim3(kQmvThreads), lds, s, p);
  return hipGetLastError();
}

}  // namespace tq
