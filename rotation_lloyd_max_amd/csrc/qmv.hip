// qmv and gather_qmv: y = W R x with W decoded inline from packed codes.
//
// turboquant-mlx "How it works", "Running a quantized layer": the layer rotates its input
// and multiplies by the packed weights, decoding them inline, so full-precision weights
// never exist in memory: y_i = sum_g scale_{i,g} sum_{j in g} c[idx_ij] x'_j. The kernel
// table of that section has gather_qmv for one token, each routed expert reading the
// same (shared) input.
//
// Work split. One 16-wave workgroup per compute unit shares one input rotation. Grid row
// y = routed slot (its expert id is uniform in the workgroup); grid columns loop over
// groups of output rows. A wave owns NIT consecutive row steps of a group; a row is cut into chunks (32 elements, or one 20-trit word) and the lanes of a
// wave take fixed chunk positions, so every lane keeps the rotated input of its chunks in
// registers for all rows. Memory latency is hidden by issuing all code and scale loads of
// a group before using any of them, and, for the first group, before the input rotation.
//
// The input is rotated by every workgroup in LDS (fp32), scaled by a power of two so that
// its largest entry lies in [2^14, 2^15), and rounded to fp16 pairs. Codes are decoded
// through LDS tables into fp16 centroid pairs and multiplied with v_dot2 (fp32
// accumulate); each group's partial sum is multiplied by its fp16 scale.
#include "decode_common.hpp"
#include "internal.hpp"
#include "prologue.hpp"

namespace tq {

// Threads per workgroup: 16 waves (one workgroup per compute unit, sharing one input
// rotation) while a lane's rotated input fits the 128 registers that allows; 8 waves (two
// workgroups per compute unit, 256 registers) for rows of more than 128 chunks.
template <int CPL>
constexpr int qmv_threads() {
  return CPL <= 2 ? 1024 : 512;
}

struct QmvParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  const int32_t* ids;  // routed expert per slot, or nullptr for a dense layer
  const void* x;
  void* y;
  int K, N, E, wpr, group, m, P;
  int xdt, ydt, rotated;
  int Q;        // chunks per row
  int lpr_log;  // log2(lanes per row)
  float inv_sqrt_k;
  CodebookArgs cb;
};

// Row steps per wave and group. One step per group keeps up to four workgroups on a
// compute unit for small layers; large layers are streamed by the persistent loop with two
// groups in flight per wave.
template <int L, int CPL>
constexpr int qmv_nit() {
  return 1;
}

// The codes and scales of one group of rows, held in registers.
template <int L, int CPL, int NIT>
struct GroupRegs {
  uint32_t w[NIT][CPL][Fmt<L>::cw];
  uint32_t s[NIT][CPL];
};

template <int L, int CPL, int NIT, bool G16>
__device__ __forceinline__ void qmv_load_group(GroupRegs<L, CPL, NIT>& g, const QmvParams& p,
                                               int grp, int rows_per_group, int wave, int rpw,
                                               int sub, int c0, int lpr, int64_t ebase,
                                               int ngroups) {
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    int n = grp * rows_per_group + (wave * NIT + it) * rpw + sub;
    n = n < p.N ? n : p.N - 1;
    const uint32_t* crow = p.codes + (ebase + n) * p.wpr;
    const uint16_t* srow = p.scales + (ebase + n) * ngroups;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int c = c0 + j * lpr;
      c = c < p.Q ? c : p.Q - 1;
      load_chunk_words<L>(crow, c, g.w[it][j]);
      g.s[it][j] = load_chunk_scales<L, G16>(srow, c, p.group, ngroups);
    }
  }
}

template <int L, int CPL, int NIT, bool G16>
__device__ __forceinline__ void qmv_compute_group(const GroupRegs<L, CPL, NIT>& g, const QmvParams& p,
                                                  int grp, int rows_per_group, int wave, int rpw,
                                                  int sub, int c0, int lpr, int lane31,
                                                  const uint32_t* lut,
                                                  const uint32_t (&xr)[CPL][Fmt<L>::np],
                                                  float out_scale, bool bad, int slot) {
  using F = Fmt<L>;
  constexpr bool TWO = (L == 3) || G16;  // a chunk may span two groups
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int n = grp * rows_per_group + (wave * NIT + it) * rpw + sub;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + j * lpr;
      int pb = F::np;
      if constexpr (L == 3) {
        const int e0 = c * F::ce;
        const int bound = ((e0 / p.group) + 1) * p.group - e0;
        pb = bound >= F::ce ? F::np : bound / 2;
      } else if constexpr (G16) {
        pb = F::np / 2;
      }
      float a0 = 0.f, a1 = 0.f;
      chunk_dot_regs<L>(g.w[it][j], lut, lane31, xr[j], pb, a0, a1);
      float v = a0 * half_bits_to_float(static_cast<uint16_t>(g.s[it][j] & 0xffff));
      if constexpr (TWO) v += a1 * half_bits_to_float(static_cast<uint16_t>(g.s[it][j] >> 16));
      acc += c < p.Q ? v : 0.f;
    }
    acc = segment_sum(acc, p.lpr_log);
    if (seg_sum_lane(c0, p.lpr_log) && n < p.N)
      store_any(p.y, p.ydt, static_cast<int64_t>(slot) * p.N + n,
                bad ? __builtin_nanf("") : acc * out_scale);
  }
}

template <int L, int CPL, bool G16, bool X32>
__global__ __launch_bounds__(qmv_threads<CPL>()) void k_qmv(QmvParams p) {
  using F = Fmt<L>;
  constexpr int NIT = qmv_nit<L, CPL>();
  constexpr int kQmvThreads = qmv_threads<CPL>();
  constexpr int kQmvWaves = kQmvThreads / 64;
  extern __shared__ uint32_t smem_u[];
  uint32_t* lut = smem_u;
  float* xf = reinterpret_cast<float*>(lut + F::entries * kLutCopies);  // padded row
  double* red = reinterpret_cast<double*>(xf + ((padded_len(p.K) + 1) & ~1));
  uint16_t* hs = reinterpret_cast<uint16_t*>(red + kQmvWaves);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lane31 = lane & 31;
  const int lpr = 1 << p.lpr_log;
  const int sub = lane >> p.lpr_log, c0 = lane & (lpr - 1);
  const int rpw = 64 >> p.lpr_log;
  const int rows_per_group = kQmvWaves * NIT * rpw;
  const int ngroups_rows = (p.N + rows_per_group - 1) / rows_per_group;
  const int ngroups = p.K / p.group;
  const int slot = blockIdx.y;

  // Loads, all unconditional and in this order: input row and sign words, centroids,
  // expert id, then the first group's codes and scales. The rotation below waits only for
  // the first ones while the codes stream in.
  InputLoad<X32, kQmvThreads> xin;
  xin.issue(p.x, p.xdt, 0, p.K, p.signs);
  // without ids, a harmless word of the sign array is read and ignored (no branch); the
  // address is uniform, so this is a scalar load that no vector load has to wait for
  const int eraw = *(p.ids ? p.ids + slot : reinterpret_cast<const int32_t*>(p.signs));
  const int e = p.ids ? eraw : 0;
  const bool bad = e < 0 || e >= p.E;
  const int64_t ebase = static_cast<int64_t>(bad ? 0 : e) * p.N;

  int grp = blockIdx.x;
  GroupRegs<L, CPL, NIT> ga, gb;
  qmv_load_group<L, CPL, NIT, G16>(ga, p, grp, rows_per_group, wave, rpw, sub, c0, lpr, ebase,
                                   ngroups);

  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) hs[k] = p.cb.h[k];  // uniform (scalar) loads
  }
  __syncthreads();
  build_lut<L, kQmvThreads>(lut, hs);
  float out_scale;
  const float sc = xin.finish(xf, red, p.K, p.m, p.P, p.rotated != 0, p.inv_sqrt_k, &out_scale);
  uint32_t xr[CPL][F::np];
  lane_pairs<L, CPL>(xf, p.K, p.Q, c0, lpr, sc, xr);

  // Two register sets: the next group's loads are in flight while a group is computed.
  // Past its last group a workgroup re-reads its current group (cached lines it just
  // read, different for every workgroup), which keeps the loads unconditional.
  const int stride = gridDim.x;
  while (true) {
    const int gb_idx = grp + stride;
    qmv_load_group<L, CPL, NIT, G16>(gb, p, gb_idx < ngroups_rows ? gb_idx : grp,
                                     rows_per_group, wave, rpw, sub, c0, lpr, ebase, ngroups);
    qmv_compute_group<L, CPL, NIT, G16>(ga, p, grp, rows_per_group, wave, rpw, sub, c0, lpr,
                                        lane31, lut, xr, out_scale, bad, slot);
    if (gb_idx >= ngroups_rows) break;
    grp = gb_idx;
    const int ga_idx = grp + stride;
    qmv_load_group<L, CPL, NIT, G16>(ga, p, ga_idx < ngroups_rows ? ga_idx : grp,
                                     rows_per_group, wave, rpw, sub, c0, lpr, ebase, ngroups);
    qmv_compute_group<L, CPL, NIT, G16>(gb, p, grp, rows_per_group, wave, rpw, sub, c0, lpr,
                                        lane31, lut, xr, out_scale, bad, slot);
    if (ga_idx >= ngroups_rows) break;
    grp = ga_idx;
  }
}

static int pow2_ceil_log(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

template <int L>
static hipError_t launch_qmv_l(QmvParams& p, int n_slots, hipStream_t s) {
  using F = Fmt<L>;
  p.Q = (p.wpr + F::cw - 1) / F::cw;
  int lpr_log = pow2_ceil_log(p.Q);
  if (lpr_log > 6) lpr_log = 6;
  p.lpr_log = lpr_log;
  const int lpr = 1 << lpr_log;
  const int cpl_need = (p.Q + lpr - 1) / lpr;
  const bool g16 = (L != 3) && p.group == 16;
  const bool x32 = p.xdt == 0;
  const int rpw = 64 / lpr;
  void (*kern)(QmvParams) = nullptr;
  int nit = 1, threads = 1024;
#define TQ_PICK(C)                                                                   \
  do {                                                                               \
    threads = qmv_threads<C>();                                                      \
    if constexpr (L == 3) kern = x32 ? k_qmv<L, C, false, true> : k_qmv<L, C, false, false>; \
    else kern = g16 ? (x32 ? k_qmv<L, C, true, true> : k_qmv<L, C, true, false>)    \
                    : (x32 ? k_qmv<L, C, false, true> : k_qmv<L, C, false, false>); \
    nit = qmv_nit<L, C>();                                                           \
  } while (0)
  if (cpl_need <= 1) TQ_PICK(1);
  else if (cpl_need <= 2) TQ_PICK(2);
  else if (cpl_need <= 4) TQ_PICK(4);
  else TQ_PICK(8);
#undef TQ_PICK
  const int waves = threads / 64;
  const int rows_per_group = waves * nit * rpw;
  const int groups = (p.N + rows_per_group - 1) / rows_per_group;
  // 16 waves per compute unit in total; each workgroup loops over its row groups
  const int total_wgs = 256 * (1024 / threads);
  int per_slot = (total_wgs + n_slots - 1) / n_slots;
  if (per_slot > groups) per_slot = groups;
  if (per_slot < 1) per_slot = 1;
  const size_t lds = F::entries * kLutCopies * 4 + ((padded_len(p.K) + 1) & ~1) * 4 +
                     waves * 8 + 64;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(per_slot, n_slots), dim3(threads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_qmv(const WeightArgs& w, const int32_t* ids, int n, const void* x, int xdt,
                      bool x_rotated, void* y, int ydt, hipStream_t s) {
  if (n == 0 || w.N == 0) return hipSuccess;
  QmvParams p{};
  p.codes = w.codes; p.scales = w.scales; p.signs = w.signs; p.ids = ids;
  p.x = x; p.y = y;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group; p.m = w.m; p.P = w.P;
  p.xdt = xdt; p.ydt = ydt; p.rotated = x_rotated ? 1 : 0;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  p.cb = *codebook_for(w.levels);
  switch (w.levels) {
    case 16: return launch_qmv_l<16>(p, n, s);
    case 8: return launch_qmv_l<8>(p, n, s);
    case 4: return launch_qmv_l<4>(p, n, s);
    default: return launch_qmv_l<3>(p, n, s);
  }
}

}  // namespace tq
