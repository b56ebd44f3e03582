// multi_gather_qmv: y[p] = W_{ids[p]} R x[p] for P (input, expert) pairs.
//
// turboquant-mlx "How it works", "Running a quantized layer", kernel table, second row:
// prefill with a different input per expert. Two launches:
//   k_rot16    every input rotated once into fp16 rows (rot16.hpp), plus one zero row; one
//              more workgroup of the same launch sorts the pairs by expert into the
//              workspace (bucket.hpp: offsets, order); pairs with an expert id outside
//              [0, E) get a row of NaN
//   k_mg       one workgroup per (expert, block of 128 output rows): each wave decodes the
//              codes of 16 rows straight into matrix-core operands (mfma_decode.hpp) and
//              multiplies them by the rotated inputs of up to 16 of the expert's pairs at a
//              time with v_mfma_f32_16x16x32_f16, so every code word is read from memory
//              and decoded once per 16 pairs, whatever the number of pairs.
#include <mutex>

#include "internal.hpp"
#include "mfma_decode.hpp"
#include "rot16.hpp"

namespace tq {

constexpr int kMaxExperts = 8192;
// 8 waves (128 rows) per workgroup and at most 128 VGPRs per lane (4 waves per SIMD), so
// that two trit workgroups (70 KB of LDS each) share a CU, each with a whole 128-row K-chunk
// of loads in flight.
constexpr int kMgWaves = 8;
constexpr int kMgThreads = 64 * kMgWaves;

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Workspace: offsets [E+1] int32 | order [P] int32 | scale [P+1] float |
// rotated rows [P+1][rot16_row_halves(K)] fp16 (row P all zero); 256-byte aligned sections.
struct MgLayout {
  size_t offsets, order, scale, rows, total;
};
static MgLayout mg_layout(const WeightArgs& w, int64_t P) {
  MgLayout l{};
  l.offsets = 0;
  l.order = align256(static_cast<size_t>(w.E + 1) * 4);
  l.scale = l.order + align256(static_cast<size_t>(P) * 4);
  l.rows = l.scale + align256(static_cast<size_t>(P + 1) * 4);
  l.total = l.rows + align256(static_cast<size_t>(P + 1) * rot16_row_halves(w.K) * 2);
  return l;
}

size_t multi_gather_workspace(const WeightArgs& w, int64_t P) { return mg_layout(w, P).total; }

struct MgParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const int32_t* offsets;
  const int32_t* order;
  const _Float16* xh;  // rotated rows
  const float* xs;     // their scales
  void* y;
  int64_t rowh;        // halves per rotated row
  int64_t zero_row;    // index of the all-zero row
  int K, N, E, wpr, lg_group, ngk, ydt;
  CodebookArgs cb;
};

// k_mg works through K in chunks of 4 super-blocks (4 spans of 4 lane groups each: 512
// elements for the bit formats, 640 for trits). A chunk's code words and scales of the
// workgroup's 64 rows, and the rotated inputs of its pairs, are first copied to LDS with
// loads in which consecutive lanes read consecutive words of a row (each cache line is
// touched once per chunk); the next chunk's loads are held in registers meanwhile. The
// matrix-core operands are then read from LDS, where each lane's span is contiguous.
template <int L>
struct MgChunk {
  static constexpr int SB = 4 * Span<L>::elems;  // elements per super-block
  static constexpr int KC = 4 * SB;              // elements per chunk
  static constexpr int WPC = L == 3 ? KC / 20 : KC * (L == 16 ? 4 : L == 8 ? 3 : 2) / 32;
  static constexpr int CST = WPC + 4;            // LDS words per row of codes
  static constexpr int AST = KC + 8;             // LDS halves per row of inputs
  static constexpr int ROWS = 16 * kMgWaves;     // weight rows per workgroup
  static constexpr int CW = ROWS * WPC / kMgThreads;        // code words per thread
  static constexpr int AU = (16 * (KC / 8) + kMgThreads - 1) / kMgThreads;  // 16-byte input units per thread (units past 16 rows are never pairs)
};

constexpr int kMaxScalesPerChunk = 640 / 16;  // groups of a chunk at most (trits, g16)

template <int L>
struct MgStage {
  uint32_t c[MgChunk<L>::CW];
  uint32_t s[(MgChunk<L>::ROWS * kMaxScalesPerChunk + kMgThreads - 1) / kMgThreads];
  u32x4_t a[MgChunk<L>::AU];
};

struct MgTile {
  int row0;    // first weight row of the workgroup
  int cnt;     // pairs of this tile (<= 16)
  int spc;     // scale groups per chunk (KC / group, at least 1)
  uint32_t spc_inv;  // ceil(2^32 / spc): i / spc = umulhi(i, spc_inv) for i < 2^16
  int sst;     // LDS halves per row of scales
  bool full;   // every row of the workgroup exists (row0 + ROWS <= N)
  bool s32;    // scales staged as 4-byte pairs (K / group and spc even: 4-byte aligned)
  const uint32_t* cexp;   // the expert's codes
  const uint16_t* sexp;   // the expert's scales
  const int32_t* pairs;   // the tile's pair indices
  // the row of staging index i (i / spc; i < 2^16)
  __device__ __forceinline__ int row_of(int i) const {
    return spc_inv ? static_cast<int>(__umulhi(static_cast<uint32_t>(i), spc_inv)) : i;
  }
};

// A thread's input units for the tile: byte offset of unit j's 16 bytes at K position 0
// (chunk c adds 2 KC c), or kNoUnit for a unit that belongs to no pair of the tile.
constexpr uint32_t kNoUnit = 0xffffffffu;
template <int L>
struct MgInputs {
  uint32_t off[MgChunk<L>::AU];
  __device__ __forceinline__ bool on(int j) const { return off[j] != kNoUnit; }
};

template <int L>
__device__ __forceinline__ void mg_inputs(MgInputs<L>& in, const MgParams& p, const MgTile& t) {
  using C = MgChunk<L>;
  int tid = static_cast<int>(threadIdx.x);
  __asm__ volatile("" : "+v"(tid));
#pragma unroll
  for (int j = 0; j < C::AU; ++j) {
    const int i = tid + j * kMgThreads;
    const int m = i / (C::KC / 8), u = i - m * (C::KC / 8);
    in.off[j] = m < t.cnt
                    ? (static_cast<uint32_t>(t.pairs[m]) * static_cast<uint32_t>(p.rowh) + 8u * u) * 2u
                    : kNoUnit;
  }
}

// Global -> registers for chunk c. Where the workgroup's rows all exist, consecutive load
// steps move by whole rows, so their row offsets are uniform (scalar) and each load costs
// no vector arithmetic; otherwise rows are clamped per lane.
template <int L>
__device__ __forceinline__ void mg_fetch(MgStage<L>& st, const MgParams& p, const MgTile& t, int c) {
  using C = MgChunk<L>;
  MgInputs<L> in;
  mg_inputs<L>(in, p, t);
  const int w0 = c * C::WPC;
  // the thread index is made opaque so that the per-load offsets are recomputed for every
  // chunk instead of being kept in registers for the whole loop
  int tid = static_cast<int>(threadIdx.x);
  __asm__ volatile("" : "+v"(tid));
  if constexpr (kMgThreads % C::WPC == 0) {
    constexpr int RS = kMgThreads / C::WPC;  // rows per load step
    const int r0 = tid / C::WPC, w = tid % C::WPC;
    int wi = w0 + w;
    wi = wi < p.wpr ? wi : p.wpr - 1;
    if (t.full) {
      // a running offset: one add per load, nothing kept across chunks
      uint32_t off = (__umul24(static_cast<uint32_t>(t.row0 + r0), p.wpr) + wi) * 4u;
      const uint32_t step = static_cast<uint32_t>(RS * 4) * p.wpr;
#pragma unroll
      for (int j = 0; j < C::CW; ++j) {
        st.c[j] = ld_at<uint32_t>(t.cexp, off);
        off += step;
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::CW; ++j) {
        int row = t.row0 + r0 + j * RS;
        row = row < p.N ? row : p.N - 1;
        st.c[j] = ld_at<uint32_t>(t.cexp, (__umul24(static_cast<uint32_t>(row), p.wpr) + wi) * 4u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::CW; ++j) {
      const int i = tid + j * kMgThreads;
      const int r = i / C::WPC, w = i - r * C::WPC;
      int row = t.row0 + r;
      row = row < p.N ? row : p.N - 1;
      int wi = w0 + w;
      wi = wi < p.wpr ? wi : p.wpr - 1;
      // 24-bit multiplies (full rate; rows and words per row are below 2^24, checked on
      // the host)
      st.c[j] = ld_at<uint32_t>(t.cexp, (__umul24(static_cast<uint32_t>(row), p.wpr) + wi) * 4u);
    }
  }
  const int g0 = (c * C::KC) >> p.lg_group;
  constexpr int NS = sizeof(st.s) / sizeof(st.s[0]);
  if (kMgThreads % C::WPC == 0 && t.full && t.s32) {
    // 4-byte pairs of groups: thread -> (row tid / 32 + 16 j, pair tid % 32); pairs past
    // the chunk's groups read a valid pair and are not stored
    static_assert(NS >= C::ROWS / (kMgThreads / 32), "scale staging registers");
    const int r0 = tid >> 5;
    int gi = g0 + 2 * (tid & 31);
    gi = gi < p.ngk - 1 ? gi : p.ngk - 2;
    uint32_t off = (__umul24(static_cast<uint32_t>(t.row0 + r0), p.ngk) + gi) * 2u;
    const uint32_t step = static_cast<uint32_t>((kMgThreads / 32) * 2) * p.ngk;
#pragma unroll
    for (int j = 0; j < C::ROWS / (kMgThreads / 32); ++j) {
      st.s[j] = ld_at<uint32_t>(t.sexp, off);
      off += step;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = tid + j * kMgThreads;
      const int r = t.row_of(i), k = i - static_cast<int>(__umul24(r, t.spc));
      int row = t.row0 + (r < C::ROWS ? r : C::ROWS - 1);
      row = row < p.N ? row : p.N - 1;
      int gi = g0 + k;
      gi = gi < p.ngk ? gi : p.ngk - 1;
      st.s[j] = ld_at<uint16_t>(t.sexp, (__umul24(static_cast<uint32_t>(row), p.ngk) + gi) * 2u);
    }
  }
  const uint32_t kbyte = static_cast<uint32_t>(c * C::KC) * 2u;
#pragma unroll
  for (int j = 0; j < C::AU; ++j) {
    const int i = tid + j * kMgThreads;
    const int u = i % (C::KC / 8);
    const int e = c * C::KC + 8 * u;
    if (in.on(j)) {
      // a unit past K reads the row's last unit and is stored as zero
      const uint32_t back = e < p.K ? 0u : static_cast<uint32_t>(e - (p.K - 8)) * 2u;
      const u32x4_t v = ld_at<u32x4_t>(p.xh, in.off[j] + kbyte - back);
      st.a[j] = e < p.K ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// Registers -> LDS.
template <int L>
__device__ __forceinline__ void mg_stash(const MgStage<L>& st, const MgTile& t, uint32_t* lc,
                                         uint16_t* ls, _Float16* la) {
  using C = MgChunk<L>;
#pragma unroll
  for (int j = 0; j < C::CW; ++j) {
    const int i = threadIdx.x + j * kMgThreads;
    const int r = i / C::WPC, w = i - r * C::WPC;
    lc[r * C::CST + w] = st.c[j];
  }
  constexpr int NS = sizeof(st.s) / sizeof(st.s[0]);
  if (kMgThreads % C::WPC == 0 && t.full && t.s32) {
    const int r0 = threadIdx.x >> 5, d = threadIdx.x & 31;
    if (2 * d < t.spc) {
      uint32_t* ls32 = reinterpret_cast<uint32_t*>(ls);
#pragma unroll
      for (int j = 0; j < C::ROWS / (kMgThreads / 32); ++j)
        ls32[__umul24(r0 + j * (kMgThreads / 32), t.sst >> 1) + d] = st.s[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = threadIdx.x + j * kMgThreads;
      const int r = t.row_of(i), k = i - static_cast<int>(__umul24(r, t.spc));
      if (r < C::ROWS) ls[__umul24(r, t.sst) + k] = static_cast<uint16_t>(st.s[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < C::AU; ++j) {
    const int i = threadIdx.x + j * kMgThreads;
    const int m = i / (C::KC / 8), u = i - m * (C::KC / 8);
    if (m < t.cnt) *reinterpret_cast<u32x4_t*>(la + m * C::AST + 8 * u) = st.a[j];
  }
}

template <int L>
__global__ __launch_bounds__(kMgThreads, 4) void k_mg(MgParams p) {
  using S = Span<L>;
  using C = MgChunk<L>;
  // the table is the only static LDS array: it starts at address 0
  __shared__ __attribute__((aligned(16))) uint32_t lut[mlut_bytes<L>() / 4];
  __shared__ __attribute__((aligned(16))) uint32_t lc[C::ROWS * C::CST];
  __shared__ __attribute__((aligned(16))) _Float16 la[16 * C::AST];
  __shared__ __attribute__((aligned(16))) uint16_t ls[C::ROWS * (kMaxScalesPerChunk + 2)];
  __shared__ uint16_t hs[16];
  const int e = blockIdx.y;
  const int off0 = p.offsets[e], cnt_all = p.offsets[e + 1] - off0;
  if (cnt_all <= 0) return;  // uniform per workgroup

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const uint32_t slot = mlut_slot<L>(lane);
  MgTile t;
  t.row0 = blockIdx.x * C::ROWS;
  t.spc = (C::KC >> p.lg_group) > 0 ? (C::KC >> p.lg_group) : 1;
  // the staging index i stays below 2^16, where the quotient by a multiply-high is exact
  // (ceil(2^32 / d) d - 2^32 < d); d = 1 would need 2^32
  t.spc_inv = t.spc > 1 ? 0xffffffffu / static_cast<uint32_t>(t.spc) + 1u : 0u;
  t.sst = t.spc + 2;
  t.full = t.row0 + C::ROWS <= p.N;
  t.s32 = (p.ngk % 2 == 0) && (t.spc % 2 == 0);
  t.cexp = p.codes + static_cast<int64_t>(e) * p.N * p.wpr;
  t.sexp = p.scales + static_cast<int64_t>(e) * p.N * p.ngk;
  const int nrow = wave * 16 + col;  // this lane's weight row within the workgroup
  const int n = t.row0 + nrow;
  const int nchunk = (p.K + C::KC - 1) / C::KC;
  // fragment f of a span uses scale ((e0 + 8 f) >> lg) - (chunk start >> lg) of the chunk
  MgStage<L> st;

  if (threadIdx.x < 16) hs[threadIdx.x] = p.cb.h[threadIdx.x];
  for (int m0 = 0; m0 < cnt_all; m0 += 16) {
    t.cnt = cnt_all - m0 < 16 ? cnt_all - m0 : 16;
    t.pairs = p.order + off0 + m0;
    mg_fetch<L>(st, p, t, 0);
    if (m0 == 0) {
      __syncthreads();
      build_mlut<L, kMgThreads>(lut, hs);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nchunk; ++c) {
      __syncthreads();  // previous chunk's LDS reads are done
      mg_stash<L>(st, t, lc, ls, la);
      __syncthreads();
      if (c + 1 < nchunk) mg_fetch<L>(st, p, t, c + 1);
      // super-blocks of this chunk that hold elements below K
      const int kc0 = c * C::KC;
      const int nsb = (p.K - kc0 + C::SB - 1) / C::SB < 4 ? (p.K - kc0 + C::SB - 1) / C::SB : 4;
#pragma unroll 1
      for (int sb = 0; sb < nsb; ++sb) {
        const int e0 = sb * C::SB + g * S::elems;  // within the chunk
        uint32_t w[S::words];
        const uint32_t* src = lc + nrow * C::CST + span_first_word<L>(e0);
#pragma unroll
        for (int i = 0; i < S::words; ++i) w[i] = src[i];
        uint32_t s2[S::mf];
#pragma unroll
        for (int f = 0; f < S::mf; ++f) {
          const int gi = (kc0 + e0 + 8 * f) >> p.lg_group;
          const int gl = gi - (kc0 >> p.lg_group);
          s2[f] = __umul24(static_cast<uint32_t>(ls[nrow * t.sst + gl]), 0x10001u);
        }
        u32x4_t b[S::mf];
        span_fragments<L>(w, lut, slot, s2, b);
#pragma unroll
        for (int f = 0; f < S::mf; ++f) {
          // input rows at or past the tile's pair count hold stale values; they only reach
          // rows of D that are never stored (row i of D depends on row i of A alone)
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(la + col * C::AST + e0 + 8 * f);
          acc = mfma_f16(a, b[f], acc);
        }
      }
    }
    // D[4 g + r][col] = output row n of pair m0 + 4 g + r
    if (n < p.N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * g + r;
        if (m < t.cnt) {
          const int pr = t.pairs[m];
          store_any(p.y, p.ydt, static_cast<int64_t>(pr) * p.N + n, acc[r] * p.xs[pr]);
        }
      }
    }
  }
}

// The workspace of tq_multi_gather_qmv_static: one fixed array per GPU, for callers that
// cannot allocate. Host code never passes `scratch` itself (on the host it names a stand-in,
// not device memory): static_scratch() resolves its address on the current device once
// and the kernels receive that address like any other workspace.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_multi_gather(const WeightArgs& w, const int32_t* ids, int64_t P, const void* x,
                               int xdt, bool x_rotated, void* y, int ydt, void* ws,
                               hipStream_t s) {
  if (P == 0 || w.N == 0) return hipSuccess;
  const MgLayout lay = mg_layout(w, P);
  char* base = static_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + lay.offsets);
  int32_t* order = reinterpret_cast<int32_t*>(base + lay.order);
  float* xs = reinterpret_cast<float*>(base + lay.scale);
  _Float16* xh = reinterpret_cast<_Float16*>(base + lay.rows);
  if (w.E > kMaxExperts) return hipErrorInvalidValue;
  // one launch rotates every pair's input and (one extra workgroup) buckets the pairs
  BucketJob job{ids, P, w.E, offsets, order, y, ydt, w.N};
  hipError_t err = launch_rot16(x, xdt, nullptr, P, /*zero_rows=*/1, w, x_rotated, xh, xs, &job, s);
  if (err != hipSuccess) return err;

  MgParams p{};
  p.codes = w.codes; p.scales = w.scales; p.offsets = offsets; p.order = order;
  p.xh = xh; p.xs = xs; p.y = y;
  p.rowh = rot16_row_halves(w.K);
  p.zero_row = P;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.ngk = w.K / w.group;
  p.lg_group = __builtin_ctz(w.group);
  p.ydt = ydt;
  p.cb = *codebook_for(w.levels);
  const dim3 grid((w.N + 16 * kMgWaves - 1) / (16 * kMgWaves), w.E);
  switch (w.levels) {
    case 16: hipLaunchKernelGGL(k_mg<16>, grid, dim3(kMgThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_mg<8>, grid, dim3(kMgThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_mg<4>, grid, dim3(kMgThreads), 0, s, p); break;
    default: hipLaunchKernelGGL(k_mg<3>, grid, dim3(kMgThreads), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace tq
