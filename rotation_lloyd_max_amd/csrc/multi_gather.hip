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
#include <type_traits>

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
// rotated rows [P+1][rot16_row_halves(K)] fp16 (row P all zero) | tile count int32 |
// tiles int4 [T] | tile rows int32 [T][16], T = ceil(P / 16) + min(E, P) at most;
// 256-byte aligned sections.
struct MgLayout {
  size_t offsets, order, scale, rows, ntiles, tiles, tile_rows, total;
};
static int64_t mg_max_tiles(const WeightArgs& w, int64_t P) {
  return (P + kTilePairs - 1) / kTilePairs + (P < w.E ? P : w.E);
}
static MgLayout mg_layout(const WeightArgs& w, int64_t P) {
  MgLayout l{};
  l.offsets = 0;
  l.order = align256(static_cast<size_t>(w.E + 1) * 4);
  l.scale = l.order + align256(static_cast<size_t>(P) * 4);
  l.rows = l.scale + align256(static_cast<size_t>(P + 1) * 4);
  l.ntiles = l.rows + align256(static_cast<size_t>(P + 1) * rot16_row_halves(w.K) * 2);
  l.tiles = l.ntiles + 256;
  l.tile_rows = l.tiles + align256(static_cast<size_t>(mg_max_tiles(w, P)) * 16);
  l.total = l.tile_rows + align256(static_cast<size_t>(mg_max_tiles(w, P)) * kTilePairs * 4);
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

// k_mgt: the trit layer with its staging done by direct loads into LDS.
//
// One persistent workgroup of 8 waves per compute unit walks its items (a tile of up to 16
// pairs of one expert times a block of 128 output rows): items w, w + G, w + 2G, ... of
// the tile-major list, every item's K in chunks of 480 elements (3 super-blocks of 160).
// A chunk's code words, group scales and rotated inputs go from memory straight into LDS
// (global_load_lds: no staging registers, no LDS store instructions) into stage s % 3 of a
// ring, two chunks ahead of the chunk being decoded and across item boundaries, with one
// barrier per chunk. Every thread requests the same number of direct loads per chunk
// (rows, words and units past the data load valid addresses into LDS padding that is never
// read), so a constant vmcnt waits for exactly the chunk about to be read. The direct loads
// are written as inline assembly: the compiler then neither waits for them before reading
// other stages nor counts them, and the kernel has no vector loads of its own (the items'
// pairs and input scales come through scalar loads), so every wait for memory is the
// explicit one before each barrier. Decode and matrix multiplies are those of k_mg.
constexpr int kMtSB = 3;                                           // super-blocks per chunk
constexpr int kMtKC = 160 * kMtSB;                                 // elements per chunk
constexpr int kMtWPC = kMtKC / 20;                                 // code words per row and chunk
constexpr int kMtCST = kMtWPC + 2;                                 // LDS words per row of codes
constexpr int kMtCW = (128 * kMtCST + kMgThreads - 1) / kMgThreads;  // code loads per thread
constexpr int kMtUnits = kMtKC / 8;                                // 16-byte input units per pair
constexpr int kMtAST = 65;                                         // LDS units per pair (64 + pad)

template <int LG>
struct MtScales {
  // groups a chunk touches at most, plus one half for a window that starts on an odd group
  // (the loads move 4-byte pairs of scales)
  static constexpr int halves = ((kMtKC + (1 << LG) - 1) >> LG) + 2;
  static constexpr int SST = ((halves + 1) / 2) | 1;                   // dwords per row (odd)
  static constexpr int SW = (128 * SST + kMgThreads - 1) / kMgThreads;  // scale loads per thread
  static constexpr int NDMA = kMtCW + SW + 2;                           // direct loads per chunk
};

struct MtParams {
  const uint32_t* codes;
  const uint16_t* scales;
  const _Float16* xh;
  void* y;
  int64_t rowh, zero_row;
  int K, N, E, wpr, ngk, ydt, nblk;
  CodebookArgs cb;
  // a second weight over the same pairs (the two-weight kernels: a MoE layer's gate and
  // up): items nitems .. 2 nitems - 1 read it and write rows P .. 2 P - 1
  const uint32_t* codes2;
  const uint16_t* scales2;
};

// Wait until at most N direct loads (and stores) of this wave are outstanding and its LDS
// and scalar loads are done, then the workgroup barrier (no memory fence: a fence would
// wait for every load in flight).
template <int N>
__device__ __forceinline__ void mt_sync() {
  static_assert(N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void mt_wait_vm() {
  static_assert(N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// LDS byte address of a __shared__ pointer (the value M0 takes for a direct load).
__device__ __forceinline__ uint32_t mt_lds_addr(const void* ptr) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(ptr)));
}

// Direct loads: every lane reads BYTES at base + voff (base uniform) and the wave writes
// them to LDS at lds + BYTES * lane (lds uniform). M0 holds the LDS address; its write
// needs one wait state before the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; the compiler reloads it
__device__ __forceinline__ void mt_dma4(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(mt_lds_addr(lds)),
               "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void mt_dma4_at(const void* addr, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(mt_lds_addr(lds)),
               "v"(addr)
               : "memory", "m0");
}
__device__ __forceinline__ void mt_dma16(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(mt_lds_addr(lds)),
               "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// The request side's per-item state: where the item's rows are, the rotated rows of this
// wave's two pair slots, and each thread's row offsets of its code and scale loads.
template <int LG>
struct MtReq {
  const uint32_t* codes;
  const uint16_t* scales;
  uint32_t slim;  // last 4-byte scale offset inside the array, from `scales`
  int in[2];
  uint32_t zoff[2];           // byte offset of the all-zero row from each slot's row
  uint32_t cofs[kMtCW];       // byte offset of the thread's code word in chunk 0
  uint32_t cend[kMtCW];       // ... and of the last word of its row
  uint32_t sofs[MtScales<LG>::SW];  // byte offset of the thread's scale pair in chunk 0
};

// The request side's state for an item: e its expert, in0 / in1 the rotated rows of this
// wave's two pair slots, row0 its first weight row. The thread's row and word of each
// load depend on its index only, so per chunk every load address is one add and a clamp.
template <int LG>
__device__ __forceinline__ void mt_request_item(MtReq<LG>& d, const MtParams& p, int e, int in0,
                                                int in1, int row0, int tid, int wsel) {
  using SC = MtScales<LG>;
  d.codes = (wsel ? p.codes2 : p.codes) + static_cast<int64_t>(e) * p.N * p.wpr;
  d.scales = (wsel ? p.scales2 : p.scales) + static_cast<int64_t>(e) * p.N * p.ngk;
  const int64_t lim = (static_cast<int64_t>(p.E - e) * p.N * p.ngk - 2) * 2;
  d.slim = lim < 0xfffffffcll ? static_cast<uint32_t>(lim) : 0xfffffffcu;
  d.in[0] = in0;
  d.in[1] = in1;
  d.zoff[0] = static_cast<uint32_t>((p.zero_row - in0) * p.rowh) * 2u;
  d.zoff[1] = static_cast<uint32_t>((p.zero_row - in1) * p.rowh) * 2u;
  const uint32_t wpr4 = static_cast<uint32_t>(p.wpr) * 4u, ngk2 = static_cast<uint32_t>(p.ngk) * 2u;
  // code words: LDS word i holds row i / 26, word i % 26 of the chunk (24, 25: padding,
  // which load the row's word 23)
#pragma unroll
  for (int j = 0; j < kMtCW; ++j) {
    const int i = j * kMgThreads + tid, r = i / kMtCST, wd = i - r * kMtCST;
    int row = row0 + (r < 128 ? r : 127);
    row = row < p.N ? row : p.N - 1;
    const uint32_t base = __umul24(static_cast<uint32_t>(row), wpr4);
    d.cofs[j] = base + static_cast<uint32_t>(wd < kMtWPC ? wd : kMtWPC - 1) * 4u;
    d.cend[j] = base + wpr4 - 4u;
  }
#pragma unroll
  for (int j = 0; j < SC::SW; ++j) {
    const int i = j * kMgThreads + tid, r = i / SC::SST, dw = i - r * SC::SST;
    int row = row0 + (r < 128 ? r : 127);
    row = row < p.N ? row : p.N - 1;
    d.sofs[j] = __umul24(static_cast<uint32_t>(row), ngk2) + static_cast<uint32_t>(dw) * 4u;
  }
}

// Direct load I (of NDMA) of chunk c of the request item into one stage: code words,
// then scale pairs, then the inputs of the wave's two pair slots.
template <int LG, int I>
__device__ __forceinline__ void mt_dma_one(const MtReq<LG>& d, const MtParams& p, int c,
                                           uint32_t* lcw, uint32_t* lsw, u32x4_t* law, int wave,
                                           int lane) {
  using SC = MtScales<LG>;
  if constexpr (I < kMtCW) {
    // LDS word i holds row i / 26, word i % 26 of the chunk (24, 25: padding)
    const uint32_t off = d.cofs[I] + static_cast<uint32_t>(c * kMtWPC) * 4u;
    mt_dma4(d.codes, off < d.cend[I] ? off : d.cend[I], lcw + I * kMgThreads + wave * 64);
  } else if constexpr (I < kMtCW + SC::SW) {
    // 4-byte pairs from the even group at or below the chunk's first group
    const uint32_t off = d.sofs[I - kMtCW] + static_cast<uint32_t>(((c * kMtKC) >> LG) & ~1) * 2u;
    mt_dma4(d.scales, off < d.slim ? off : d.slim, lsw + (I - kMtCW) * kMgThreads + wave * 64);
  } else {
    // unit = lane of pair slot 2 wave + jj, as a byte offset from the slot's row (units past
    // the chunk or past K read the all-zero row, which follows every pair's)
    constexpr int jj = I - kMtCW - SC::SW;
    const int e = c * kMtKC + 8 * lane;
    const bool ok = lane < kMtUnits && e < p.K;
    mt_dma16(p.xh + static_cast<int64_t>(d.in[jj]) * p.rowh,
             ok ? static_cast<uint32_t>(e) * 2u : d.zoff[jj], law + (2 * wave + jj) * kMtAST);
  }
}

// Part PART (of three) of the direct loads of chunk c: spread over the decode of the chunk
// being read, so that the waves' address processing overlaps their arithmetic.
template <int LG, int PART, int... I>
__device__ __forceinline__ void mt_request_part_(std::integer_sequence<int, I...>, const MtReq<LG>& d,
                                                 const MtParams& p, int c, uint32_t* lcw,
                                                 uint32_t* lsw, u32x4_t* law, int wave, int lane) {
  constexpr int per = (MtScales<LG>::NDMA + 2) / 3;
  (mt_dma_one<LG, PART * per + I>(d, p, c, lcw, lsw, law, wave, lane), ...);
}
template <int LG, int PART>
__device__ __forceinline__ void mt_request_part(const MtReq<LG>& d, const MtParams& p, int c,
                                                uint32_t* lcw, uint32_t* lsw, u32x4_t* law,
                                                int wave, int lane) {
  constexpr int n = MtScales<LG>::NDMA, per = (n + 2) / 3;
  constexpr int cnt = n - PART * per < per ? n - PART * per : per;
  mt_request_part_<LG, PART>(std::make_integer_sequence<int, cnt>{}, d, p, c, lcw, lsw, law, wave,
                             lane);
}

// The 16-byte layout (groups of 16, rows of scales a multiple of 16 bytes, N * wpr a
// multiple of 4, 16-byte aligned arrays): a chunk's code words come as 7 aligned 16-byte
// units per row from the aligned word at or below the row's first word of the chunk (the
// row's word r * wpr mod 4 is its shift inside the units; LDS rows of 28 words), its
// scales as 5 aligned units from the aligned group at or below its first group (LDS rows of
// 40 halves). 896 code units and 640 scale units: waves 0..5 load two code units and one
// scale unit per lane, waves 6 and 7 one and two, so every wave issues 5 loads per chunk
// (with its two input units). Units never cross the end of the arrays (their ends are
// 16-byte aligned); units past a row's data hold the next row's (never decoded values
// past K, whose inputs are zero).
constexpr int kMt4CU = 7;   // code units per row and chunk
constexpr int kMt4SU = 5;   // scale units per row and chunk
constexpr int kMt4NDMA = 5;
struct MtReq4 {
  const uint32_t* codes;
  const uint16_t* scales;
  uint32_t clim, slim;  // last 16-byte unit inside each array, from `codes` / `scales`
  int in[2];
  uint32_t zoff[2];     // byte offset of the all-zero row from each slot's row
  uint32_t cofs[2];     // byte offset of the thread's code units in chunk 0
  uint32_t sofs[2];     // ... and of its scale units
};

__device__ __forceinline__ void mt_request_item4(MtReq4& d, const MtParams& p, int e, int in0,
                                                 int in1, int row0, int wave, int lane, int wsel) {
  d.codes = (wsel ? p.codes2 : p.codes) + static_cast<int64_t>(e) * p.N * p.wpr;
  d.scales = (wsel ? p.scales2 : p.scales) + static_cast<int64_t>(e) * p.N * p.ngk;
  const int64_t cl = static_cast<int64_t>(p.E - e) * p.N * p.wpr * 4 - 16;
  const int64_t sl = static_cast<int64_t>(p.E - e) * p.N * p.ngk * 2 - 16;
  d.clim = cl < 0xfffffff0ll ? static_cast<uint32_t>(cl) : 0xfffffff0u;
  d.slim = sl < 0xfffffff0ll ? static_cast<uint32_t>(sl) : 0xfffffff0u;
  d.in[0] = in0;
  d.in[1] = in1;
  d.zoff[0] = static_cast<uint32_t>((p.zero_row - in0) * p.rowh) * 2u;
  d.zoff[1] = static_cast<uint32_t>((p.zero_row - in1) * p.rowh) * 2u;
  // code unit u = row u / 7, unit u % 7; units 0..511 by every wave, 512..895 by waves 0..5
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = j * kMgThreads + wave * 64 + lane;
    const int r = u / kMt4CU, q = u - r * kMt4CU;
    int row = row0 + (r < 128 ? r : 127);
    row = row < p.N ? row : p.N - 1;
    d.cofs[j] = (__umul24(static_cast<uint32_t>(row), static_cast<uint32_t>(p.wpr)) & ~3u) * 4u +
                static_cast<uint32_t>(q) * 16u;
  }
  // scale unit u = row u / 5, unit u % 5; units 0..511 by every wave, 512..639 by waves 6, 7
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int u = j * kMgThreads + (j ? wave - 6 : wave) * 64 + lane;
    const int r = u / kMt4SU, q = u - r * kMt4SU;
    int row = row0 + (r < 128 ? r : 127);
    row = row < p.N ? row : p.N - 1;
    d.sofs[j] = __umul24(static_cast<uint32_t>(row), static_cast<uint32_t>(p.ngk) * 2u) +
                static_cast<uint32_t>(q) * 16u;
  }
}

// Part PART (of three) of the 16-byte loads of chunk c: code units and the wave's second
// unit (code or scale), the first scale unit, the inputs.
template <int PART>
__device__ __forceinline__ void mt_request4_part(const MtReq4& d, const MtParams& p, int c,
                                                 uint32_t* lcw, uint32_t* lsw, u32x4_t* law,
                                                 int wave, int lane) {
  const uint32_t cadd = static_cast<uint32_t>(c * kMtWPC) * 4u;            // 24 c words
  const uint32_t sadd = static_cast<uint32_t>((c * kMtKC) >> 4) * 2u & ~15u;  // group 30 c
  if constexpr (PART == 0) {
    uint32_t off = d.cofs[0] + cadd;
    mt_dma16(d.codes, off < d.clim ? off : d.clim, lcw + wave * 256);
    if (wave < 6) {
      off = d.cofs[1] + cadd;
      mt_dma16(d.codes, off < d.clim ? off : d.clim, lcw + (kMgThreads + wave * 64) * 4);
    } else {
      off = d.sofs[1] + sadd;
      mt_dma16(d.scales, off < d.slim ? off : d.slim, lsw + (kMgThreads + (wave - 6) * 64) * 4);
    }
  } else if constexpr (PART == 1) {
    const uint32_t off = d.sofs[0] + sadd;
    mt_dma16(d.scales, off < d.slim ? off : d.slim, lsw + wave * 256);
  } else {
    const int e = c * kMtKC + 8 * lane;
    const bool ok = lane < kMtUnits && e < p.K;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      mt_dma16(p.xh + static_cast<int64_t>(d.in[jj]) * p.rowh,
               ok ? static_cast<uint32_t>(e) * 2u : d.zoff[jj], law + (2 * wave + jj) * kMtAST);
  }
}

// Super-block SB of a chunk.
template <int LG, int SB>
__device__ __forceinline__ void mt_decode_sb(f32x4_t& acc, int kr, const uint32_t* cw,
                                             const uint16_t* sw, const u32x4_t* aw,
                                             const uint32_t* lut, uint32_t slot, int g) {
  constexpr int sb = SB;
  const uint32_t w[2] = {cw[8 * sb], cw[8 * sb + 1]};
  uint32_t s2[5];
  if constexpr (LG == 4) {
    // the 40-element span of lane group g starts at 40 g: fragment f is in group
    // 10 sb + floor(5 g / 2) + (g odd + f) / 2 of the chunk
    const uint16_t* sg = sw + 10 * sb + ((5 * g) >> 1);
    const uint32_t a0 = __umul24(static_cast<uint32_t>(sg[0]), 0x10001u);
    const uint32_t a1 = __umul24(static_cast<uint32_t>(sg[1]), 0x10001u);
    const uint32_t a2 = __umul24(static_cast<uint32_t>(sg[2]), 0x10001u);
    const bool odd = (g & 1) != 0;
    s2[0] = a0;
    s2[1] = odd ? a1 : a0;
    s2[2] = a1;
    s2[3] = odd ? a2 : a1;
    s2[4] = a2;
  } else {
#pragma unroll
    for (int f = 0; f < 5; ++f)
      s2[f] = __umul24(static_cast<uint32_t>(sw[(kr + 160 * sb + 40 * g + 8 * f) >> LG]),
                       0x10001u);
  }
  u32x4_t b[5];
  span_fragments<3>(w, lut, slot, s2, b);
#pragma unroll
  for (int f = 0; f < 5; ++f) acc = mfma_f16(aw[20 * sb + f], b[f], acc);
}


// Super-blocks 0 .. NSB - 1 of a chunk, after(sb) called after each (see mt_decode).
template <int LG, int NSB, typename After>
__device__ __forceinline__ void mt_decode_sbs(f32x4_t& acc, int kr, const uint32_t* cw,
                                              const uint16_t* sw, const u32x4_t* aw,
                                              const uint32_t* lut, uint32_t slot, int g,
                                              After after) {
  [&]<int... SB>(std::integer_sequence<int, SB...>) {
    ((mt_decode_sb<LG, SB>(acc, kr, cw, sw, aw, lut, slot, g),
      after(std::integral_constant<int, SB>{})),
     ...);
  }(std::make_integer_sequence<int, NSB>{});
}

// Decode chunk c from one stage into the lane's accumulator.
template <int LG, bool X4, typename After>
__device__ __forceinline__ void mt_decode(f32x4_t& acc, const MtParams& p, int c,
                                          const uint32_t* lcr, const uint32_t* lsr,
                                          const u32x4_t* lar, const uint32_t* lut, uint32_t slot,
                                          int nrow, int cshift, int g, int col, After after) {
  using SC = MtScales<LG>;
  const int kc0 = c * kMtKC;
  const int nsb = (p.K - kc0 + 159) / 160 < kMtSB ? (p.K - kc0 + 159) / 160 : kMtSB;
  const int g0 = kc0 >> LG;
  // code words of this row (after the row's shift in the 16-byte layout); half index of
  // group gi of this row: (gi - g0) + the window's offset (g0 mod 8 in 16-byte units,
  // g0 mod 2 in 4-byte pairs)
  const uint32_t* cw = X4 ? lcr + nrow * (4 * kMt4CU) + cshift + 2 * g : lcr + nrow * kMtCST + 2 * g;
  const uint16_t* sw = X4 ? reinterpret_cast<const uint16_t*>(lsr) + nrow * (8 * kMt4SU) + (g0 & 7)
                          : reinterpret_cast<const uint16_t*>(lsr) + nrow * (2 * SC::SST) + (g0 & 1);
  const u32x4_t* aw = lar + col * kMtAST + 5 * g;
  const int kr = kc0 - (g0 << LG);  // chunk start within its group
  // a full chunk as one block of straight-line code (the scheduler can then overlap the
  // super-blocks' LDS reads with the arithmetic of the ones before); the last chunk of a
  // row may hold fewer super-blocks, and after() still runs three times
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (nsb == kMtSB) {
    mt_decode_sbs<LG, kMtSB>(acc, kr, cw, sw, aw, lut, slot, g, after);
  } else if (nsb == 2) {
    mt_decode_sbs<LG, 2>(acc, kr, cw, sw, aw, lut, slot, g, after);
    after(I2{});
  } else {
    mt_decode_sbs<LG, 1>(acc, kr, cw, sw, aw, lut, slot, g, after);
    after(I1{});
    after(I2{});
  }
}

// Items have at least two chunks (K > 480). Besides the chunks, wave 0 requests the
// description of item k + 2 into LDS at the first chunk of item k (the tile's 16 pair rows
// and its {expert, first position, pairs} entry) and the pairs' input scales at the second
// (three slots, item j in slot j % 3), before that step's chunk requests, so that the
// barrier's wait covers them; both sides then read the items from LDS. Item 0's expert and
// pair rows for the first requests come from scalar loads.
constexpr int kMtInfo = kTilePairs + 4;  // LDS words per item: pair rows, tile entry
template <int LG, bool X4, bool NW2>
__global__ __launch_bounds__(kMgThreads) void k_mgt(MtParams p, const int4* __restrict__ tiles,
                                                    const int32_t* __restrict__ tile_rows,
                                                    const int32_t* __restrict__ ntiles,
                                                    const float* __restrict__ xs) {
  using SC = MtScales<LG>;
  static_assert(!X4 || LG == 4, "the 16-byte layout is for groups of 16");
  constexpr int NDMA = X4 ? kMt4NDMA : SC::NDMA;  // direct loads per thread and chunk
  constexpr int CS = X4 ? 896 * 4 : kMtCW * kMgThreads;
  constexpr int SS = X4 ? 640 * 4 : SC::SW * kMgThreads;
  constexpr int AS = kTilePairs * kMtAST;
  __shared__ __attribute__((aligned(16))) uint32_t lut[mlut_bytes<3>() / 4];
  __shared__ __attribute__((aligned(16))) uint32_t lc0[CS], lc1[CS], lc2[CS];
  __shared__ __attribute__((aligned(16))) uint32_t ls0[SS], ls1[SS], ls2[SS];
  __shared__ __attribute__((aligned(16))) u32x4_t la0[AS], la1[AS], la2[AS];
  __shared__ __attribute__((aligned(16))) int32_t info[3][kMtInfo];
  __shared__ __attribute__((aligned(16))) float ixs[3][kTilePairs];
  __shared__ uint16_t hs[16];

  const int nitems1 = *ntiles * p.nblk;  // items of one weight
  const int nitems = NW2 ? 2 * nitems1 : nitems1;
  const int G = static_cast<int>(gridDim.x), w0 = static_cast<int>(blockIdx.x);
  if (w0 >= nitems) return;  // uniform
  const int nch = (p.K + kMtKC - 1) / kMtKC;  // at least 2
  const int nk = (nitems - w0 + G - 1) / G;   // items of this workgroup
  const int total = nk * nch;                  // chunks of this workgroup

  const int tid = static_cast<int>(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, col = lane & 15;
  const uint32_t slot = mlut_slot<3>(lane);
  const int nrow = wave * 16 + col;  // this lane's weight row within the block
  auto item_tile = [&](int k, int& T, int& row0, int& wsel) __attribute__((always_inline)) {
    int i = w0 + k * G;
    wsel = NW2 && i >= nitems1 ? 1 : 0;  // a constant 0 in the one-weight kernels
    i -= wsel ? nitems1 : 0;
    T = i / p.nblk;
    row0 = (i - T * p.nblk) * 128;
  };
  // wave 0: item k's pair rows (lanes 0..15) and tile entry (lanes 16..19) into LDS ...
  auto info_req = [&](int k) __attribute__((always_inline)) {
    if (wave == 0 && lane < kMtInfo) {
      int T, row0, wsel;
      item_tile(k, T, row0, wsel);
      const void* a = lane < kTilePairs
                          ? static_cast<const void*>(tile_rows + T * kTilePairs + lane)
                          : static_cast<const void*>(reinterpret_cast<const int32_t*>(tiles + T) +
                                                     (lane - kTilePairs));
      mt_dma4_at(a, info[k % 3]);
    }
  };
  // ... and, once those are in LDS, its pairs' input scales
  auto info_xs = [&](int k) __attribute__((always_inline)) {
    if (wave == 0 && lane < kTilePairs)
      mt_dma4(xs, static_cast<uint32_t>(info[k % 3][lane]) * 4u, ixs[k % 3]);
  };

  // Request side: every step requests a chunk, so that each wave has the same loads in
  // flight on every path; requests past the last chunk repeat it into a stage that is never
  // read again. Counters move by arithmetic (a branch that picks which counter to bump turns
  // them into memory).
  std::conditional_t<X4, MtReq4, MtReq<LG>> d;
  int dk = 0, dc = 0;
  auto request_item = [&](int e, int in0, int in1, int row0, int wsel)
                          __attribute__((always_inline)) {
    if constexpr (X4) mt_request_item4(d, p, e, in0, in1, row0, wave, lane, wsel);
    else mt_request_item<LG>(d, p, e, in0, in1, row0, tid, wsel);
  };
  auto request_part = [&](auto part, int c, uint32_t* lcw, uint32_t* lsw, u32x4_t* law)
                          __attribute__((always_inline)) {
    if constexpr (X4) mt_request4_part<decltype(part)::value>(d, p, c, lcw, lsw, law, wave, lane);
    else mt_request_part<LG, decltype(part)::value>(d, p, c, lcw, lsw, law, wave, lane);
  };
  // request_begin returns the chunk to request (switching items where one starts), the
  // parts go out during the decode, request_end moves on
  auto request_begin = [&]() __attribute__((always_inline)) {
    if (dc == 0 && dk > 0 && dk < nk) {
      int T, row0, wsel;
      item_tile(dk, T, row0, wsel);
      const int* it = info[dk % 3];
      request_item(__builtin_amdgcn_readfirstlane(it[kTilePairs]),
                   __builtin_amdgcn_readfirstlane(it[2 * wave]),
                   __builtin_amdgcn_readfirstlane(it[2 * wave + 1]), row0, wsel);
    }
    return dk < nk ? dc : nch - 1;
  };
  auto request_end = [&]() __attribute__((always_inline)) {
    const bool wrap = dc + 1 == nch;
    dk += wrap ? 1 : 0;
    dc = wrap ? 0 : dc + 1;
  };
  auto request = [&](uint32_t* lcw, uint32_t* lsw, u32x4_t* law) __attribute__((always_inline)) {
    const int c = request_begin();
    request_part(std::integral_constant<int, 0>{}, c, lcw, lsw, law);
    request_part(std::integral_constant<int, 1>{}, c, lcw, lsw, law);
    request_part(std::integral_constant<int, 2>{}, c, lcw, lsw, law);
    request_end();
  };

  // Prologue: items 0 and 1 described in LDS, the first two chunks requested (item 0 from
  // scalar loads), the table built; wave 0 then waits for the descriptions (its oldest
  // loads) and requests the input scales.
  {
    int T, row0, wsel;
    item_tile(0, T, row0, wsel);
    request_item(tiles[T].x, tile_rows[T * kTilePairs + 2 * wave],
                 tile_rows[T * kTilePairs + 2 * wave + 1], row0, wsel);
  }
  info_req(0);
  if (nk > 1) info_req(1);
  if (tid < 16) hs[tid] = p.cb.h[tid];
  request(lc0, ls0, la0);
  request(lc1, ls1, la1);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  build_mlut<3, kMgThreads>(lut, hs);
  if (wave == 0) {
    mt_wait_vm<2 * NDMA>();
    info_xs(0);
    if (nk > 1) info_xs(1);
  }

  // Decode side.
  int kk = 0, kc = 0;
  int cshift = 0;  // this lane's row's shift inside the 16-byte code units
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](uint32_t* lcw, uint32_t* lsw, u32x4_t* law, const uint32_t* lcr,
                  const uint32_t* lsr, const u32x4_t* lar) __attribute__((always_inline)) {
    mt_sync<NDMA>();
    if constexpr (X4) {
      if (kc == 0) {
        int T, row0, wsel;
        item_tile(kk, T, row0, wsel);
        const int row = row0 + nrow < p.N ? row0 + nrow : p.N - 1;
        cshift = static_cast<int>(__umul24(static_cast<uint32_t>(row), static_cast<uint32_t>(p.wpr)) & 3u);
      }
    }
    if (kk + 2 < nk) {
      if (kc == 0) info_req(kk + 2);
      else if (kc == 1) info_xs(kk + 2);
    }
    const int rc = request_begin();
    mt_decode<LG, X4>(acc, p, kc, lcr, lsr, lar, lut, slot, nrow, cshift, g, col,
                      [&](auto part) { request_part(part, rc, lcw, lsw, law); });
    request_end();
    if (kc == nch - 1) {
      // D[4 g + r][col] = output row row0 + nrow of the tile's pair 4 g + r
      int T, row0, wsel;
      item_tile(kk, T, row0, wsel);
      const int n = row0 + nrow;
      const int64_t ybase = wsel ? p.zero_row : 0;  // the second weight's rows follow the P first
      const int* it = info[kk % 3];
      const int cnt = it[kTilePairs + 2];
      const int4 pr = *reinterpret_cast<const int4*>(it + 4 * g);
      const float4 sc = *reinterpret_cast<const float4*>(&ixs[kk % 3][4 * g]);
      const int prs[4] = {pr.x, pr.y, pr.z, pr.w};
      const float scs[4] = {sc.x, sc.y, sc.z, sc.w};
      if (n < p.N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g + r < cnt)
            store_any(p.y, p.ydt, (ybase + prs[r]) * p.N + n, acc[r] * scs[r]);
      }
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bool wrap = kc + 1 == nch;
    kk += wrap ? 1 : 0;
    kc = wrap ? 0 : kc + 1;
  };

  for (int s = 0; s < total; s += 3) {
    step(lc2, ls2, la2, lc0, ls0, la0);
    if (s + 1 >= total) break;
    step(lc0, ls0, la0, lc1, ls1, la1);
    if (s + 2 >= total) break;
    step(lc1, ls1, la1, lc2, ls2, la2);
  }
  // the repeated requests of the last steps land in LDS before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

// Compute units of the current device (looked up once per device).
static hipError_t compute_units(int* n) {
  static std::mutex mu;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    e = hipDeviceGetAttribute(&cache[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cache[dev] <= 0) return hipErrorInvalidDevice;
  }
  *n = cache[dev];
  return hipSuccess;
}

hipError_t launch_multi_gather(const WeightArgs& w, const int32_t* ids, int64_t P, const void* x,
                               int xdt, bool x_rotated, void* y, int ydt, void* ws,
                               hipStream_t s, const WeightArgs* w2) {
  if (P == 0 || w.N == 0) return hipSuccess;
  const MgLayout lay = mg_layout(w, P);
  char* base = static_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + lay.offsets);
  int32_t* order = reinterpret_cast<int32_t*>(base + lay.order);
  float* xs = reinterpret_cast<float*>(base + lay.scale);
  _Float16* xh = reinterpret_cast<_Float16*>(base + lay.rows);
  if (w.E > kMaxExperts) return hipErrorInvalidValue;
  // trits with 4-byte aligned rows of scales: the direct-load kernel, which needs the tiles
  const bool direct = w.levels == 3 && w.group >= 16 && w.group <= 128 &&
                      (w.K / w.group) % 2 == 0 && w.K > kMtKC &&
                      (P + 1) * rot16_row_halves(w.K) * 2 < (int64_t(1) << 32);
  int4* tiles = reinterpret_cast<int4*>(base + lay.tiles);
  int32_t* tile_rows = reinterpret_cast<int32_t*>(base + lay.tile_rows);
  int32_t* ntiles = reinterpret_cast<int32_t*>(base + lay.ntiles);
  // one launch rotates every pair's input and (one extra workgroup) buckets the pairs
  BucketJob job{ids, P, w.E, offsets, order, y, ydt, w.N,
                direct ? tiles : nullptr, tile_rows, ntiles, static_cast<int32_t>(P), w2 ? 2 : 1};
  hipError_t err = launch_rot16(x, xdt, nullptr, P, /*zero_rows=*/1, w, x_rotated, xh, xs, &job, s);
  if (err != hipSuccess) return err;
  if (direct) {
    MtParams q{};
    q.codes = w.codes; q.scales = w.scales; q.xh = xh; q.y = y;
    q.rowh = rot16_row_halves(w.K);
    q.zero_row = P;
    q.K = w.K; q.N = w.N; q.E = w.E; q.wpr = w.wpr; q.ngk = w.K / w.group; q.ydt = ydt;
    q.nblk = (w.N + 127) / 128;
    q.cb = *codebook_for(w.levels);
    q.codes2 = w2 ? w2->codes : w.codes;
    q.scales2 = w2 ? w2->scales : w.scales;
    const int nw = w2 ? 2 : 1;
    // one workgroup per compute unit (each holds 141 KB of LDS); the items are shared out
    // on the device, where their number is known
    int ncu = 0;
    err = compute_units(&ncu);
    if (err != hipSuccess) return err;
    const int64_t items = mg_max_tiles(w, P) * q.nblk * nw;
    const int grid = static_cast<int>(items < ncu ? items : ncu);
    // 16-byte loads where every unit stays inside its array: groups of 16, rows of scales a
    // multiple of 16 bytes, whole 16-byte units of codes per expert, aligned arrays
    const bool x4 = w.group == 16 && q.ngk % 8 == 0 && (static_cast<int64_t>(w.N) * w.wpr) % 4 == 0 &&
                    ((reinterpret_cast<uintptr_t>(w.codes) | reinterpret_cast<uintptr_t>(q.codes2)) & 15) == 0 &&
                    ((reinterpret_cast<uintptr_t>(w.scales) | reinterpret_cast<uintptr_t>(q.scales2)) & 15) == 0;
    const auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kMgThreads), 0, s, q, tiles, tile_rows, ntiles, xs);
    };
    const auto pick = [&](auto nw2) {
      constexpr bool N2 = decltype(nw2)::value;
      if (x4) {
        launch(k_mgt<4, true, N2>);
      } else {
        switch (__builtin_ctz(w.group)) {
          case 4: launch(k_mgt<4, false, N2>); break;
          case 5: launch(k_mgt<5, false, N2>); break;
          case 6: launch(k_mgt<6, false, N2>); break;
          default: launch(k_mgt<7, false, N2>); break;
        }
      }
    };
    if (nw == 2) pick(std::true_type{});
    else pick(std::false_type{});
    return hipGetLastError();
  }

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
  // with a second weight: a second launch over the same rotated inputs and buckets
  for (int h = 0; h < (w2 ? 2 : 1); ++h) {
    if (h == 1) {
      p.codes = w2->codes;
      p.scales = w2->scales;
      p.y = static_cast<char*>(y) + P * w.N * (ydt == 0 ? 4 : 2);
    }
    switch (w.levels) {
      case 16: hipLaunchKernelGGL(k_mg<16>, grid, dim3(kMgThreads), 0, s, p); break;
      case 8: hipLaunchKernelGGL(k_mg<8>, grid, dim3(kMgThreads), 0, s, p); break;
      case 4: hipLaunchKernelGGL(k_mg<4>, grid, dim3(kMgThreads), 0, s, p); break;
      default: hipLaunchKernelGGL(k_mg<3>, grid, dim3(kMgThreads), 0, s, p); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tq
