// Counting sort of (input, expert) pairs by expert, for multi_gather_qmv: offsets[e] = first
// position of expert e's pairs in `order`, order[] = pair indices grouped by expert (in any
// order within an expert: atomics). Pairs with an expert id outside [0, E) get a row of NaN
// in y and no position. With `tiles` set, the pairs of every expert are also cut into tiles
// of up to kTilePairs: tiles[t] = {expert, first position in order, pairs, 0} (experts in
// increasing order), tile_rows[t][m] = pair m of the tile (zero_row past its pairs), and
// *ntiles = their number. Run by one workgroup of NT threads.
#pragma once

#include "device_common.hpp"

namespace tq {

constexpr int kTilePairs = 16;

struct BucketJob {
  const int32_t* ids;
  int64_t P;
  int E;
  int32_t* offsets;
  int32_t* order;
  void* y;
  int ydt, N;
  int4* tiles;         // optional tile table (nullptr: none)
  int32_t* tile_rows;
  int32_t* ntiles;
  int32_t zero_row;
  int nw = 1;  // weights sharing the pairs: the NaN row of a bad pair is written in each
               // weight's rows (weight h at rows h P ..)
};

// Exclusive scan of v(e) over e < E by the whole workgroup, NT values at a time with a
// running carry: put(e, sum of v(e') for e' < e) for every e < E; returns the total. v(e)
// is read before, and put called after, the barriers of its chunk.
template <int NT, typename V, typename Put>
__device__ __forceinline__ int block_exclusive_scan(int E, int32_t* wsum, V v_of, Put put) {
  int carry = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < E; base += NT) {
    const int e = base + threadIdx.x;
    const int c = e < E ? v_of(e) : 0;
    int v = c;
    for (int off = 1; off < 64; off <<= 1) {  // inclusive wave scan
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = carry, total = carry;
    for (int k = 0; k < NT / 64; ++k) {
      before += k < wave ? wsum[k] : 0;
      total += wsum[k];
    }
    __syncthreads();
    if (e < E) put(e, before + v - c);
    carry = total;
  }
  return carry;
}

// The same scan for two values at once: put(e, sums of a(e'), sums of b(e') for e' < e,
// a(e), b(e)); returns both totals. wsum: 2 NT / 64 ints of LDS.
template <int NT, typename V, typename Put>
__device__ __forceinline__ int2 block_exclusive_scan2(int E, int32_t* wsum, V v_of, Put put) {
  int2 carry = make_int2(0, 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < E; base += NT) {
    const int e = base + threadIdx.x;
    const int2 c = e < E ? v_of(e) : make_int2(0, 0);
    int2 v = c;
    for (int off = 1; off < 64; off <<= 1) {  // inclusive wave scans
      const int tx = __shfl_up(v.x, off, 64), ty = __shfl_up(v.y, off, 64);
      if (lane >= off) {
        v.x += tx;
        v.y += ty;
      }
    }
    if (lane == 63) {
      wsum[wave] = v.x;
      wsum[NT / 64 + wave] = v.y;
    }
    __syncthreads();
    int2 before = carry, total = carry;
    for (int k = 0; k < NT / 64; ++k) {
      const int ax = wsum[k], ay = wsum[NT / 64 + k];
      if (k < wave) {
        before.x += ax;
        before.y += ay;
      }
      total.x += ax;
      total.y += ay;
    }
    __syncthreads();
    if (e < E) put(e, before.x + v.x - c.x, before.y + v.y - c.y, c.x, c.y);
    carry = total;
  }
  return carry;
}

// cnt: E ints of LDS (2 E with tiles); wsum: 2 NT / 64 ints.
template <int NT>
__device__ __forceinline__ void bucket_pairs(const BucketJob& b, int32_t* cnt, int32_t* wsum) {
  const int E = b.E;
  int32_t* t0 = cnt + E;  // with tiles: first tile of each expert
  for (int e = threadIdx.x; e < E; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < b.P; p += NT) {
    const int e = b.ids[p];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
    } else {
      for (int h = 0; h < b.nw; ++h)
        for (int n = 0; n < b.N; ++n)
          store_any(b.y, b.ydt, (h * b.P + p) * b.N + n, __builtin_nanf(""));
    }
  }
  __syncthreads();
  if (!b.tiles) {
    const int total = block_exclusive_scan<NT>(
        E, wsum, [&](int e) { return cnt[e]; },
        [&](int e, int excl) {
          b.offsets[e] = excl;
          cnt[e] = excl;  // becomes the scatter cursor
        });
    if (threadIdx.x == 0) b.offsets[E] = total;
  } else {
    // offsets and tile starts in one scan; each expert's tile entries, and the padding of
    // its last tile, written by its thread
    const int2 total = block_exclusive_scan2<NT>(
        E, wsum,
        [&](int e) { return make_int2(cnt[e], (cnt[e] + kTilePairs - 1) / kTilePairs); },
        [&](int e, int start, int tstart, int n, int nt) {
          b.offsets[e] = start;
          cnt[e] = start;  // becomes the scatter cursor
          t0[e] = tstart;
          for (int t = 0; t < nt; ++t) {
            const int m = n - t * kTilePairs < kTilePairs ? n - t * kTilePairs : kTilePairs;
            b.tiles[tstart + t] = make_int4(e, start + t * kTilePairs, m, 0);
          }
          for (int j = n; j < nt * kTilePairs; ++j)
            b.tile_rows[tstart * kTilePairs + j] = b.zero_row;
        });
    if (threadIdx.x == 0) {
      b.offsets[E] = total.x;
      *b.ntiles = total.y;
    }
  }
  __syncthreads();
  for (int64_t p = threadIdx.x; p < b.P; p += NT) {
    const int e = b.ids[p];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&cnt[e], 1);
      b.order[pos] = static_cast<int32_t>(p);
      // pair j of expert e is pair j % 16 of its tile j / 16
      if (b.tiles) b.tile_rows[t0[e] * kTilePairs + (pos - b.offsets[e])] = static_cast<int32_t>(p);
    }
  }
}

}  // namespace tq
