// Counting sort of (input, expert) pairs by expert, for multi_gather_qmv: offsets[e] = first
// position of expert e's pairs in `order`, order[] = pair indices grouped by expert (in any
// order within an expert: atomics). Pairs with an expert id outside [0, E) get a row of NaN
// in y and no position. Run by one workgroup of NT threads; cnt is LDS for E counters and
// wsum LDS for NT / 64 wave sums.
#pragma once

#include "device_common.hpp"

namespace tq {

struct BucketJob {
  const int32_t* ids;
  int64_t P;
  int E;
  int32_t* offsets;
  int32_t* order;
  void* y;
  int ydt, N;
};

template <int NT>
__device__ __forceinline__ void bucket_pairs(const BucketJob& b, int32_t* cnt, int32_t* wsum) {
  const int E = b.E;
  for (int e = threadIdx.x; e < E; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < b.P; p += NT) {
    const int e = b.ids[p];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
    } else {
      for (int n = 0; n < b.N; ++n) store_any(b.y, b.ydt, p * b.N + n, __builtin_nanf(""));
    }
  }
  __syncthreads();
  // exclusive scan of cnt[0..E) in chunks of NT, carried as a running sum
  int carry = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < E; base += NT) {
    const int e = base + threadIdx.x;
    const int c = e < E ? cnt[e] : 0;
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
    if (e < E) {
      const int excl = before + v - c;
      b.offsets[e] = excl;
      cnt[e] = excl;  // becomes the scatter cursor
    }
    carry = total;
  }
  if (threadIdx.x == 0) b.offsets[E] = carry;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < b.P; p += NT) {
    const int e = b.ids[p];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&cnt[e], 1);
      b.order[pos] = static_cast<int32_t>(p);
    }
  }
}

}  // namespace tq
