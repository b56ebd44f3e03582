// Rows rotated once into an fp16 workspace, for the kernels that multiply many inputs by
// decoded weights on the matrix cores (multi_gather_qmv, gather_qmm).
//
// Row r of the workspace holds x'_r = H_K diag(s) x_r (unnormalized) times a power of two
// sc_r chosen from max |x_r| (prologue.hpp), as K consecutive fp16 values, so 8 elements
// starting at a multiple of 8 are one aligned 16-byte load. scale[r] = 1 / (sc_r sqrt(K))
// (or 1 / sc_r for an input that is already rotated) is applied to the products.
#pragma once

#include "bucket.hpp"
#include "prologue.hpp"

namespace tq {

constexpr int kRotThreads = 256;

__host__ __device__ constexpr int64_t rot16_row_halves(int K) { return K; }

struct Rot16Params {
  const void* x;        // [rows][K] input rows (dtype xdt)
  const int32_t* rows;  // optional: row r of the output is input row rows[r]
  const uint32_t* signs;
  _Float16* out;        // [rows][rot16_row_halves(K)]
  float* scale;         // [rows]
  int64_t nrows;        // rows with an input; rows nrows .. nrows + zero_rows - 1 are zeros
  int64_t zero_rows;
  int K, m, P, lk, xdt, rotated;
  float inv_sqrt_k;
  BucketJob bucket;  // with bucket.ids set, the workgroup after the last row sorts pairs
};

// NT threads per row; MAXK bounds K (registers per thread). Short rows take one wave each
// (NT = 64: the passes' barriers are a single wave's, and many rows are in flight per CU).
template <bool X32, int NT, int MAXK>
__global__ __launch_bounds__(NT) void k_rot16(Rot16Params p) {
  extern __shared__ uint32_t smem_r[];
  const int Q = (p.K + 31) / 32;
  uint32_t* xh = smem_r;                                     // Q * 20 words
  float* xf = reinterpret_cast<float*>(xh + Q * (kChunkHalves / 2));
  float* red = xf + padded_len(p.K);
  // with pairs to sort, workgroup 0 sorts them (dispatched first, it runs beside the
  // rotations) and row r is workgroup r + 1
  int64_t r = blockIdx.x + static_cast<int64_t>(blockIdx.y) * gridDim.x;
  if (p.bucket.ids) {
    if (r == 0) {  // uniform per workgroup
      int32_t* cnt = reinterpret_cast<int32_t*>(smem_r);
      bucket_pairs<NT>(p.bucket, cnt, cnt + (p.bucket.tiles ? 2 : 1) * p.bucket.E);
      return;
    }
    --r;
  }
  if (r >= p.nrows + p.zero_rows) return;  // uniform per workgroup
  if (r >= p.nrows) {
    uint4* dst = reinterpret_cast<uint4*>(p.out + r * rot16_row_halves(p.K));
    for (int i = threadIdx.x; i < Q * 4; i += NT) dst[i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) p.scale[r] = 0.f;
    return;
  }
  const int64_t src = p.rows ? p.rows[r] : r;
  InputLoad<X32, NT, MAXK> xin;
  xin.issue(p.x, p.xdt, src, p.K, p.rotated ? nullptr : p.signs);
  float out_scale;
  const bool rotated = p.rotated != 0;
  const float sc = xin.template finish_a<true>(xf, red, p.K, p.lk, p.P, rotated, p.inv_sqrt_k,
                                               &out_scale);
  xin.template finish_b<true>(xf, xh, p.K, p.m, p.P, rotated, sc);
  // copy the row out with 16-byte stores, dropping the 8 padding halves of every chunk
  uint4* dst = reinterpret_cast<uint4*>(p.out + r * rot16_row_halves(p.K));
  const uint4* srcv = reinterpret_cast<const uint4*>(xh);
  for (int i = threadIdx.x; i < Q * 4; i += NT)
    dst[i] = srcv[(i >> 2) * (kChunkHalves / 8) + (i & 3)];
  if (threadIdx.x == 0) p.scale[r] = out_scale;
}

// K up to this many elements take one wave per row
constexpr int kRotShortK = 2048;

// bucket_words: LDS words of the pair sort (0: none)
inline size_t rot16_lds_bytes(int K, int bucket_words) {
  const int Q = (K + 31) / 32;
  const size_t rot = static_cast<size_t>(Q) * kChunkHalves * 2 + padded_len(K) * 4 +
                     (kRotThreads / 64) * 4 + 16;
  const size_t bkt = bucket_words > 0 ? static_cast<size_t>(bucket_words + 2 * (kRotThreads / 64)) * 4 : 0;
  return rot > bkt ? rot : bkt;
}

}  // namespace tq
