// Declarations shared by the host entry points (tq_api.cpp) and the kernel launchers
// (*.hip). Nothing here is part of the public interface in include/tq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// A codebook as the kernels see it: centroids and thresholds in binary32, centroids also
// as fp16 bit patterns (for the packed-fp16 decode tables). Passed by value.
struct CodebookArgs {
  float c[16];
  float t[15];
  uint16_t h[16];
  int levels;
};

// Lloyd-Max codebook for `levels` in {3, 4, 8, 16}; nullptr otherwise.
const CodebookArgs* codebook_for(int levels);

// The 256-level codebook (8-bit codes of KV-cache rows), binary32 and fp16.
struct BigCodebook {
  float c[256];
  float t[255];
  uint16_t h[256];
};
const BigCodebook* codebook256();

// K = m * P with m in {1, 12, 20, 28}, P a power of two.
bool split_dim(int64_t K, int* m, int* P);

// Everything a qmv-family launch needs about the weight, resolved on the host.
struct WeightArgs {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint32_t* signs;
  int levels, group, K, N, E, wpr, m, P;
};

hipError_t launch_signs(uint64_t seed, int K, uint32_t* bits, hipStream_t s);

// out[r] = R x[r]; `signbits` (device) or, when null, signs computed from `seed`.
hipError_t launch_fwht(const void* x, int xdt, int64_t rows, int K, int m, int P,
                       const uint32_t* signbits, uint64_t seed, void* out, int odt,
                       hipStream_t s);

hipError_t launch_encode(const void* W, int wdt, int64_t rows, int K, int m, int P,
                         int levels, int group, uint64_t seed, uint32_t* codes,
                         uint16_t* scales, hipStream_t s);
// Encode of rows already rotated (fp64): group RMS, fp16 scale, snap, pack.
hipError_t launch_encode_rotated(const double* V, int64_t rows, int K, int levels, int group,
                                 uint32_t* codes, uint16_t* scales, hipStream_t s);
// out = x R^T (dense rotation, fp64 matrix cores); odt 3 = fp64 output.
hipError_t launch_dense_rot(const void* x, int xdt, int64_t rows, int K, const float* R, void* out,
                            int odt, hipStream_t s);

// The register-resident encode for K = 2^p, 64 <= K <= 4096 (W 16-byte aligned).
// rows of m * 2^k (m = 12, 20, 28; 32 <= 2^k <= 256) with the rotation in registers
bool encode_m_supported(int K, int m);
hipError_t launch_encode_m(const void* W, int wdt, int64_t rows, int K, int m, int levels,
                           int group, uint64_t seed, uint32_t* codes, uint16_t* scales,
                           hipStream_t s);
bool encode_p2_supported(int K, int m, int levels);
hipError_t launch_encode_p2(const void* W, int wdt, int64_t rows, int K, int levels, int group,
                            uint64_t seed, uint32_t* codes, uint16_t* scales, hipStream_t s);

// qmv (ids == nullptr, n = 1) and gather_qmv.
// out[k] = decoded weights of expert ids[k] (k when ids is null) in the rotated basis.
hipError_t launch_dequant(const WeightArgs& w, const int32_t* ids, int n, void* out, int odt,
                          hipStream_t s);

// With w2 (same format, shape and experts as w, rotated alike), 2n slots: slot k < n
// reads w at ids[k], slot n + k reads w2 at ids[k]; y holds 2n rows.
hipError_t launch_qmv(const WeightArgs& w, const int32_t* ids, int n, const void* x, int xdt,
                      bool x_rotated, void* y, int ydt, hipStream_t s,
                      const WeightArgs* w2 = nullptr);

// Rotate nrows input rows (input row rows[r], or r when rows is null) into fp16 rows in
// the layout of rot16.hpp, then write zero_rows rows of zeros after them; with a bucket job
// (bucket.hpp), one more workgroup of the same launch sorts the pairs by expert.
struct BucketJob;
hipError_t launch_rot16(const void* x, int xdt, const int32_t* rows, int64_t nrows,
                        int64_t zero_rows, const WeightArgs& w, bool x_rotated, _Float16* out,
                        float* scale, const BucketJob* bucket, hipStream_t s);
size_t multi_gather_workspace(const WeightArgs& w, int64_t P);
// The fixed per-GPU workspace of tq_multi_gather_qmv_static (device address on the current
// device, resolved once per device).
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
hipError_t static_scratch(void** ptr);
// With w2 (same format, shape and experts as w, rotated alike): both weights over the same
// pairs, one rotation and one bucketing; y holds 2P rows (w2's from row P).
hipError_t launch_multi_gather(const WeightArgs& w, const int32_t* ids, int64_t P,
                               const void* x, int xdt, bool x_rotated, void* y, int ydt,
                               void* ws, hipStream_t s, const WeightArgs* w2 = nullptr);

size_t gather_qmm_workspace(const WeightArgs& w, int64_t M, int64_t T);
// With w2 (same format, shape and experts as w, rotated alike): y holds 2M rows, w2's
// from row M; the rows are rotated and the tiles scheduled once.
hipError_t launch_gather_qmm(const WeightArgs& w, const void* x, int xdt, int64_t T,
                             const int32_t* row_token, const int32_t* offsets, int64_t M,
                             bool x_rotated, void* y, int ydt, void* ws, hipStream_t s,
                             const WeightArgs* w2 = nullptr);

// KV-cache fetch: out[r] = R^T (c[idx] * scale) for `rows` rows of a power-of-two K <= 2048.
bool kv_fetch_supported(int K, int levels);
hipError_t launch_kv_fetch(const WeightArgs& w, int64_t rows, void* out, int odt, hipStream_t s);

// Up to kMaxSlotIds int32 values passed by value to a kernel (tq_expert_cache_fetch).
constexpr int kMaxSlotIds = 512;
struct SlotIds {
  int32_t n;
  int32_t v[kMaxSlotIds];
};
hipError_t launch_put_ids(const SlotIds& ids, int32_t* dst, hipStream_t s);

}  // namespace tq
