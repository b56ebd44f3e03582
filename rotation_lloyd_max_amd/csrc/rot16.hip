// Launcher of k_rot16 (rot16.hpp): every input row rotated once into fp16.
#include "internal.hpp"
#include "rot16.hpp"

namespace tq {

hipError_t launch_rot16(const void* x, int xdt, const int32_t* rows, int64_t nrows,
                        int64_t zero_rows, const WeightArgs& w, bool x_rotated, _Float16* out,
                        float* scale, const BucketJob* bucket, hipStream_t s) {
  const int64_t total = nrows + zero_rows + (bucket ? 1 : 0);
  if (total == 0) return hipSuccess;
  Rot16Params p{};
  p.x = x; p.rows = rows; p.signs = w.signs; p.out = out; p.scale = scale;
  p.nrows = nrows; p.zero_rows = zero_rows;
  p.K = w.K; p.m = w.m; p.P = w.P; p.xdt = xdt; p.rotated = x_rotated ? 1 : 0;
  int lk = 0;
  while ((1 << lk) < w.K) ++lk;
  p.lk = lk;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  if (bucket) p.bucket = *bucket;
  const size_t lds =
      rot16_lds_bytes(w.K, bucket ? bucket->E * (bucket->tiles ? 2 : 1) : 0);
  const dim3 grid(static_cast<unsigned>(total < 65536 ? total : 65536),
                  static_cast<unsigned>((total + 65535) / 65536));
  // short rows take one wave each, unless the launch also sorts pairs (that workgroup
  // wants the full width)
  void (*kern)(Rot16Params) = nullptr;
  unsigned nt = kRotThreads;
  if (w.K <= kRotShortK && !bucket) {
    kern = xdt == 0 ? k_rot16<true, 64, kRotShortK> : k_rot16<false, 64, kRotShortK>;
    nt = 64;
  } else {
    kern = xdt == 0 ? k_rot16<true, kRotThreads, kMaxK> : k_rot16<false, kRotThreads, kMaxK>;
  }
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(nt), lds, s, p);
  return hipGetLastError();
}

}  // namespace tq
