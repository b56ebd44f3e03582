// qmv and gather_qmv: y = W R x with W decoded inline from packed codes (the kernel is in
// qmv_kernel.hpp; each code format is instantiated in its own translation unit).
#include "qmv_kernel.hpp"

namespace tq {

extern template hipError_t launch_qmv_l<16>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);
extern template hipError_t launch_qmv_l<8>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);
extern template hipError_t launch_qmv_l<4>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);
extern template hipError_t launch_qmv_l<3>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);

hipError_t launch_qmv(const WeightArgs& w, const int32_t* ids, int n, const void* x, int xdt,
                      bool x_rotated, void* y, int ydt, hipStream_t s, const WeightArgs* w2) {
  if (n == 0 || w.N == 0) return hipSuccess;
  // the kernel addresses one expert's codes with 32-bit byte offsets and 24-bit row indices
  if (static_cast<uint64_t>(w.N) * w.wpr * 4 > 0xffffffffull || w.N >= (1 << 24))
    return hipErrorInvalidValue;
  QmvParams p{};
  p.codes = w.codes; p.scales = w.scales; p.signs = w.signs; p.ids = ids;
  p.codes2 = w2 ? w2->codes : w.codes;
  p.scales2 = w2 ? w2->scales : w.scales;
  const int nw = w2 ? 2 : 1;
  p.x = x; p.y = y;
  p.K = w.K; p.N = w.N; p.E = w.E; p.wpr = w.wpr; p.group = w.group; p.m = w.m; p.P = w.P;
  p.xdt = xdt; p.ydt = ydt; p.rotated = x_rotated ? 1 : 0;
  p.inv_sqrt_k = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(w.K)));
  p.cb = *codebook_for(w.levels);
  switch (w.levels) {
    case 16: return launch_qmv_l<16>(p, n, nw, s);
    case 8: return launch_qmv_l<8>(p, n, nw, s);
    case 4: return launch_qmv_l<4>(p, n, nw, s);
    default: return launch_qmv_l<3>(p, n, nw, s);
  }
}

}  // namespace tq
