// k_qmv instantiations for 2-bit codes.
#include "qmv_kernel.hpp"

namespace tq {

template hipError_t launch_qmv_l<4>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);

}  // namespace tq
