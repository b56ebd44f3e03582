// k_qmv instantiations for 4-bit codes.
#include "qmv_kernel.hpp"

namespace tq {

template hipError_t launch_qmv_l<16>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);

}  // namespace tq
