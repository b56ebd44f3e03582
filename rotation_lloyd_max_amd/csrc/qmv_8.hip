// k_qmv instantiations for 3-bit codes.
#include "qmv_kernel.hpp"

namespace tq {

template hipError_t launch_qmv_l<8>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);

}  // namespace tq
