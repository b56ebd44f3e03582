// k_qmv instantiations for trit words.
#include "qmv_kernel.hpp"

namespace tq {

template hipError_t launch_qmv_l<3>(QmvParams& p, int n_slots, int n_weights, hipStream_t s);

}  // namespace tq
