// Slot ids of an expert-cache fetch (tq_expert_cache_fetch) written to device memory by a
// kernel that receives them as launch arguments: the host array they come from may change
// as soon as the call returns, while a copy from it would run later.
#include "internal.hpp"

namespace tq {

__global__ void k_put_ids(SlotIds ids, int32_t* dst) {
  for (int k = threadIdx.x; k < ids.n; k += blockDim.x) dst[k] = ids.v[k];
}

hipError_t launch_put_ids(const SlotIds& ids, int32_t* dst, hipStream_t s) {
  if (ids.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_put_ids, dim3(1), dim3(256), 0, s, ids, dst);
  return hipGetLastError();
}

}  // namespace tq
