// Identity routing for the dense int8-weight MLP (an MLP layer is the MoE
// layer with one expert that every token uses with weight 1): expert_offsets
// = {0, T}, sorted_slots[r] = r, slot_to_row[s] = s, topk_w[s] = 1. Lets the
// dense path run the same expert kernels and combine without a router.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void dense_init_kernel(int T, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_slots,
                                                         int32_t* __restrict__ slot_to_row, float* __restrict__ w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) {
    sorted_slots[i] = i;
    slot_to_row[i] = i;
    w[i] = 1.0f;
  }
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
  }
}

}  // namespace

hipError_t launch_dense_init(int T, int32_t* offsets, int32_t* sorted_slots, int32_t* slot_to_row, float* w,
                             hipStream_t stream) {
  const int blocks = (T + 255) / 256;
  hipLaunchKernelGGL(dense_init_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, T, offsets,
                     sorted_slots, slot_to_row, w);
  return hipGetLastError();
}

}  // namespace moe
