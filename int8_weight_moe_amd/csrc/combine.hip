// Weighted combine back to token order: y[t] = sum_k w[t,k] * y_rows[row(t,k)],
// k ascending, fp32 accumulation, one write per output element (no atomics,
// so the result is deterministic). Bound by HBM: K fp32 rows in, one row out.
// Workgroup (t, c): token t, columns 1024*c .. +1024, four per thread, so a
// decode batch of a few tokens still spreads over many workgroups.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 4;

template <bool kOutBf16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ y_rows,
                                                                  const int32_t* __restrict__ slot_to_row,
                                                                  const float* __restrict__ topk_w, int T, int d,
                                                                  int K, void* __restrict__ y) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * kCombineCols + threadIdx.x * 4;
  if (c >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      const int row = slot_to_row[(long)t * K + k];
      const float w = topk_w[(long)t * K + k];
      if (row >= 0) {
        const float4 v = *reinterpret_cast<const float4*>(y_rows + (long)row * d + c);
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
    }
  }
  if constexpr (kOutBf16) {
    bf16x4 o;
    o[0] = (__bf16)acc.x;
    o[1] = (__bf16)acc.y;
    o[2] = (__bf16)acc.z;
    o[3] = (__bf16)acc.w;
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(y) + (long)t * d + c) = o;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + (long)t * d + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_rows, const int32_t* slot_to_row, const float* topk_w, int T, int d,
                          int K, bool act_bf16, void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(T, (d + kCombineCols - 1) / kCombineCols);
  const dim3 block(kCombineThreads);
  if (act_bf16) {
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, y_rows, slot_to_row, topk_w, T, d, K, y);
  } else {
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, y_rows, slot_to_row, topk_w, T, d, K, y);
  }
  return hipGetLastError();
}

}  // namespace moe
