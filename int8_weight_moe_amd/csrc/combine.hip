// Weighted combine back to token order: y[t] = sum_k w[t,k] * y_rows[row(t,k)],
// k ascending, fp32 accumulation, one write per output element (no atomics,
// so the result is deterministic). Bound by HBM: K fp32 rows in, one row out.
// A workgroup handles 4 tokens with one wave each; lanes walk the row in
// 16-byte pieces.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kCombineWaves = 4;

template <bool kOutBf16>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(const float* __restrict__ y_rows,
                                                                        const int32_t* __restrict__ slot_to_row,
                                                                        const float* __restrict__ topk_w, int T,
                                                                        int d, int K, void* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[8];
  float w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      rows[k] = slot_to_row[(long)t * K + k];
      w[k] = topk_w[(long)t * K + k];
    }
  }
  for (int c = lane * 4; c < d; c += kWave * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && rows[k] >= 0) {
        const float4 v = *reinterpret_cast<const float4*>(y_rows + (long)rows[k] * d + c);
        acc.x += w[k] * v.x;
        acc.y += w[k] * v.y;
        acc.z += w[k] * v.z;
        acc.w += w[k] * v.w;
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
}

}  // namespace

hipError_t launch_combine(const float* y_rows, const int32_t* slot_to_row, const float* topk_w, int T, int d,
                          int K, bool act_bf16, void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kCombineWaves - 1) / kCombineWaves);
  const dim3 block(kCombineWaves * kWave);
  if (act_bf16) {
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, stream, y_rows, slot_to_row, topk_w, T, d, K, y);
  } else {
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, stream, y_rows, slot_to_row, topk_w, T, d, K, y);
  }
  return hipGetLastError();
}

}  // namespace moe
