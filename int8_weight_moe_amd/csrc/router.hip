// Router and top-K gate (Jamba-1.5 paper, "Model Architecture": a router picks
// the top K of n experts for every token).
//
// One workgroup scores 16 tokens against every expert (one token when the
// batch has at most 64, so that more CUs share the reads: mini-decode 10.3 ->
// 7.5 us, large-decode 17.4 -> 11.8 us). The 16 waves split the
// hidden dimension (so even a decode batch of a few tokens keeps many waves
// loading in parallel), each accumulating a 16x16 logit tile per block of 16
// experts with MFMA (bf16 inputs: 16x16x32 bf16, products exact, fp32 sums;
// fp32 inputs: 16x16x4 fp32). The partial tiles are summed through LDS in a
// fixed wave order, so the logits do not depend on scheduling. Then each wave
// takes one token: lane e holds logit e, K rounds of a wavefront argmax
// (ties to the lower expert index) pick the experts, and the gate weights are
// the softmax renormalised over the chosen set,
//   w_k = exp(l_k - l_max) / sum_j exp(l_j - l_max).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kRouterWaves = 16;
constexpr int kRouterTokens = 16;
constexpr int kMaxExperts = 64;
// batches of at most SMALL_T tokens are scored SMALL_TPW tokens per workgroup
#ifndef MOE_ROUTER_SMALL_T
#define MOE_ROUTER_SMALL_T 64
#endif
#ifndef MOE_ROUTER_SMALL_TPW
#define MOE_ROUTER_SMALL_TPW 1
#endif
static_assert(MOE_ROUTER_SMALL_TPW >= 1 && MOE_ROUTER_SMALL_TPW <= kRouterTokens, "tokens per workgroup");

// Eight consecutive elements of row `row` of a [rows, d] tensor at column kk,
// as bf16 (the MFMA input; fp32 inputs are rounded) or as fp32.
__device__ __forceinline__ bf16x8 load8(const __bf16* p) { return as_bf16x8(*reinterpret_cast<const uint4*>(p)); }

// Partial logits of one wave: for the 32-wide chunks c = wave, wave + 16, ...
// of the hidden dimension, the U chunks of a batch are all loaded before any
// of them is used, so a decode batch (a few tokens: two workgroups in all)
// keeps U loads in flight per operand instead of one.
template <typename Act, int EB>
__device__ __forceinline__ void router_accumulate(const Act* __restrict__ x, const Act* __restrict__ wr,
                                                  int T, int d, int E, int tok0, int tpw, int wave, int lane,
                                                  f32x4 (&acc)[4]) {
  constexpr int U = (sizeof(Act) == 2 ? 8 : 4) / EB > 0 ? (sizeof(Act) == 2 ? 8 : 4) / EB : 1;
  const int i = lane & 15;
  const int g = lane >> 4;
  const int tok = tok0 + i;
  const bool tok_ok = i < tpw && tok < T;
  const int nchunks = d >> 5;  // 32 reduction elements per chunk
  for (int c0 = wave; c0 < nchunks; c0 += kRouterWaves * U) {
    if constexpr (sizeof(Act) == 2) {
      bf16x8 a[U], b[U][EB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kRouterWaves;
        const int kk = c * 32 + 8 * g;
        const bool ok = c < nchunks;
        a[u] = (ok && tok_ok) ? load8(x + (long)tok * d + kk) : zero_bf16x8();
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          const int e = eb * 16 + i;
          b[u][eb] = (ok && e < E) ? load8(wr + (long)e * d + kk) : zero_bf16x8();
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) acc[eb] = mfma_bf16(a[u], b[u][eb], acc[eb]);
    } else {
      float4 a[U][2], b[U][EB][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kRouterWaves;
        const int kk = c * 32 + 8 * g;
        const bool ok = c < nchunks;
        a[u][0] = a[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok && tok_ok) {
          const float4* q = reinterpret_cast<const float4*>(x + (long)tok * d + kk);
          a[u][0] = q[0];
          a[u][1] = q[1];
        }
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          const int e = eb * 16 + i;
          b[u][eb][0] = b[u][eb][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (ok && e < E) {
            const float4* q = reinterpret_cast<const float4*>(wr + (long)e * d + kk);
            b[u][eb][0] = q[0];
            b[u][eb][1] = q[1];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float av[8] = {a[u][0].x, a[u][0].y, a[u][0].z, a[u][0].w, a[u][1].x, a[u][1].y, a[u][1].z, a[u][1].w};
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          const float bv[8] = {b[u][eb][0].x, b[u][eb][0].y, b[u][eb][0].z, b[u][eb][0].w,
                               b[u][eb][1].x, b[u][eb][1].y, b[u][eb][1].z, b[u][eb][1].w};
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[eb] = mfma_f32(av[j], bv[j], acc[eb]);
        }
      }
    }
  }
}

// argmax over the wavefront of (value, index); ties to the lower index.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(idx, off);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
}

// A workgroup scores tpw <= 16 tokens (the MFMA tile keeps 16 rows; rows past
// tpw stay zero). Small batches take fewer tokens per workgroup so more CUs
// share the router-weight reads; a token's logits do not depend on tpw.
template <typename Act, int EB>
__global__ __launch_bounds__(kRouterWaves * kWave) void router_topk_kernel(
    const Act* __restrict__ x, const Act* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int K, int tpw, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  __shared__ float red[kRouterWaves][kRouterTokens][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * tpw;

  f32x4 acc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
  router_accumulate<Act, EB>(x, wr, T, d, E, tok0, tpw, wave, lane, acc);

  // C[token 4*(l/16)+r][expert 16*eb + l%16]
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) {
    if (eb < EB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * (lane >> 4) + r][eb * 16 + (lane & 15)] = acc[eb][r];
    }
  }
  __syncthreads();

  for (int tl = wave; tl < tpw; tl += kRouterWaves) {
    const int t = tok0 + tl;
    if (t >= T) break;
    float l = -INFINITY;
    if (lane < E) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kRouterWaves; ++w) s += red[w][tl][lane];
      if (bias) s += bias[lane];
      l = s;
    }
    float v = l;
    float top = 0.f;
    float den = 0.f;
    float my_e = 0.f;   // this lane's exp(l_k - l_max) when lane == k
    int my_id = 0;
    bool chosen = false;
    for (int k = 0; k < K; ++k) {
      float bv = chosen ? -INFINITY : v;
      int bi = lane;
      wave_argmax(bv, bi);
      if (k == 0) top = bv;
      const float ek = __expf(bv - top);
      den += ek;
      if (lane == bi) chosen = true;
      if (lane == k) {
        my_e = ek;
        my_id = bi;
      }
    }
    if (lane < K) {
      topk_ids[(long)t * K + lane] = my_id;
      topk_w[(long)t * K + lane] = my_e / den;
    }
  }
}

template <typename Act, int EB>
void launch_router_eb(const void* x, const void* router_w, const float* bias, int T, int d, int E, int K,
                      int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  const int tpw = T <= MOE_ROUTER_SMALL_T ? MOE_ROUTER_SMALL_TPW : kRouterTokens;
  const dim3 grid((T + tpw - 1) / tpw);
  const dim3 block(kRouterWaves * kWave);
  hipLaunchKernelGGL((router_topk_kernel<Act, EB>), grid, block, 0, stream, static_cast<const Act*>(x),
                     static_cast<const Act*>(router_w), bias, T, d, E, K, tpw, topk_ids, topk_w);
}

template <typename Act>
void launch_router_act(const void* x, const void* router_w, const float* bias, int T, int d, int E, int K,
                       int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  if (E <= 16) {
    launch_router_eb<Act, 1>(x, router_w, bias, T, d, E, K, topk_ids, topk_w, stream);
  } else if (E <= 32) {
    launch_router_eb<Act, 2>(x, router_w, bias, T, d, E, K, topk_ids, topk_w, stream);
  } else {
    launch_router_eb<Act, 4>(x, router_w, bias, T, d, E, K, topk_ids, topk_w, stream);
  }
}

}  // namespace

hipError_t launch_router(const void* x, const void* router_w, const float* bias, int T, int d, int E, int K,
                         bool act_bf16, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (act_bf16) {
    launch_router_act<__bf16>(x, router_w, bias, T, d, E, K, topk_ids, topk_w, stream);
  } else {
    launch_router_act<float>(x, router_w, bias, T, d, E, K, topk_ids, topk_w, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
