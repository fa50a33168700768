// ExpertsInt8 quantizer (Jamba-1.5 paper, "Serving Considerations and
// Improvements": weights are quantized to INT8 when the model is loaded, in
// seconds, without calibration).
//
// Row-wise symmetric quantization, one scale per output channel:
//   a = max |w[r, :]|,  s = a / 127 rounded once, to nearest-even, into the
//   scale dtype,  q = round-half-even(w / s) clamped to [-127, 127];
//   an all-zero row stores s = 0 and q = 0.
// The rounding decisions are exact: a and w have at most 24 significant bits,
// so an fp64 quotient reaches a rounding midpoint only when the exact quotient
// is that midpoint, and rounding the fp64 value is rounding the exact one.
// The fp64 -> bf16 step is done on the bit pattern (round-to-nearest-even of
// the 45 dropped mantissa bits), with the subnormal bf16 grid (2^-133) handled
// separately.
//
// The FP8 comparator's quantizer is the same with OCP e4m3 codes: s = a / 448
// rounded once into the scale dtype, code = the e4m3 value nearest to w / s
// (ties to the even mantissa) saturated to +-448, encoded as its byte; a zero
// result is the canonical +0 byte. The e4m3 midpoints have at most 5
// significant bits, so the same exactness argument holds.
//
// Row-major codes: one workgroup per row: pass 1 reduces max|w| (16-byte
// loads, wave shuffles, then LDS across waves), pass 2 re-reads the row
// (mostly from L2) and writes 16 codes per 16-byte store. Codes in the tiled
// layout of the expert kernels: one workgroup per 16 rows (below).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kQuantThreads = 256;

// nearest bf16 value (ties to even) of a finite, non-negative fp64 value
__device__ __forceinline__ double round_f64_to_bf16(double v) {
  if (v < 0x1p-126) {
    return rint(v * 0x1p133) * 0x1p-133;  // subnormal bf16 grid, exact in fp64
  }
  uint64_t b = __double_as_longlong(v);
  const uint64_t lsb = (b >> 45) & 1ull;
  b += ((1ull << 44) - 1ull) + lsb;
  b &= ~((1ull << 45) - 1ull);
  return __longlong_as_double(b);
}

// byte of the e4m3 value nearest to r (ties to even), saturated to +-448.
// With a = |r| = m * 2^e (0.5 <= m < 1) the quantum of a's binade is 2^(e-4),
// never below the subnormal quantum 2^-9; a carry into the next binade gives
// its first value.
__device__ __forceinline__ uint32_t encode_e4m3(double r) {
  const double a = fabs(r);
  int e;
  (void)frexp(a, &e);
  const int step = max(e - 4, -9);
  double q = ldexp(rint(ldexp(a, -step)), step);
  q = fmin(q, 448.0);
  if (q == 0.0) return 0u;
  uint32_t code;
  if (q < 0x1p-6) {
    code = (uint32_t)(q * 0x1p9);                   // exponent field 0: q = M * 2^-9
  } else {
    int eq;
    (void)frexp(q, &eq);                            // q = (1 + M/8) * 2^(eq-1)
    const uint32_t M = (uint32_t)((ldexp(q, 1 - eq) - 1.0) * 8.0);
    code = ((uint32_t)(eq - 1 + 7) << 3) | M;
  }
  return r < 0.0 ? (code | 0x80u) : code;
}

template <bool kSrcBf16>
__device__ __forceinline__ void load16(const void* w, long idx, float (&v)[16]) {
  if constexpr (kSrcBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + idx);
    const uint4 u0 = p[0], u1 = p[1];
    const uint32_t u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  }
}

// Byte offset of the 16 codes of row `row`, columns c .. c+15 (c % 16 == 0):
// row-major, or the tiled layout (block (row/16, c/64) at block index
// (row/16)*(cols/64) + c/64, piece 16*(row%16) + 256*((c%64)/16) inside it).
template <bool kTiled>
__device__ __forceinline__ long code_offset(long row, int c, int cols) {
  if constexpr (kTiled) {
    return ((row >> 4) * (cols >> 6) + (c >> 6)) * 1024 + 256 * ((c & 63) >> 4) + 16 * (row & 15);
  } else {
    return row * cols + c;
  }
}

template <bool kSrcBf16, bool kScaleBf16, bool kFp8, bool kTiled>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(const void* __restrict__ w, int cols,
                                                                      int8_t* __restrict__ q, void* __restrict__ s) {
  __shared__ float wmax[kQuantThreads / kWave];
  const long row = blockIdx.x;
  const long base = row * cols;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  float m = 0.f;
  for (int c = threadIdx.x * 16; c < cols; c += kQuantThreads * 16) {
    float v[16];
    load16<kSrcBf16>(w, base + c, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  float a = wmax[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / kWave; ++i) a = fmaxf(a, wmax[i]);

  const double sd = (double)a / (kFp8 ? 448.0 : 127.0);
  double scale;
  if constexpr (kScaleBf16) {
    scale = round_f64_to_bf16(sd);
  } else {
    scale = (double)(float)sd;  // IEEE conversion: round to nearest even
  }
  if (threadIdx.x == 0) {
    if constexpr (kScaleBf16) {
      static_cast<uint16_t*>(s)[row] = (uint16_t)(__float_as_uint((float)scale) >> 16);
    } else {
      static_cast<float*>(s)[row] = (float)scale;
    }
  }

  for (int c = threadIdx.x * 16; c < cols; c += kQuantThreads * 16) {
    float v[16];
    load16<kSrcBf16>(w, base + c, v);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (scale > 0.0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t b;
        if constexpr (kFp8) {
          b = encode_e4m3((double)v[i] / scale);
        } else {
          double r = rint((double)v[i] / scale);
          r = fmin(fmax(r, -127.0), 127.0);
          b = (uint32_t)(uint8_t)(int8_t)(int)r;
        }
        packed[i >> 2] |= b << (8 * (i & 3));
      }
    }
    *reinterpret_cast<uint4*>(q + code_offset<kTiled>(row, c, cols)) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

// Tiled output: one workgroup per 16-row group (the rows of one row of
// blocks). Pass 1: wave w reduces max|w| of rows 4w .. 4w+3 and the 16 scales
// go through LDS. Pass 2: every store of a wave writes one whole 1 KiB block
// (lane l: row l%16, columns 16*(l/16) .. +16 of the block), read back from L2.
template <bool kSrcBf16, bool kScaleBf16, bool kFp8>
__global__ __launch_bounds__(kQuantThreads) void quantize_pack_kernel(const void* __restrict__ w, int cols,
                                                                      int8_t* __restrict__ q, void* __restrict__ s) {
  constexpr int kRowsPerWave = 16 / (kQuantThreads / kWave);
  __shared__ double scale_of[16];
  const long rg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const long row = rg * 16 + wave * kRowsPerWave + i;
    float m = 0.f;
    for (int c = lane * 16; c < cols; c += kWave * 16) {
      float v[16];
      load16<kSrcBf16>(w, row * cols + c, v);
#pragma unroll
      for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[k]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const double sd = (double)m / (kFp8 ? 448.0 : 127.0);
    double scale;
    if constexpr (kScaleBf16) {
      scale = round_f64_to_bf16(sd);
    } else {
      scale = (double)(float)sd;  // IEEE conversion: round to nearest even
    }
    if (lane == 0) {
      scale_of[wave * kRowsPerWave + i] = scale;
      if constexpr (kScaleBf16) {
        static_cast<uint16_t*>(s)[row] = (uint16_t)(__float_as_uint((float)scale) >> 16);
      } else {
        static_cast<float*>(s)[row] = (float)scale;
      }
    }
  }
  __syncthreads();
  const int r = lane & 15;
  const long row = rg * 16 + r;
  const double scale = scale_of[r];
  const int kblocks = cols >> 6;
  for (int ks = wave; ks < kblocks; ks += kQuantThreads / kWave) {
    const int c = ks * 64 + 16 * (lane >> 4);
    float v[16];
    load16<kSrcBf16>(w, row * cols + c, v);
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (scale > 0.0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t b;
        if constexpr (kFp8) {
          b = encode_e4m3((double)v[i] / scale);
        } else {
          double rr = rint((double)v[i] / scale);
          rr = fmin(fmax(rr, -127.0), 127.0);
          b = (uint32_t)(uint8_t)(int8_t)(int)rr;
        }
        packed[i >> 2] |= b << (8 * (i & 3));
      }
    }
    *reinterpret_cast<uint4*>(q + code_offset<true>(row, c, cols)) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
}

template <bool kFp8, bool kTiled>
hipError_t launch_quantize(int64_t rows, int cols, bool src_bf16, const void* w, bool scale_bf16, int8_t* q, void* s,
                           hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 block(kQuantThreads);
  if constexpr (kTiled) {
    const dim3 grid((unsigned)(rows / 16));
    if (src_bf16) {
      if (scale_bf16)
        hipLaunchKernelGGL((quantize_pack_kernel<true, true, kFp8>), grid, block, 0, stream, w, cols, q, s);
      else
        hipLaunchKernelGGL((quantize_pack_kernel<true, false, kFp8>), grid, block, 0, stream, w, cols, q, s);
    } else {
      if (scale_bf16)
        hipLaunchKernelGGL((quantize_pack_kernel<false, true, kFp8>), grid, block, 0, stream, w, cols, q, s);
      else
        hipLaunchKernelGGL((quantize_pack_kernel<false, false, kFp8>), grid, block, 0, stream, w, cols, q, s);
    }
    return hipGetLastError();
  }
  // grid.x is limited to 2^31-1; rows beyond that are rejected by the caller
  const dim3 grid((unsigned)rows);
  if (src_bf16) {
    if (scale_bf16)
      hipLaunchKernelGGL((quantize_rows_kernel<true, true, kFp8, false>), grid, block, 0, stream, w, cols, q, s);
    else
      hipLaunchKernelGGL((quantize_rows_kernel<true, false, kFp8, false>), grid, block, 0, stream, w, cols, q, s);
  } else {
    if (scale_bf16)
      hipLaunchKernelGGL((quantize_rows_kernel<false, true, kFp8, false>), grid, block, 0, stream, w, cols, q, s);
    else
      hipLaunchKernelGGL((quantize_rows_kernel<false, false, kFp8, false>), grid, block, 0, stream, w, cols, q, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(int64_t rows, int cols, bool src_bf16, const void* w, bool scale_bf16, int8_t* q,
                                void* s, bool fp8, bool tiled, hipStream_t stream) {
  if (tiled) {
    return fp8 ? launch_quantize<true, true>(rows, cols, src_bf16, w, scale_bf16, q, s, stream)
               : launch_quantize<false, true>(rows, cols, src_bf16, w, scale_bf16, q, s, stream);
  }
  return fp8 ? launch_quantize<true, false>(rows, cols, src_bf16, w, scale_bf16, q, s, stream)
             : launch_quantize<false, false>(rows, cols, src_bf16, w, scale_bf16, q, s, stream);
}

}  // namespace moe
