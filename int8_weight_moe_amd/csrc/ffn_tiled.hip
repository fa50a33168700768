// Expert FFN, tiled MFMA schedule (many rows per expert: prefill).
//
// A grouped GEMM over the per-expert row segments produced by the permutation.
// One workgroup computes a BM x BN output tile of one expert:
//   gate/up pass: C = X_e (BM rows, gathered from x through sorted_slots)
//                 times [W_gate_e ; W_up_e] channels n0..n0+BN/2 of each,
//                 epilogue h = silu(s_g * g) * (s_u * u) -> bf16;
//   down pass:    C = H_e (BM rows of h) times W_down_e channels n0..n0+BN,
//                 epilogue y_rows = s_d * acc -> fp32.
// Per 64-wide reduction step the workgroup stages the activation tile (bf16)
// and the weight tile in LDS; the weight tile arrives as int8 (half the bytes
// of bf16 -- the ExpertsInt8 point) and is converted to bf16 exactly on its
// way into LDS, once per workgroup. The LDS tiles are double buffered, so the
// global loads of step k+1 are in flight while step k's MFMAs run; one barrier
// per step. Rows are 128 bytes in LDS with the 16-byte chunks XOR-swizzled by
// (row mod 8), so the fragment reads (16 rows at one chunk) and the tile writes
// are free of bank conflicts.
// Waves are arranged WM x WN; a wave owns (BM/WM) x (BN/WN) outputs and issues
// 16x16x32 bf16 MFMAs with the channels as MFMA rows and the tokens as MFMA
// columns, so each lane ends with 4 consecutive channels of one row.
// Tile order: row tiles are numbered expert by expert; tiles are visited in
// groups of GM consecutive row tiles, channel tile by channel tile inside a
// group, so the tiles that run together share GM activation tiles and a few
// weight tiles. Workgroup ids are spread so that each XCD (workgroups are dealt
// round-robin to the 8 XCDs) runs a contiguous range of that order and keeps
// its operands in its own L2.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;      // reduction step (elements)
constexpr int kChunks = kBK / 8;  // 16-byte bf16 chunks per LDS row
constexpr int kXcds = 8;

// Tile shape (compile-time; overridable for tuning builds).
#ifndef MOE_TILE_BM
#define MOE_TILE_BM 256
#endif
#ifndef MOE_TILE_BN
#define MOE_TILE_BN 256
#endif
#ifndef MOE_TILE_WM
#define MOE_TILE_WM 4
#endif
#ifndef MOE_TILE_WN
#define MOE_TILE_WN 2
#endif
#ifndef MOE_TILE_GM
#define MOE_TILE_GM 4
#endif

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

template <bool kGateUp, typename Act, bool kScaleBf16, int BM, int BN, int WM, int WN, int GM>
__global__ __launch_bounds__(WM * WN * kWave) void ffn_tiled_kernel(
    const Act* __restrict__ X, const int32_t* __restrict__ sorted_slots, int topk,
    const int8_t* __restrict__ W0, const int8_t* __restrict__ W1, const void* __restrict__ S0,
    const void* __restrict__ S1, const int32_t* __restrict__ offsets, int E, int N, int Kd, int n_tiles_n,
    int m_tiles, int total_blocks, void* __restrict__ out) {
  constexpr int NT = WM * WN * kWave;       // threads
  constexpr int TM = BM / WM;               // rows per wave
  constexpr int TN = BN / WN;               // effective columns per wave
  constexpr int MB = TM / 16;
  constexpr int NB = TN / 16;
  constexpr int A_CHUNKS = BM * kChunks / NT;        // 8-element chunks per thread per step
  constexpr int B_PIECES = BN * (kBK / 16) / NT;     // 16-byte int8 pieces per thread per step
  static_assert(A_CHUNKS * NT == BM * kChunks, "A tile split");
  static_assert(B_PIECES * NT == BN * (kBK / 16), "B tile split");
  static_assert(!kGateUp || (NB % 2 == 0), "gate/up pairs");
  constexpr int CH_TILE = kGateUp ? BN / 2 : BN;     // output channels per tile

  __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[2][BN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- XCD-contiguous tile id, then (expert, row tile, channel tile)
  const int per_xcd = total_blocks / kXcds;
  const int tile = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int group_tiles = GM * n_tiles_n;
  const int group = tile / group_tiles;
  const int in_group = tile - group * group_tiles;
  const int gm = min(GM, m_tiles - group * GM);   // row tiles in this (possibly last) group
  if (gm <= 0) return;
  const int mt_global = group * GM + in_group % gm;
  const int nt = in_group / gm;
  if (nt >= n_tiles_n) return;
  int e = -1, row0 = 0, nrows = 0;
  {
    int cum = 0;
    for (int x = 0; x < E; ++x) {
      const int o0 = offsets[x], o1 = offsets[x + 1];
      const int mt_e = (o1 - o0 + BM - 1) / BM;
      if (mt_global < cum + mt_e) {
        e = x;
        row0 = o0 + (mt_global - cum) * BM;
        nrows = min(BM, o1 - row0);
        break;
      }
      cum += mt_e;
    }
  }
  if (e < 0) return;
  const int n0 = nt * CH_TILE;

  // ---- global source pointers of this thread's pieces
  const Act* a_src[A_CHUNKS];
  bool a_ok[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * NT;
    const int r = c / kChunks;
    const int ck = c % kChunks;
    a_ok[i] = r < nrows;
    long src = 0;
    if (a_ok[i]) {
      if constexpr (kGateUp) {
        src = (long)(sorted_slots[row0 + r] / topk) * Kd;
      } else {
        src = (long)(row0 + r) * Kd;
      }
    }
    a_src[i] = X + src + ck * 8;
  }
  // Weight pieces: the tile's channels are BN/16 groups of 16, each one 1 KiB
  // block per step in the tiled layout; piece c = 64*j + l is lane l's 16 bytes
  // of block j (tile row 16*j + l%16, reduction bytes 16*(l/16)..+16).
  // Channels past N (last channel tile when N is not a tile multiple) load zeros.
  const int8_t* b_src[B_PIECES];
  bool b_ok[B_PIECES];
#pragma unroll
  for (int i = 0; i < B_PIECES; ++i) {
    const int c = tid + i * NT;
    const int j = c >> 6;
    const int l = c & 63;
    const int8_t* base;
    int chl;
    if constexpr (kGateUp) {
      base = (j < BN / 32) ? W0 : W1;
      chl = n0 + 16 * (j % (BN / 32));
    } else {
      base = W0;
      chl = n0 + 16 * j;
    }
    b_ok[i] = chl < N;
    const long group = ((long)e * N + (b_ok[i] ? chl : 0)) >> 4;
    b_src[i] = base + group * (long)(Kd / kBK) * 1024 + 16 * l;
  }

  // ---- register staging of one step
  uint4 a_reg[A_CHUNKS];
  uint4 b_reg[B_PIECES];
  auto gload = [&](int kt) {
    const long off = (long)kt * kBK;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      if (a_ok[i]) {
        if constexpr (sizeof(Act) == 2) {
          a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + off);
        } else {
          const float4* p = reinterpret_cast<const float4*>(a_src[i] + off);
          a_reg[i] = __builtin_bit_cast(uint4, f32x8_to_bf16(p[0], p[1]));
        }
      } else {
        a_reg[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PIECES; ++i)
      b_reg[i] = b_ok[i] ? load_nt16(b_src[i] + (long)kt * 1024) : make_uint4(0, 0, 0, 0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&As[buf][swz(c / kChunks, c % kChunks)]) = a_reg[i];
    }
#pragma unroll
    for (int i = 0; i < B_PIECES; ++i) {
      const int c = tid + i * NT;
      const int r = 16 * (c >> 6) + (c & 15);
      const int pc = (c & 63) >> 4;
      const bf16x8 lo = i8x8_to_bf16(b_reg[i].x, b_reg[i].y);
      const bf16x8 hi = i8x8_to_bf16(b_reg[i].z, b_reg[i].w);
      *reinterpret_cast<bf16x8*>(&Bs[buf][swz(r, 2 * pc)]) = lo;
      *reinterpret_cast<bf16x8*>(&Bs[buf][swz(r, 2 * pc + 1)]) = hi;
    }
  };

  // LDS row of the wave's channel block nb
  auto b_row = [&](int nb) {
    if constexpr (kGateUp) {
      constexpr int HALF = NB / 2;  // blocks per matrix in a wave
      const int mat = nb / HALF;
      return mat * (BN / 2) + wn * (HALF * 16) + (nb % HALF) * 16;
    } else {
      return wn * TN + nb * 16;
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kd / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ck = ks * 4 + lg;
      bf16x8 xf[MB];
      bf16x8 wf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        xf[i] = *reinterpret_cast<const bf16x8*>(&As[cur][swz(wm * TM + i * 16 + li, ck)]);
#pragma unroll
      for (int j = 0; j < NB; ++j) wf[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][swz(b_row(j) + li, ck)]);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma_bf16(wf[j], xf[i], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: acc[i][j] holds channels (block j) 4*lg + q, row wm*TM + i*16 + li
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = wm * TM + i * 16 + li;
    if (r >= nrows) continue;
    const long orow = (long)(row0 + r) * N;
    if constexpr (kGateUp) {
      constexpr int HALF = NB / 2;
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const int ch = n0 + wn * (HALF * 16) + j * 16 + 4 * lg;
        if (ch >= N) continue;
        bf16x4 hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = acc[i][j][q] * load_scale<kScaleBf16>(S0, (long)e * N + ch + q);
          const float u = acc[i][j + HALF][q] * load_scale<kScaleBf16>(S1, (long)e * N + ch + q);
          hv[q] = (__bf16)(silu(g) * u);
        }
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + orow + ch) = hv;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int ch = n0 + wn * TN + j * 16 + 4 * lg;
        if (ch >= N) continue;
        float4 yv;
        yv.x = acc[i][j][0] * load_scale<kScaleBf16>(S0, (long)e * N + ch + 0);
        yv.y = acc[i][j][1] * load_scale<kScaleBf16>(S0, (long)e * N + ch + 1);
        yv.z = acc[i][j][2] * load_scale<kScaleBf16>(S0, (long)e * N + ch + 2);
        yv.w = acc[i][j][3] * load_scale<kScaleBf16>(S0, (long)e * N + ch + 3);
        *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + ch) = yv;
      }
    }
  }
}

template <bool kGateUp, typename Act, bool kScaleBf16>
hipError_t launch_tiled_pass(const FfnArgs& a, hipStream_t stream) {
  constexpr int BM = MOE_TILE_BM, BN = MOE_TILE_BN, WM = MOE_TILE_WM, WN = MOE_TILE_WN, GM = MOE_TILE_GM;
  constexpr int CH_TILE = kGateUp ? BN / 2 : BN;
  const int N = kGateUp ? a.f : a.d;
  const int Kd = kGateUp ? a.d : a.f;
  const int n_tiles_n = (N + CH_TILE - 1) / CH_TILE;
  // row tiles: at most one partial tile per expert beyond S / BM
  const long m_tiles_max = (long)(a.S + BM - 1) / BM + a.E;
  long blocks = m_tiles_max * n_tiles_n;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)blocks);
  const dim3 block(WM * WN * kWave);
  if constexpr (kGateUp) {
    hipLaunchKernelGGL((ffn_tiled_kernel<true, Act, kScaleBf16, BM, BN, WM, WN, GM>), grid, block, 0, stream,
                       static_cast<const Act*>(a.x), a.sorted_slots, a.K, a.w_gate, a.w_up, a.s_gate, a.s_up,
                       a.offsets, a.E, N, Kd, n_tiles_n, (int)m_tiles_max, (int)blocks, static_cast<void*>(a.h));
  } else {
    hipLaunchKernelGGL((ffn_tiled_kernel<false, __bf16, kScaleBf16, BM, BN, WM, WN, GM>), grid, block, 0, stream,
                       static_cast<const __bf16*>(a.h), a.sorted_slots, a.K, a.w_down, nullptr, a.s_down, nullptr,
                       a.offsets, a.E, N, Kd, n_tiles_n, (int)m_tiles_max, (int)blocks, static_cast<void*>(a.y_rows));
  }
  return hipGetLastError();
}

template <bool kGateUp>
hipError_t dispatch_tiled(const FfnArgs& a, hipStream_t stream) {
  if (a.act_bf16) {
    return a.scale_bf16 ? launch_tiled_pass<kGateUp, __bf16, true>(a, stream)
                        : launch_tiled_pass<kGateUp, __bf16, false>(a, stream);
  }
  return a.scale_bf16 ? launch_tiled_pass<kGateUp, float, true>(a, stream)
                      : launch_tiled_pass<kGateUp, float, false>(a, stream);
}

}  // namespace

hipError_t launch_tiled_gate_up(const FfnArgs& a, hipStream_t stream) { return dispatch_tiled<true>(a, stream); }
hipError_t launch_tiled_down(const FfnArgs& a, hipStream_t stream) { return dispatch_tiled<false>(a, stream); }

}  // namespace moe
