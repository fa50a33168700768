// Device-side helpers shared by the gfx950 kernels of libmoe_int8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// compile-time arguments for generic lambdas (select a specialised loop)
template <bool B>
struct bool_constant {
  static constexpr bool value = B;
};
template <int I>
struct int_constant {
  static constexpr int value = I;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 MFMA (gfx950). Operand lane layout: lane l supplies row
// (l % 16) of its operand with 8 reduction elements; lanes l/16 = 0..3 supply
// four disjoint groups of 8 along the reduction axis. Any consistent
// assignment of reduction indices to (lane group, element) works, because the
// instruction sums over all 32. Result: lane l holds C[4*(l/16) + i][l % 16],
// i = 0..3, where rows come from operand a and columns from operand b.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x4 fp32 MFMA: lane l supplies row (l % 16), reduction index (l / 16).
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- streaming loads
// 16-byte load marked non-temporal: weights are read once per launch, so they
// should not push reusable data (activations, scales) out of the caches.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- direct global->LDS loads
// One 16-byte-per-lane global->LDS load: lane l reads base + voff (its own
// 32-bit byte offset) and its 16 bytes land at LDS byte address lds + 16*l.
// Written as inline asm with no output register and a memory clobber: the
// compiler's own handling of these loads waits for all of them before every
// LDS read, which would drain the ring; here the only waits are the explicit
// vmcnt counts of the pipeline. m0 (the LDS base of the load) is set right
// before each load; nothing else in the FFN kernels uses m0. `base` and `lds`
// are wave-uniform.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory");
}

// LDS byte address of a __shared__ object: the low 32 bits of its generic
// address (the shared aperture base has zero low bits).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
  return (uint32_t)(uintptr_t)p;
}

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// operations are outstanding and all LDS operations have completed.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// ---------------------------------------------------------------- expert segment lookup
// Both lookups read the E+1 segment offsets once, one expert per lane (E <= 64),
// instead of walking the experts one dependent load at a time; every lane of
// the wave returns the same (wave-uniform) answer.

// Tiles of a grouped pass: the expert-grouped rows x output-channel tiles
// grid, where expert x owns ceil(count_x / BM) consecutive row tiles.
//   - The real tile count (row tiles x n_tiles) comes from the offsets. The
//     tiles are cut into 8 XCD queues, contiguous ranges of per_xcd tiles
//     (the count divided by the XCDs, rounded up to a multiple of `grain`), so
//     each XCD works on a contiguous range and keeps its operands in its own
//     L2 (sizing the queues by the grid, which is launched for the most row
//     tiles the slot count allows, left the last XCD idle for the tiles that
//     do not exist).
//   - Each expert's row tiles form groups of at most GM (GM_LONG for an
//     expert with at least 3*GM row tiles; as even as possible; no group spans
//     two experts), and a group takes every channel tile before the next
//     group, so a weight tile is read by all the row tiles of its group in a
//     row. (Groups of GM over all row tiles, which span expert boundaries and
//     then read two experts' weights, measured 1-1.5% slower on the Mini
//     prefill passes.)
// Per-workgroup view of that grid, one expert per lane.
struct TileGrid {
  int o0, o1, tiles, excl;   // lane x: expert x's rows [o0, o1), its row tiles, the row tiles before it
  int total, per_xcd;        // wave-uniform
};

template <int BM>
__device__ __forceinline__ TileGrid tile_grid(const int32_t* __restrict__ offsets, int E, int n_tiles_n, int xcds,
                                              int grain) {
  const int lane = threadIdx.x & (kWave - 1);
  TileGrid g;
  g.o0 = 0;
  g.o1 = 0;
  if (lane < E) {
    g.o0 = offsets[lane];
    g.o1 = offsets[lane + 1];
  }
  g.tiles = (g.o1 - g.o0 + BM - 1) / BM;
  int incl = g.tiles;   // inclusive scan of the tile counts over the lanes
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  g.excl = incl - g.tiles;
  g.total = __builtin_amdgcn_readlane(incl, kWave - 1) * n_tiles_n;
  g.per_xcd = ((g.total + xcds - 1) / xcds + grain - 1) / grain * grain;
  return g;
}

// Expert, first row, row count and channel tile of tile `tile` (0 <= tile < total):
// the expert owning it (expert x owns tiles [excl_x, excl_x + tiles_x) * n_tiles),
// then its balanced group of at most GM of that expert's row tiles:
// ceil(mt / GM) groups whose sizes differ by at most one, the larger first.
template <int BM, int GM, int GM_LONG = GM>
__device__ __forceinline__ void decode_tile(const TileGrid& g, int tile, int E, int n_tiles_n, int& e, int& row0,
                                            int& nrows, int& nt) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t hit = __ballot(lane < E && tile >= g.excl * n_tiles_n && tile < (g.excl + g.tiles) * n_tiles_n);
  const int x = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  const int mt_e = __shfl(g.tiles, x);
  const int local = tile - __shfl(g.excl, x) * n_tiles_n;
  const int gmax = (mt_e >= 3 * GM) ? GM_LONG : GM;   // experts with many row tiles: larger groups
  const int ngroups = (mt_e + gmax - 1) / gmax;
  const int gbase = mt_e / ngroups, gextra = mt_e - gbase * ngroups;
  const int big = (gbase + 1) * n_tiles_n;
  int start_m, gm, in_group;
  if (local < gextra * big) {
    const int gi = local / big;
    gm = gbase + 1;
    start_m = gi * gm;
    in_group = local - gi * big;
  } else {
    const int l2 = local - gextra * big;
    const int g2 = l2 / (gbase * n_tiles_n);
    gm = gbase;
    start_m = gextra * (gbase + 1) + g2 * gbase;
    in_group = l2 - g2 * gbase * n_tiles_n;
  }
  nt = __builtin_amdgcn_readfirstlane(in_group / gm);
  e = x;
  row0 = __builtin_amdgcn_readfirstlane(__shfl(g.o0, x) + (start_m + in_group % gm) * BM);
  nrows = __builtin_amdgcn_readfirstlane(min(BM, __shfl(g.o1, x) - row0));
}

// Static tile order: block b works on tile (b % xcds) * per_xcd + b / xcds, so
// workgroups, which are dealt to the XCDs in turn, take their XCD's queue in
// order. The grid must hold xcds * per_xcd blocks. -1 for blocks past the tiles.
__device__ __forceinline__ int static_tile(const TileGrid& g, int xcds) {
  const int k = blockIdx.x / xcds;
  if (k >= g.per_xcd) return -1;
  const int tile = (blockIdx.x % xcds) * g.per_xcd + k;
  return tile < g.total ? tile : -1;
}

// Claimed tail (load balance across XCDs that run at different speeds, and a
// less ragged end of the pass): the first len - P tiles of each XCD queue go
// statically to the workgroups of that XCD (block b takes tile
// x*per_xcd + b/xcds, x = b % xcds, for b/xcds < per_xcd - P), and the last P
// tiles of each queue form its tail, which the later blocks claim with one
// atomic increment of claims[x]: their own XCD's tail first, then the others'
// in turn, so an XCD that runs faster takes part of the slower ones' tails.
// Only the tail blocks pay for an atomic. Every tile is claimed exactly once
// (each claim sees the claims before it) as long as the tail blocks outnumber
// the tail tiles; blocks that find every tail claimed exit. claims[0..7] start
// at zero.
// Returns -1 for blocks without a tile. All threads of the block call it.
__device__ __forceinline__ int claimed_tail_tile(const TileGrid& g, int xcds, int P,
                                                 unsigned long long* __restrict__ claims, int* s_tile) {
  const int x = blockIdx.x % xcds, k = blockIdx.x / xcds;
  const int pre = max(0, g.per_xcd - P);   // static tiles of a full queue
  if (k < pre) {
    const int len = min(g.per_xcd, g.total - x * g.per_xcd);
    return k < len ? x * g.per_xcd + k : -1;
  }
  if (threadIdx.x == 0) {
    int t = -1;
    for (int i = 0; i < xcds && t < 0; ++i) {
      const int y = (x + i) % xcds;
      const int tail = min(g.per_xcd, g.total - y * g.per_xcd) - pre;
      if (tail <= 0) continue;
      const int j = (int)atomicAdd(&claims[y], 1ull);
      if (j < tail) t = y * g.per_xcd + pre + j;
    }
    *s_tile = t;
  }
  __syncthreads();
  return *s_tile;
}

// Tile of this workgroup in the static order (the decode of static_tile).
// Returns false for blocks past the real tiles.
template <int BM, int GM, int GM_LONG = GM>
__device__ __forceinline__ bool block_tile(const int32_t* __restrict__ offsets, int E, int n_tiles_n, int xcds,
                                           int grain, int& e, int& row0, int& nrows, int& nt) {
  const TileGrid g = tile_grid<BM>(offsets, E, n_tiles_n, xcds, grain);
  const int tile = static_tile(g, xcds);
  if (tile < 0) return false;
  decode_tile<BM, GM, GM_LONG>(g, tile, E, n_tiles_n, e, row0, nrows, nt);
  return true;
}

// The experts' row segments, one expert per lane (lanes >= E hold empty
// segments), and the mask of the experts that have rows.
struct ExpertSegments {
  int o0, o1;
  uint64_t touched;
};

__device__ __forceinline__ ExpertSegments load_segments(const int32_t* __restrict__ offsets, int E) {
  const int lane = threadIdx.x & (kWave - 1);
  ExpertSegments g{0, 0, 0};
  if (lane < E) {
    g.o0 = offsets[lane];
    g.o1 = offsets[lane + 1];
  }
  g.touched = __ballot(lane < E && g.o1 > g.o0);
  return g;
}

// The te-th expert (in index order) among those with at least one row: its
// index, first row and row count. Returns false when fewer experts have rows.
__device__ __forceinline__ bool touched_expert(const ExpertSegments& g, int te, int& e, int& row0, int& nrows) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const bool mine = (g.touched >> lane) & 1ull;
  const uint64_t hit = __ballot(mine && __popcll(g.touched & below) == te);
  if (hit == 0) return false;
  const int x = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
  e = x;
  row0 = __builtin_amdgcn_readfirstlane(__shfl(g.o0, x));
  nrows = __builtin_amdgcn_readfirstlane(__shfl(g.o1, x) - row0);
  return true;
}

__device__ __forceinline__ bool find_touched_expert(const int32_t* __restrict__ offsets, int E, int te, int& e,
                                                    int& row0, int& nrows) {
  return touched_expert(load_segments(offsets, E), te, e, row0, nrows);
}

// ---------------------------------------------------------------- permutation of at most 256 slots
// For S <= 64*kIdChunks slots one wave holds every expert id (chunk c, lane
// l: slot 64c + l; -1 past S), so a kernel can derive the permutation itself
// instead of reading it. It is the one the permutation kernel writes: experts
// in index order, slots ascending inside an expert, ids outside [0, E) not
// placed.
constexpr int kIdChunks = 4;

struct WaveIds {
  int id[kIdChunks];
  int chunks;   // ceil(S / 64)
};

__device__ __forceinline__ WaveIds load_wave_ids(const int32_t* __restrict__ ids, int S) {
  const int lane = threadIdx.x & (kWave - 1);
  WaveIds w;
  w.chunks = (S + kWave - 1) / kWave;
#pragma unroll
  for (int c = 0; c < kIdChunks; ++c) {
    const int sl = c * kWave + lane;
    w.id[c] = (c < w.chunks && sl < S) ? ids[sl] : -1;
  }
  return w;
}

// Position of the k-th (from 0) set bit of m; k < popcount(m).
__device__ __forceinline__ int select_bit(uint64_t m, int k) {
  for (int i = 0; i < k; ++i) m &= m - 1;
  return __ffsll((unsigned long long)m) - 1;
}

// The slots of expert x, one 64-slot chunk per mask; all lanes must call it
// (ballots).
__device__ __forceinline__ void expert_masks(const WaveIds& w, int x, uint64_t (&m)[kIdChunks]) {
#pragma unroll
  for (int c = 0; c < kIdChunks; ++c) m[c] = (c < w.chunks) ? __ballot(w.id[c] == x) : 0ull;
}

// The k-th (from 0) slot among the masks, k < their total popcount. Lane-local.
__device__ __forceinline__ int select_slot(const uint64_t (&m)[kIdChunks], int k) {
#pragma unroll
  for (int c = 0; c < kIdChunks; ++c) {
    const int n = __popcll(m[c]);
    if (k < n) return c * kWave + select_bit(m[c], k);
    k -= n;
  }
  return -1;
}

// The experts' row segments (as load_segments) from the wave's ids.
__device__ __forceinline__ ExpertSegments segments_from_ids(const WaveIds& w, int E) {
  const int lane = threadIdx.x & (kWave - 1);
  int cnt = 0;   // lane x: rows of expert x
  for (int x = 0; x < E; ++x) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < kIdChunks; ++c)
      if (c < w.chunks) n += __popcll(__ballot(w.id[c] == x));
    if (lane == x) cnt = n;
  }
  int incl = cnt;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int v = __shfl_up(incl, dd);
    if (lane >= dd) incl += v;
  }
  ExpertSegments g;
  g.o0 = incl - cnt;
  g.o1 = incl;
  g.touched = __ballot(lane < E && cnt > 0);
  return g;
}

// Writes the permutation (expert_offsets [E+1], sorted_slots [S],
// slot_to_row [S]) from the wave's ids and segments; one wave calls it.
__device__ __forceinline__ void write_permutation(const WaveIds& w, const ExpertSegments& g, int E, int S,
                                                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
                                                  int32_t* __restrict__ slot_to_row) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  if (lane < E) offsets[lane] = g.o0;
  const int total = __builtin_amdgcn_readlane(g.o1, E - 1);
  if (lane == 0) offsets[E] = total;
  int row[kIdChunks], slot[kIdChunks];
#pragma unroll
  for (int c = 0; c < kIdChunks; ++c) row[c] = slot[c] = -1;
  for (int x = 0; x < E; ++x) {
    const int lo = __builtin_amdgcn_readlane(g.o0, x), hi = __builtin_amdgcn_readlane(g.o1, x);
    uint64_t m[kIdChunks];
    expert_masks(w, x, m);
    int before = 0;   // rows of expert x in the chunks before c
#pragma unroll
    for (int c = 0; c < kIdChunks; ++c) {
      if (w.id[c] == x) row[c] = lo + before + __popcll(m[c] & below);
      before += __popcll(m[c]);
    }
#pragma unroll
    for (int c = 0; c < kIdChunks; ++c) {
      const int r = c * kWave + lane;   // sorted row held by this lane
      if (r >= lo && r < hi) slot[c] = select_slot(m, r - lo);
    }
  }
#pragma unroll
  for (int c = 0; c < kIdChunks; ++c) {
    const int sl = c * kWave + lane;
    if (c < w.chunks && sl < S) {
      slot_to_row[sl] = row[c];
      sorted_slots[sl] = slot[c];
    }
  }
}

// ---------------------------------------------------------------- conversions
// Eight int8 codes (two dwords, byte 0 first) -> eight bf16 values. Exact: a
// code has at most 8 significant bits. Compiles to one sign-extending
// byte->fp32 convert per code and one packed fp32->bf16 convert per pair.
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)(float)(int8_t)(lo >> (8 * i));
#pragma unroll
  for (int i = 0; i < 4; ++i) r[4 + i] = (__bf16)(float)(int8_t)(hi >> (8 * i));
  return r;
}

__device__ __forceinline__ bf16x8 f32x8_to_bf16(float4 a, float4 b) {
  bf16x8 r;
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Scale value of either dtype as fp32 (bf16 -> fp32 is exact).
template <bool kScaleBf16>
__device__ __forceinline__ float load_scale(const void* s, long idx) {
  if constexpr (kScaleBf16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s)[idx]);
  } else {
    return reinterpret_cast<const float*>(s)[idx];
  }
}

// Four consecutive scales (idx % 4 == 0) as fp32, one vector load.
template <bool kScaleBf16>
__device__ __forceinline__ float4 load_scale4(const void* s, long idx) {
  if constexpr (kScaleBf16) {
    const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(s) + idx);
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                       __uint_as_float(b.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s) + idx);
  }
}

// SiLU in fp32: z / (1 + exp(-z)), with the hardware reciprocal (about 1 ulp);
// the result is rounded to bf16 right after, so this costs no accuracy.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// ---------------------------------------------------------------- activation loads
// Sixteen consecutive activations starting at p, as two bf16x8 (elements 0-7, 8-15).
template <typename Act>
struct Act16;

template <>
struct Act16<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, bf16x8& a0, bf16x8& a1) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    a0 = as_bf16x8(q[0]);
    a1 = as_bf16x8(q[1]);
  }
};

template <>
struct Act16<float> {
  static __device__ __forceinline__ void load(const float* p, bf16x8& a0, bf16x8& a1) {
    const float4* q = reinterpret_cast<const float4*>(p);
    a0 = f32x8_to_bf16(q[0], q[1]);
    a1 = f32x8_to_bf16(q[2], q[3]);
  }
};

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return as_bf16x8(make_uint4(0, 0, 0, 0));
}

// Eight consecutive activations starting at p, as bf16x8.
__device__ __forceinline__ bf16x8 load_act8(const __bf16* p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ bf16x8 load_act8(const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
  return f32x8_to_bf16(q[0], q[1]);
}

// ---------------------------------------------------------------- weight encodings
// The FFN kernels read expert weights in the tiled layout of their bytes (the
// layout moe_pack_rows makes, applied to a row of 2*cols bytes for bf16): per
// 16-channel group and 64-wide reduction step a wave reads kPieces 1 KiB blocks,
// lane l taking the 16 bytes at 16*l of each (channel l%16). Each encoding
// turns a lane's pieces into the two bf16x8 MFMA operands of the step and says
// which reduction elements they hold: operand 0 holds elements
// kActLane*(l/16) + 0..7 of the step, operand 1 the same plus kActSecond.
enum WFmt : int { kWInt8 = 0, kWBf16 = 1, kWFp8 = 2 };

template <int F>
struct WFormat;

// int8 codes (ExpertsInt8), one scale per output channel. Byte j of a piece is
// reduction element 16*(l/16) + j.
template <>
struct WFormat<kWInt8> {
  static constexpr int kPieces = 1;
  static constexpr bool kScaled = true;
  static constexpr int kActLane = 16;
  static constexpr int kActSecond = 8;
  static __device__ __forceinline__ bf16x8 operand(const uint4 (&p)[1], int k) {
    return k == 0 ? i8x8_to_bf16(p[0].x, p[0].y) : i8x8_to_bf16(p[0].z, p[0].w);
  }
  static __device__ __forceinline__ void operands(const uint4 (&p)[1], bf16x8& w0, bf16x8& w1) {
    w0 = operand(p, 0);
    w1 = operand(p, 1);
  }
};

// bf16 weights as they are (the comparator without quantization): two pieces
// per step, piece h holding elements 32*h + 8*(l/16) + 0..7.
template <>
struct WFormat<kWBf16> {
  static constexpr int kPieces = 2;
  static constexpr bool kScaled = false;
  static constexpr int kActLane = 8;
  static constexpr int kActSecond = 32;
  static __device__ __forceinline__ bf16x8 operand(const uint4 (&p)[2], int k) { return as_bf16x8(p[k]); }
  static __device__ __forceinline__ void operands(const uint4 (&p)[2], bf16x8& w0, bf16x8& w1) {
    w0 = as_bf16x8(p[0]);
    w1 = as_bf16x8(p[1]);
  }
};

// OCP fp8 e4m3 codes, one scale per output channel; byte order as int8. Every
// e4m3 value is exact in bf16 (3 mantissa bits, exponents 2^-9..2^8), so the
// gfx950 packed convert with a unit scale is exact.
template <>
struct WFormat<kWFp8> {
  static constexpr int kPieces = 1;
  static constexpr bool kScaled = true;
  static constexpr int kActLane = 16;
  static constexpr int kActSecond = 8;
  static __device__ __forceinline__ bf16x8 fp8x8(uint32_t lo, uint32_t hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
  static __device__ __forceinline__ bf16x8 operand(const uint4 (&p)[1], int k) {
    return k == 0 ? fp8x8(p[0].x, p[0].y) : fp8x8(p[0].z, p[0].w);
  }
  static __device__ __forceinline__ void operands(const uint4 (&p)[1], bf16x8& w0, bf16x8& w1) {
    w0 = operand(p, 0);
    w1 = operand(p, 1);
  }
};

}  // namespace moe
