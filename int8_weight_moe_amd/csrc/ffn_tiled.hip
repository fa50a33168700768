// Expert FFN, tiled MFMA schedule (many rows per expert: prefill).
//
// A grouped GEMM over the per-expert row segments produced by the permutation.
// One workgroup computes a BM x BN output tile of one expert:
//   gate/up pass: C = X_e (BM rows, gathered from x through sorted_slots)
//                 times [W_gate_e ; W_up_e] channels n0..n0+BN/2 of each,
//                 epilogue h = silu(s_g * g) * (s_u * u) -> bf16;
//   down pass:    C = H_e (BM rows of h) times W_down_e channels n0..n0+BN,
//                 epilogue y_rows = s_d * acc -> fp32.
// Two kernels: the register-staged one below (fp32 activations, or tensors
// past 32-bit byte offsets) and the direct-to-LDS one after it (bf16
// activations: every prefill workload). In the register-staged kernel, per
// 64-wide reduction step the workgroup stages the activation tile (bf16) and
// the weight tile in LDS; the weight tile arrives as int8 (half the bytes of
// bf16 -- the ExpertsInt8 point) and is converted to bf16 exactly on its way
// into LDS, once per workgroup. The LDS tiles are double buffered, so the
// global loads of step k+1 are in flight while step k's MFMAs run; one barrier
// per step. Rows are 128 bytes in LDS with the 16-byte chunks XOR-swizzled by
// (row mod 8), so the fragment reads (16 rows at one chunk) and the tile writes
// are free of bank conflicts.
// Waves are arranged WM x WN; a wave owns (BM/WM) x (BN/WN) outputs and issues
// 16x16x32 bf16 MFMAs with the channels as MFMA rows and the tokens as MFMA
// columns, so each lane ends with 4 consecutive channels of one row.
// Tile order: row tiles are numbered expert by expert; each expert's row
// tiles are visited in groups of at most GM, channel tile by channel tile
// inside a group, so the tiles that run together share a few activation tiles
// and weight tiles of one expert. That order is cut into 8 contiguous XCD
// queues of equal length (workgroups are dealt round-robin to the 8 XCDs), so
// each XCD keeps its operands in its own L2. Workgroup ids map to the queues
// statically; with tile claim words (a workspace), the last tiles of each
// queue are claimed with atomics instead, by the later workgroups of any XCD,
// so XCDs that run faster (the same tiles took up to 5% longer on some XCDs
// than on others) take part of the slower ones' tails.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;      // reduction step (elements)
constexpr int kChunks = kBK / 8;  // 16-byte bf16 chunks per LDS row
constexpr int kXcds = 8;

// Tiles at the end of each XCD queue that are claimed instead of assigned
// statically (about two rounds of the XCD's 64 workgroup slots). A/B on one box
// against the static order: Large prefill skewed gate/up 2.1% and down 2.6%
// faster with 128 (256: the same; 64: 0.6% and 2.2%), Mini prefill 0.6-1.2%;
// claiming every tile instead cost gate/up 1-3% (an atomic at every
// workgroup start) and, with thieves taking the front of other queues, L2
// locality.
constexpr int kClaimTail = 128;

// Granularity of the XCD shares of a pass's tiles. Gate/up: exact shares
// (balanced to a tile). Down: whole multiples of the channel-tile count, which
// on the Large prefill shapes measured 2% faster than exact shares (11.03-11.08
// against 11.26-11.28 ms) and the same on the Mini ones; exact shares measured
// 1-2% faster for gate/up.
__host__ __device__ constexpr int xcd_grain(bool gate_up, int n_tiles_n) { return gate_up ? 1 : n_tiles_n; }

// Blocks a tiled pass launches: room for the largest XCD share of the most row
// tiles S slots can make (at most one partial tile per expert beyond S / BM);
// blocks past the real tiles exit at once.
long tiled_grid_blocks(bool gate_up, long m_tiles_max, int n_tiles_n) {
  const long total = m_tiles_max * n_tiles_n;
  const long g = xcd_grain(gate_up, n_tiles_n);
  const long per_xcd = ((total + kXcds - 1) / kXcds + g - 1) / g * g;
  return per_xcd * kXcds;
}

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
// row tiles per group of the direct-to-LDS gate/up pass: its weight tiles
// (two matrices) are the larger operand, so larger groups read them fewer
// times (Mini prefill gate/up, interleaved A/B on one box: groups of 8
// 3321-3333 us, of 6 3361-3369, of 4 3434-3466; on another 3336-3341 against
// 3444-3512; dense MLP prefill 0.5-1.5% faster, Large skewed within 0.5%);
// the down pass keeps 4 (8 measured 1-2% slower on Large skewed, 2 6%). An
// expert with at least 3*8 row tiles takes gate/up groups of up to 12 (Large
// skewed's two hot experts, 52 row tiles, in 5 groups: with the claimed queue
// tails, gate/up 0.9-1.4% faster than groups of up to 16 and than 8, A/B on one
// box; 16 had measured 0.5-1% faster than 8 with a fully static order)
#ifndef MOE_TILE_GM_GU
#define MOE_TILE_GM_GU 8
#endif
#ifndef MOE_TILE_GM_GU_LONG
#define MOE_TILE_GM_GU_LONG 12
#endif
// bf16 activations use the direct-to-LDS kernel below (1) or the register-staged one (0)
#ifndef MOE_TILE_DMA
#define MOE_TILE_DMA 1
#endif

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

template <bool kGateUp, typename Act, bool kScaleBf16, int BM, int BN, int WM, int WN, int GM>
__global__ __launch_bounds__(WM * WN * kWave) void ffn_tiled_kernel(
    const Act* __restrict__ X, const int32_t* __restrict__ sorted_slots, int topk,
    const int8_t* __restrict__ W0, const int8_t* __restrict__ W1, const void* __restrict__ S0,
    const void* __restrict__ S1, const int32_t* __restrict__ offsets, int E, int N, int Kd, int n_tiles_n,
    void* __restrict__ out) {
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

  // ---- XCD-contiguous tile: (expert, row tile, channel tile)
  int e, row0, nrows, nt;
  if (!block_tile<BM, GM>(offsets, E, n_tiles_n, kXcds, xcd_grain(kGateUp, n_tiles_n), e, row0, nrows, nt)) return;
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
        const float4 sg = load_scale4<kScaleBf16>(S0, (long)e * N + ch);
        const float4 su = load_scale4<kScaleBf16>(S1, (long)e * N + ch);
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
        bf16x4 hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = (__bf16)(silu(acc[i][j][q] * sgv[q]) * (acc[i][j + HALF][q] * suv[q]));
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + orow + ch) = hv;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int ch = n0 + wn * TN + j * 16 + 4 * lg;
        if (ch >= N) continue;
        const float4 sd = load_scale4<kScaleBf16>(S0, (long)e * N + ch);
        const float4 yv = make_float4(acc[i][j][0] * sd.x, acc[i][j][1] * sd.y, acc[i][j][2] * sd.z, acc[i][j][3] * sd.w);
        *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + ch) = yv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16-activation kernel (the one prefill runs): operands reach LDS by direct
// global->LDS loads.
//
// Same tile order as above; the tile is BM x BN = 128 x 256 (gate/up: 128
// channels of each matrix) over WM x WN = 1 x 4 waves, so a wave owns all 128
// rows and 64 of the columns and no weight fragment is read by two waves.
// Nothing is staged in registers: each wave issues 16-byte global_load_lds
// instructions that write a contiguous 1 KiB of LDS. A STAGES-deep LDS ring
// (2: 64 KiB, so two workgroups share a CU) keeps the loads of the next step
// in flight while one is computed (per step: wait for this step's loads with
// an explicit vmcnt, one barrier, issue the step STAGES-1 ahead, compute).
//   activations: BM rows x 128 bytes per step; instruction c of the tile
//     covers rows 8c..8c+7, lane l writes row 8c + l/8, 16-byte chunk l%8,
//     and fetches the logical chunk (l%8) ^ (row%8) -- so the tile lands in LDS
//     already XOR-swizzled and the fragment reads stay conflict-free;
//   weights: the tiled layout is copied block for block (1 KiB per 16-channel
//     group and step; two blocks for the bf16 comparator) and stays in its
//     encoding in LDS (int8: half the bytes of bf16); a lane reads one 16-byte
//     piece per block and converts it in registers into the step's two MFMA
//     operands (WFormat).
// Rows past the expert's segment and channels past N load valid in-range
// data whose results are never stored.
// (dma16, lds_addr and waitcnt_vm_lgkm0 are in device_common.h)

// Shape of the direct-to-LDS kernel: BM x BN tile, WM x WN waves, STAGES-deep ring.
#ifndef MOE_DMA_BM
#define MOE_DMA_BM 128
#endif
#ifndef MOE_DMA_BN
#define MOE_DMA_BN 256
#endif
#ifndef MOE_DMA_WM
#define MOE_DMA_WM 1
#endif
#ifndef MOE_DMA_WN
#define MOE_DMA_WN 4
#endif
#ifndef MOE_DMA_STAGES
#define MOE_DMA_STAGES 2
#endif
// channel tile of the bf16-weight comparator: its weight tile has twice the
// bytes per channel, so half the channels keep the LDS footprint (and two
// workgroups per CU) of the int8 tile
#ifndef MOE_DMA_BN_BF16
#define MOE_DMA_BN_BF16 128
#endif

// Waves per SIMD the register allocation must leave room for: with 4-wave
// workgroups two workgroups share a CU, so one can compute while the other
// waits at its barrier.
#ifndef MOE_DMA_WAVES_PER_EU
#define MOE_DMA_WAVES_PER_EU 2
#endif

template <bool kGateUp, bool kScaleBf16, int F, int GM, int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(MOE_DMA_WAVES_PER_EU)))
void ffn_tiled_dma_kernel(
    const __bf16* __restrict__ X, const int32_t* __restrict__ sorted_slots, int topk,
    const int8_t* __restrict__ W0, const int8_t* __restrict__ W1, const void* __restrict__ S0,
    const void* __restrict__ S1, const int32_t* __restrict__ offsets, int E, int N, int Kd, int n_tiles_n,
    void* __restrict__ out, unsigned long long* __restrict__ claims) {
  constexpr int TM = BM / WM, TN = BN / WN, MB = TM / 16, NB = TN / 16;
  static_assert(STAGES == 2 || STAGES == 3, "ring depth");
  using WF = WFormat<F>;
  constexpr int PPS = WF::kPieces;           // 1 KiB blocks per 16 channels and step
  constexpr int A_STAGE = BM * 128;          // bytes per step (bf16, 64 wide)
  constexpr int B_STAGE = BN * 64 * PPS;     // bytes per step (weight encoding, 64 wide)
  constexpr int A_INSTR = A_STAGE / 1024 / (WM * WN);  // 1 KiB loads per wave per step
  constexpr int B_INSTR = B_STAGE / 1024 / (WM * WN);
  constexpr int CH_TILE = kGateUp ? BN / 2 : BN;
  constexpr int VM_PER_STEP = A_INSTR + B_INSTR;
  static_assert(A_INSTR * 1024 * WM * WN == A_STAGE && B_INSTR * 1024 * WM * WN == B_STAGE, "tile split");

  __shared__ __attribute__((aligned(1024))) uint8_t As0[A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[A_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t As2[STAGES == 3 ? A_STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[B_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs1[B_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs2[STAGES == 3 ? B_STAGE : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: SGPR addressing
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 15;
  const int lg = lane >> 4;

  // this workgroup's tile: the static order with claimed queue tails (claims
  // given), else the static order throughout (claimed_tail_tile, static_tile)
  __shared__ int s_tile;
  int e, row0, nrows, nt;
  constexpr int GM_LONG = kGateUp ? MOE_TILE_GM_GU_LONG : GM;
  {
    const TileGrid g = tile_grid<BM>(offsets, E, n_tiles_n, kXcds, claims ? 1 : xcd_grain(kGateUp, n_tiles_n));
    int tile;
    if (claims) {
      tile = claimed_tail_tile(g, kXcds, kClaimTail, claims, &s_tile);
    } else {
      tile = static_tile(g, kXcds);
    }
    if (tile < 0) return;
    decode_tile<BM, GM, GM_LONG>(g, tile, E, n_tiles_n, e, row0, nrows, nt);
  }
  const int n0 = nt * CH_TILE;

  // activation sources: instruction j of this wave covers rows 8*(A_INSTR*wave + j) + lane/8;
  // a_off = byte offset from X of this lane's 16 bytes at reduction step 0
  uint32_t a_off[A_INSTR];
#pragma unroll
  for (int j = 0; j < A_INSTR; ++j) {
    const int r = 8 * (A_INSTR * wave + j) + (lane >> 3);
    const int rr = (r < nrows) ? r : 0;   // rows past the segment re-read row 0 (results unused)
    uint32_t src_row;
    if constexpr (kGateUp) {
      src_row = (uint32_t)(sorted_slots[row0 + rr] / topk);
    } else {
      src_row = (uint32_t)(row0 + rr);
    }
    const int chunk = (lane & 7) ^ (r & 7);
    a_off[j] = (src_row * (uint32_t)Kd + (uint32_t)(chunk * 8)) * 2u;
  }
  // weight sources: instruction j of this wave copies LDS block q = B_INSTR*wave + j,
  // piece q % PPS of 16-channel block q / PPS of this expert's matrix (uniform base),
  // at byte offset b_off (+PPS KiB per step)
  const int8_t* b_base[B_INSTR];
  uint32_t b_off[B_INSTR];
#pragma unroll
  for (int j = 0; j < B_INSTR; ++j) {
    const int blk = (B_INSTR * wave + j) / PPS;
    const int piece = (B_INSTR * wave + j) % PPS;
    const int8_t* base;
    int chl;
    if constexpr (kGateUp) {
      base = (blk < BN / 32) ? W0 : W1;
      chl = n0 + 16 * (blk % (BN / 32));
    } else {
      base = W0;
      chl = n0 + 16 * blk;
    }
    if (chl >= N) chl = 0;                // past N: re-read channel group 0 (results unused)
    b_base[j] = base + (long)e * N * Kd * PPS;
    b_off[j] = (uint32_t)(chl >> 4) * (uint32_t)(Kd >> 6) * (1024u * PPS) + 1024u * piece + 16u * lane;
  }

  // LDS buffers are always named directly (never through a pointer variable) so
  // the compiler can tell the stages apart and does not drain the loads of the
  // other stages before reading this one.
#define MOE_DMA_ISSUE(KT, AS, BS)                                                                   \
  {                                                                                                 \
    _Pragma("unroll") for (int j = 0; j < A_INSTR; ++j)                                             \
      dma16(X, a_off[j] + (uint32_t)(KT) * 128u, lds_addr(AS) + (A_INSTR * wave + j) * 1024);       \
    _Pragma("unroll") for (int j = 0; j < B_INSTR; ++j)                                             \
      dma16(b_base[j], b_off[j] + (uint32_t)(KT) * (1024u * PPS), lds_addr(BS) + (B_INSTR * wave + j) * 1024); \
  }

  // weight block of the wave's channel block j (LDS block index)
  auto b_block = [&](int j) {
    if constexpr (kGateUp) {
      constexpr int HALF = NB / 2;
      return (j < HALF) ? (wn * HALF + j) : (BN / 32 + wn * HALF + (j - HALF));
    } else {
      return wn * NB + j;
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

// One 64-wide step: lane (li, lg) reads piece 16*lg + li of each of the
// PPS blocks of a 16-channel group (channel li; 16 lanes read 256 contiguous
// bytes, free of bank conflicts) and turns them into the two MFMA operands of
// the step (sub-steps ks = 0, 1); the matching activation chunk holds the
// reduction elements the encoding puts there: kActLane*lg + kActSecond*ks.
#define MOE_DMA_COMPUTE(AS, BS, MBV)                                                                \
  {                                                                                                 \
    uint4 wq[NB][PPS];                                                                              \
    _Pragma("unroll") for (int j = 0; j < NB; ++j)                                                  \
      _Pragma("unroll") for (int q = 0; q < PPS; ++q)                                               \
        wq[j][q] = *reinterpret_cast<const uint4*>(&BS[(b_block(j) * PPS + q) * 1024 + 256 * lg + 16 * li]); \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                              \
      bf16x8 xf[MB];                                                                                \
      bf16x8 wf[NB];                                                                                \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) {                                              \
        if (i < (MBV)) {                                                                            \
          const int row = wm * TM + i * 16 + li;                                                    \
          const int chunk = ((WF::kActLane * lg + WF::kActSecond * ks) >> 3) ^ (row & 7);           \
          xf[i] = *reinterpret_cast<const bf16x8*>(&AS[row * 128 + chunk * 16]);                    \
        }                                                                                           \
      }                                                                                             \
      MOE_DMA_MMA(MBV)                                                                              \
    }                                                                                               \
  }

// The MFMAs of one sub-step, weight fragment by weight fragment: fragment j is
// converted, then its MFMAs over the row blocks, so the first MFMAs wait for
// one conversion instead of all of them (the compiler interleaves the next
// fragment's conversion with these MFMAs; each accumulator still receives one
// MFMA per sub-step, so the sums are unchanged). Against converting every
// fragment before an i-j nest: Mini prefill gate/up 1-1.5% faster, Large
// 0.5-1%; pinning the interleave with scheduling groups measured 1-3% slower.
#define MOE_DMA_MMA(MBV)                                                                            \
  _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                                  \
    wf[j] = WF::operand(wq[j], ks);                                                                 \
    _Pragma("unroll") for (int i = 0; i < MB; ++i)                                                  \
      if (i < (MBV)) acc[i][j] = mfma_bf16(wf[j], xf[i], acc[i][j]);                                 \
  }

  // per-lane scales of the channels this lane holds in the result, read before
  // the main loop so the epilogue waits on no load: gate/up keeps the gate
  // scales of its HALF channel blocks then the up scales, down its NB blocks
  // (unscaled encodings and channels past N: 1)
  float4 scl[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    scl[j] = make_float4(1.f, 1.f, 1.f, 1.f);
    if constexpr (WF::kScaled) {
      if constexpr (kGateUp) {
        constexpr int HALF = NB / 2;
        const int ch = n0 + wn * (HALF * 16) + (j % HALF) * 16 + 4 * lg;
        if (ch < N) scl[j] = load_scale4<kScaleBf16>(j < HALF ? S0 : S1, (long)e * N + ch);
      } else {
        const int ch = n0 + wn * TN + j * 16 + 4 * lg;
        if (ch < N) scl[j] = load_scale4<kScaleBf16>(S0, (long)e * N + ch);
      }
    }
  }

  const int nk = Kd >> 6;
  // Every step issues the step STAGES-1 ahead, clamped to the last one: past the
  // end this reloads the last step into a buffer that is no longer read, which
  // keeps the loop free of branches around the loads and the vmcnt bookkeeping
  // exact. Before computing step kt, its loads must be done while the loads of
  // the STAGES-2 later steps may still be in flight.
  constexpr int VM_IN_FLIGHT = (STAGES - 2) * VM_PER_STEP;
#define MOE_DMA_STEP(KT, AC, BC, AN, BN_, MBV)                                              \
  {                                                                                         \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM_IN_FLIGHT));                             \
    __builtin_amdgcn_s_barrier();                                                           \
    MOE_DMA_ISSUE(min((KT) + STAGES - 1, nk - 1), AN, BN_)                                  \
    MOE_DMA_COMPUTE(AC, BC, MBV)                                                            \
  }
  // A partial row tile (the last one of an expert) skips the MFMAs and the
  // fragment reads of the 16-row blocks it does not have, in this wave's rows;
  // each count of blocks has its own copy of the loop, free of branches
  // (against one copy with a runtime count: Mini prefill gate/up and down
  // about 1% faster).
  const int mb_valid = min(MB, max(0, (nrows - wm * TM + 15) / 16));
  static_assert(MB <= 8, "one loop copy per row-block count, up to 8");
#define MOE_DMA_MAIN_LOOP(MBV)                                                              \
  {                                                                                         \
    int k0 = 0;                                                                             \
    if constexpr (STAGES == 3) {                                                            \
      MOE_DMA_ISSUE(0, As0, Bs0)                                                            \
      MOE_DMA_ISSUE(min(1, nk - 1), As1, Bs1)                                               \
      for (; k0 + 3 <= nk; k0 += 3) {                                                       \
        MOE_DMA_STEP(k0 + 0, As0, Bs0, As2, Bs2, MBV)                                       \
        MOE_DMA_STEP(k0 + 1, As1, Bs1, As0, Bs0, MBV)                                       \
        MOE_DMA_STEP(k0 + 2, As2, Bs2, As1, Bs1, MBV)                                       \
      }                                                                                     \
      if (k0 < nk) MOE_DMA_STEP(k0, As0, Bs0, As2, Bs2, MBV)                                \
      if (k0 + 1 < nk) MOE_DMA_STEP(k0 + 1, As1, Bs1, As0, Bs0, MBV)                        \
    } else {                                                                                \
      MOE_DMA_ISSUE(0, As0, Bs0)                                                            \
      for (; k0 + 2 <= nk; k0 += 2) {                                                       \
        MOE_DMA_STEP(k0 + 0, As0, Bs0, As1, Bs1, MBV)                                       \
        MOE_DMA_STEP(k0 + 1, As1, Bs1, As0, Bs0, MBV)                                       \
      }                                                                                     \
      if (k0 < nk) MOE_DMA_STEP(k0, As0, Bs0, As1, Bs1, MBV)                                \
    }                                                                                       \
  }
  auto main_loop = [&](auto mbc) {
    constexpr int MBV = decltype(mbc)::value;
    MOE_DMA_MAIN_LOOP(MBV)
  };
  switch (mb_valid) {
    case 0: main_loop(int_constant<0>{}); break;
    case 1: main_loop(int_constant<(1 < MB ? 1 : MB)>{}); break;
    case 2: main_loop(int_constant<(2 < MB ? 2 : MB)>{}); break;
    case 3: main_loop(int_constant<(3 < MB ? 3 : MB)>{}); break;
    case 4: main_loop(int_constant<(4 < MB ? 4 : MB)>{}); break;
    case 5: main_loop(int_constant<(5 < MB ? 5 : MB)>{}); break;
    case 6: main_loop(int_constant<(6 < MB ? 6 : MB)>{}); break;
    case 7: main_loop(int_constant<(7 < MB ? 7 : MB)>{}); break;
    default: main_loop(int_constant<MB>{}); break;
  }
#undef MOE_DMA_MAIN_LOOP
#undef MOE_DMA_STEP
  // no load may still be writing this workgroup's LDS when the waves exit
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
#undef MOE_DMA_ISSUE
#undef MOE_DMA_COMPUTE

  // ---- epilogue (as in the register-staged kernel)
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
        const float4 sg = scl[j], su = scl[j + HALF];
        const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
        bf16x4 hv;
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[q] = (__bf16)(silu(acc[i][j][q] * sgv[q]) * (acc[i][j + HALF][q] * suv[q]));
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + orow + ch) = hv;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int ch = n0 + wn * TN + j * 16 + 4 * lg;
        if (ch >= N) continue;
        const float4 sd = scl[j];
        const float4 yv = make_float4(acc[i][j][0] * sd.x, acc[i][j][1] * sd.y, acc[i][j][2] * sd.z, acc[i][j][3] * sd.w);
        *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + ch) = yv;
      }
    }
  }
}

__global__ void zero_claims_kernel(unsigned long long* __restrict__ claims) {
  if (threadIdx.x < kXcds) claims[threadIdx.x] = 0ull;
}


template <bool kGateUp, bool kScaleBf16, int F, int DBN>
hipError_t launch_dma_pass(const FfnArgs& a, hipStream_t stream) {
  constexpr int GM = kGateUp ? MOE_TILE_GM_GU : MOE_TILE_GM;
  constexpr int DBM = MOE_DMA_BM, DWM = MOE_DMA_WM, DWN = MOE_DMA_WN, DST = MOE_DMA_STAGES;
  constexpr int DCH = kGateUp ? DBN / 2 : DBN;
  const int N = kGateUp ? a.f : a.d;
  const int Kd = kGateUp ? a.d : a.f;
  const int dn_tiles = (N + DCH - 1) / DCH;
  const long m_tiles_max = (long)(a.S + DBM - 1) / DBM + a.E;
  unsigned long long* claims = kGateUp ? a.claims_gate_up : a.claims_down;
  long dblocks;
  if (claims) {
    // the static blocks of the longest queue, then one and a half times its tail
    const long per_xcd_max = (m_tiles_max * dn_tiles + kXcds - 1) / kXcds;
    const long tail = min(per_xcd_max, (long)kClaimTail);
    dblocks = kXcds * (per_xcd_max + tail / 2);
    hipLaunchKernelGGL(zero_claims_kernel, dim3(1), dim3(kWave), 0, stream, claims);
  } else {
    dblocks = tiled_grid_blocks(kGateUp, m_tiles_max, dn_tiles);
  }
  const dim3 dblock(DWM * DWN * kWave);
  if constexpr (kGateUp) {
    hipLaunchKernelGGL((ffn_tiled_dma_kernel<true, kScaleBf16, F, GM, DBM, DBN, DWM, DWN, DST>), dim3((unsigned)dblocks),
                       dblock, 0, stream, static_cast<const __bf16*>(a.x), a.sorted_slots, a.K, a.w_gate, a.w_up,
                       a.s_gate, a.s_up, a.offsets, a.E, N, Kd, dn_tiles, static_cast<void*>(a.h), claims);
  } else {
    hipLaunchKernelGGL((ffn_tiled_dma_kernel<false, kScaleBf16, F, GM, DBM, DBN, DWM, DWN, DST>), dim3((unsigned)dblocks),
                       dblock, 0, stream, static_cast<const __bf16*>(a.h), a.sorted_slots, a.K, a.w_down, nullptr,
                       a.s_down, nullptr, a.offsets, a.E, N, Kd, dn_tiles, static_cast<void*>(a.y_rows), claims);
  }
  return hipGetLastError();
}

template <bool kGateUp, typename Act, bool kScaleBf16>
hipError_t launch_tiled_pass(const FfnArgs& a, hipStream_t stream) {
  constexpr int BM = MOE_TILE_BM, BN = MOE_TILE_BN, WM = MOE_TILE_WM, WN = MOE_TILE_WN, GM = MOE_TILE_GM;
  constexpr int CH_TILE = kGateUp ? BN / 2 : BN;
  const int N = kGateUp ? a.f : a.d;
  const int Kd = kGateUp ? a.d : a.f;
  if (sizeof(Act) == 2 && MOE_TILE_DMA && dma_offsets_fit(a.T, a.S, a.d, a.f, 1))
    return launch_dma_pass<kGateUp, kScaleBf16, kWInt8, MOE_DMA_BN>(a, stream);
  // register-staged kernel (int8 weights only)
  const int n_tiles_n = (N + CH_TILE - 1) / CH_TILE;
  const long blocks = tiled_grid_blocks(kGateUp, (long)(a.S + BM - 1) / BM + a.E, n_tiles_n);
  const dim3 grid((unsigned)blocks);
  const dim3 block(WM * WN * kWave);
  if constexpr (kGateUp) {
    hipLaunchKernelGGL((ffn_tiled_kernel<true, Act, kScaleBf16, BM, BN, WM, WN, GM>), grid, block, 0, stream,
                       static_cast<const Act*>(a.x), a.sorted_slots, a.K, a.w_gate, a.w_up, a.s_gate, a.s_up,
                       a.offsets, a.E, N, Kd, n_tiles_n, static_cast<void*>(a.h));
  } else {
    hipLaunchKernelGGL((ffn_tiled_kernel<false, __bf16, kScaleBf16, BM, BN, WM, WN, GM>), grid, block, 0, stream,
                       static_cast<const __bf16*>(a.h), a.sorted_slots, a.K, a.w_down, nullptr, a.s_down, nullptr,
                       a.offsets, a.E, N, Kd, n_tiles_n, static_cast<void*>(a.y_rows));
  }
  return hipGetLastError();
}

// int8 weights: every activation and scale dtype (the register-staged kernel
// covers fp32 activations and tensors past 32-bit offsets). bf16 and fp8
// weights (comparators): the direct-to-LDS kernel only, bf16 activations.
template <bool kGateUp>
hipError_t dispatch_tiled(const FfnArgs& a, hipStream_t stream) {
  switch (a.wfmt) {
    case kWInt8:
      if (a.act_bf16) {
        return a.scale_bf16 ? launch_tiled_pass<kGateUp, __bf16, true>(a, stream)
                            : launch_tiled_pass<kGateUp, __bf16, false>(a, stream);
      }
      return a.scale_bf16 ? launch_tiled_pass<kGateUp, float, true>(a, stream)
                          : launch_tiled_pass<kGateUp, float, false>(a, stream);
    case kWBf16:
      if (!a.act_bf16 || !dma_offsets_fit(a.T, a.S, a.d, a.f, 2)) return hipErrorInvalidValue;
      return launch_dma_pass<kGateUp, true, kWBf16, MOE_DMA_BN_BF16>(a, stream);
    case kWFp8:
      if (!a.act_bf16 || !dma_offsets_fit(a.T, a.S, a.d, a.f, 1)) return hipErrorInvalidValue;
      return a.scale_bf16 ? launch_dma_pass<kGateUp, true, kWFp8, MOE_DMA_BN>(a, stream)
                          : launch_dma_pass<kGateUp, false, kWFp8, MOE_DMA_BN>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

// The direct-to-LDS kernel addresses with 32-bit byte offsets from the
// activation tensors (x [T, d], h [S, f] bf16) and from one expert's weight
// matrix (f*d elements of wbytes each).
bool dma_offsets_fit(long T, long S, long d, long f, int wbytes) {
  const uint64_t lim = 1ull << 32;
  return (uint64_t)T * d * 2 < lim && (uint64_t)S * f * 2 < lim && (uint64_t)d * f * wbytes < lim;
}

hipError_t launch_tiled_gate_up(const FfnArgs& a, hipStream_t stream) { return dispatch_tiled<true>(a, stream); }
hipError_t launch_tiled_down(const FfnArgs& a, hipStream_t stream) { return dispatch_tiled<false>(a, stream); }

}  // namespace moe
