// Expert FFN, weight-streaming schedule (few rows per expert: decode).
//
// With a handful of tokens per expert the layer is bound by reading the int8
// weights from HBM once (the paper's serving note: MoE/MLP layers are
// I/O-bound, and ExpertsInt8 moves the weights from HBM at half the bytes of
// BF16). Each wave owns one (expert, group of 16*NG output channels) item and
// runs the full reduction for all of the expert's rows (up to 16*RB per pass):
//   - weights are in the tiled layout (pack.hip), so each 16-channel group
//     is one contiguous run of 1 KiB blocks; per 64-wide step a wave reads one
//     block per group and matrix (lane l: channel l%16, bytes 16*(l/16)..+16)
//     with non-temporal loads, and the loads of the next P-1 steps are in
//     flight;
//   - the int8 codes become bf16 in registers (exact) and feed 16x16x32 bf16
//     MFMA, with the channels as MFMA rows and the tokens as MFMA columns;
//   - a 64-wide step is two MFMAs: code bytes 0-7 of each lane pair with
//     activation elements 0-7 of the same lane group, bytes 8-15 with 8-15;
//   - the comparator encodings (WFormat: bf16 weights, fp8 codes) change only
//     how a lane's pieces become the two operands and which activation
//     elements pair with them.
// Items are numbered over the experts that received rows only, so the grid
// has no idle waves for untouched experts. For at most 256 slots the gate/up
// pass can take the expert ids instead of the permutation and write the
// permutation itself (one launch fewer for a decode step).
// With few items (a dense MLP layer has one expert) there are too few waves
// to keep enough loads in flight, and long waves balance badly at the end of
// the pass, so the reduction axis of each item is cut into KS slices streamed
// by the KS waves of one workgroup; the slices' fp32 partial sums are added
// through LDS in ascending slice order before the epilogue, so the result does
// not depend on scheduling and costs no extra HBM traffic.
// With more than 32 rows per expert every wave would re-read its rows'
// activations from L2 at each step, so two variants share them through LDS
// among the waves of a workgroup that work on neighbouring channel groups:
// the gate/up pass (ffn_stream_shared_gu_kernel), and the down pass with a
// split reduction when the caller provides a workspace for the slices' sums
// (ffn_stream_shared_dn_kernel + split_down_reduce_kernel, bitwise the same
// result as the in-workgroup split).
// Gate/up pass: g and u accumulate side by side; the epilogue applies the
// per-channel scales and SwiGLU and stores h (bf16). Down pass: the epilogue
// applies the down scale and stores y_rows (fp32).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

// Schedule parameters (compile-time; overridable for tuning builds):
// NG 16-channel groups per wave, RB 16-row blocks per pass, P-stage load ring,
// WAVES waves per workgroup. Measured on MI355X: the gate/up pass (two
// matrices per group) streams best with one group per wave, the down pass
// with four groups and a four-deep ring.
#ifndef MOE_STREAM_NG_GU
#define MOE_STREAM_NG_GU 1
#endif
#ifndef MOE_STREAM_P_GU
#define MOE_STREAM_P_GU 3
#endif
// ring of the unsplit 32-row gate/up pass, whose waves stream whole items
// (Large decode: 5 stages 1009-1018 us against 3 stages 1031-1040 us; split
// passes measured best with 2-3)
#ifndef MOE_STREAM_P_GU_LONG
#define MOE_STREAM_P_GU_LONG 5
#endif
#ifndef MOE_STREAM_NG_DN
#define MOE_STREAM_NG_DN 4
#endif
// groups per wave of the 64-row variant: each wave re-reads its rows'
// activations from L2 for every step, so wider gate/up items halve that
// traffic; the down pass, whose accumulators and activation ring are four
// times larger, keeps fewer groups than in the 32-row variant
#ifndef MOE_STREAM_NG_DN_WIDE
#define MOE_STREAM_NG_DN_WIDE 2
#endif
#ifndef MOE_STREAM_NG_GU_WIDE
#define MOE_STREAM_NG_GU_WIDE 2
#endif
#ifndef MOE_STREAM_P_DN
#define MOE_STREAM_P_DN 4
#endif
#ifndef MOE_STREAM_RB
#define MOE_STREAM_RB 2
#endif
#ifndef MOE_STREAM_WAVES
#define MOE_STREAM_WAVES 4
#endif
// Waves a pass wants in flight: the 32-row down pass MIN_WAVES, the 64-row
// variant MIN_WAVES_WIDE (four times the MFMA and activation work per weight
// byte, so more waves are needed to keep HBM busy).
#ifndef MOE_STREAM_MIN_WAVES
#define MOE_STREAM_MIN_WAVES 1024
#endif
#ifndef MOE_STREAM_MIN_WAVES_WIDE
#define MOE_STREAM_MIN_WAVES_WIDE 4096
#endif
// The gate/up pass of the 32-row variant splits its reductions (at most 4
// ways) until it has MIN_WAVES_GU waves: shorter waves balance better at the
// end of the pass. Measured (interleaved A/B): Mini decode, 14336 items split
// in 2: 290-298 -> 277-290 us; the TP8 share of Large decode, 3072 items split
// in 4: 142-154 -> 131-145 us; Large decode, 24576 items, stays unsplit (a
// split of 2 measured 1-2% slower, 8 ways 10% slower on the TP8 share).
#ifndef MOE_STREAM_MIN_WAVES_GU
#define MOE_STREAM_MIN_WAVES_GU 16384
#endif
#ifndef MOE_STREAM_MAX_SPLIT_GU
#define MOE_STREAM_MAX_SPLIT_GU 4
#endif
// activation prefetch ring of the 64-row variant (see the main loop)
#ifndef MOE_STREAM_PA_WIDE
#define MOE_STREAM_PA_WIDE 2
#endif
// the 64-row gate/up pass shares its activations through LDS (1) or not (0);
// ring depth of that kernel; workgroups it aims for (one per CU)
#ifndef MOE_STREAM_SHARED_GU
#define MOE_STREAM_SHARED_GU 1
#endif
#ifndef MOE_STREAM_P_SHARED
#define MOE_STREAM_P_SHARED 6
#endif
// ring depth of that kernel's reduction-split shapes (six waves: the registers
// of two waves per SIMD leave room for four stages; the one-wave-per-SIMD
// shape measured the same with 3, 4 and 5 stages, slower with 6)
#ifndef MOE_STREAM_P_SHARED_SPLIT
#define MOE_STREAM_P_SHARED_SPLIT 4
#endif
#ifndef MOE_STREAM_SHARED_MIN_WGS
#define MOE_STREAM_SHARED_MIN_WGS 256
#endif
// the 64-row down pass with a reduction split: with a workspace for the
// slices' partial sums (1), workgroups of SHARED_DN_WAVES waves share each
// slice's activations through LDS and a second kernel adds the slices;
// without one (0, or no workspace) the slices stay inside one workgroup
#ifndef MOE_STREAM_SHARED_DN
#define MOE_STREAM_SHARED_DN 1
#endif
#ifndef MOE_STREAM_SHARED_DN_WAVES
#define MOE_STREAM_SHARED_DN_WAVES 4
#endif
// 16-channel groups per wave of that kernel and its ring depth: one wave per
// SIMD with 64-channel items streams the dense MLP's down pass best (A/B on
// one box: 54.6 -> 50.3 us with an 8-deep ring, 51.0 with 6, 50.4 with 5;
// 32-channel items with an 8-deep ring: 54.0). The reduction split is still
// chosen from the 32-channel item count (MOE_STREAM_NG_DN_WIDE), so the
// slices, and the result, are those of the in-workgroup split.
#ifndef MOE_STREAM_NG_SHARED_DN
#define MOE_STREAM_NG_SHARED_DN 4
#endif
#ifndef MOE_STREAM_P_SHARED_DN
#define MOE_STREAM_P_SHARED_DN 8
#endif
constexpr int kStreamWaves = MOE_STREAM_WAVES;

constexpr int ring_gcd(int a, int b) { return b == 0 ? a : ring_gcd(b, a % b); }
constexpr int ring_unroll(int a, int b) { return a / ring_gcd(a, b) * b; }

// Reduction split (1, 2, 4 or 8) of a pass with `items` (expert, channel
// group) items: the smallest that reaches the pass's wave target, within its
// largest split.
int choose_split(long items, int RB, bool gate_up = false) {
  const long want = RB >= 4 ? MOE_STREAM_MIN_WAVES_WIDE : (gate_up ? MOE_STREAM_MIN_WAVES_GU : MOE_STREAM_MIN_WAVES);
  const int max_ks = (gate_up && RB < 4) ? MOE_STREAM_MAX_SPLIT_GU : 8;
  int ks = 1;
  while (ks < max_ks && items * ks < want) ks *= 2;
  return ks;
}

// Waves of a workgroup: kStreamWaves items of one wave each (KS = 1), or the
// KS slices of one item (KS > 1).
constexpr int stream_block_waves(int KS) { return KS > 1 ? KS : kStreamWaves; }

// A workgroup holds stream_block_waves(KS)/KS items; wave w works on item
// w/KS and streams the (w%KS)-th slice of its reduction axis.
//
// Gate/up pass with `ids` (S <= 256 slots): the rows and their source tokens
// come from the expert ids themselves (one wave holds them all) instead of a
// permutation in memory, and wave 0 of workgroup 0 writes that permutation
// (perm_*) for the passes after it; offsets and sorted_slots are unused.
template <bool kGateUp, typename Act, bool kScaleBf16, int F, int NG, int RB, int P, int KS>
__global__ __launch_bounds__(stream_block_waves(KS) * kWave) void ffn_stream_kernel(
    const Act* __restrict__ X, const int32_t* __restrict__ sorted_slots, int topk,
    const int8_t* __restrict__ W0, const int8_t* __restrict__ W1, const void* __restrict__ S0,
    const void* __restrict__ S1, const int32_t* __restrict__ offsets, int E, int N, int Kd,
    void* __restrict__ out, const int32_t* __restrict__ ids, int S, int32_t* __restrict__ perm_offsets,
    int32_t* __restrict__ perm_sorted, int32_t* __restrict__ perm_s2r) {
  constexpr int NMAT = kGateUp ? 2 : 1;
  using WF = WFormat<F>;
  constexpr int PPS = WF::kPieces;  // 1 KiB blocks per group and step
  constexpr int IPW = stream_block_waves(KS) / KS;  // items per workgroup
  // partial sums of slices 1..KS-1 for one 16-row block (KS > 1: one item)
  __shared__ f32x4 red[KS > 1 ? KS - 1 : 1][NG][NMAT][kWave];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- item -> (expert among the touched ones, channel group)
  const int gpe = N / (16 * NG);
  const int witem = wave / KS;  // item within the workgroup
  const int item = blockIdx.x * IPW + witem;
  const int kslice = wave % KS;
  const int te = item / gpe;
  const int grp = item - te * gpe;
  int e, row0, nrows;
  uint64_t e_slots[kIdChunks] = {};   // ids mode: the slots of expert e
  // With KS > 1 the workgroup is one item: every wave takes this return, the
  // row loop and the barriers below together.
  if (kGateUp && ids) {
    const WaveIds wid = load_wave_ids(ids, S);
    const ExpertSegments segs = segments_from_ids(wid, E);
    if (blockIdx.x == 0 && wave == 0) write_permutation(wid, segs, E, S, perm_offsets, perm_sorted, perm_s2r);
    if (!touched_expert(segs, te, e, row0, nrows)) return;
    expert_masks(wid, e, e_slots);
  } else if (!find_touched_expert(offsets, E, te, e, row0, nrows)) {
    return;
  }

  const int ch_base = grp * 16 * NG;
  // first 1 KiB block of each 16-channel group (tiled layout), this lane's piece
  const int8_t* wp[NG][NMAT];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const long group = ((long)e * N + ch_base + ng * 16) >> 4;
    const long off = group * (long)(Kd >> 6) * (1024 * PPS) + 16 * lane;
    wp[ng][0] = W0 + off;
    if constexpr (kGateUp) wp[ng][1] = W1 + off;
  }
  // per-lane scales of the 4 channels this lane holds in the result
  // (unscaled encodings: 1)
  float4 sc[NG][NMAT];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const long ch = (long)e * N + ch_base + ng * 16 + 4 * lg;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) sc[ng][m] = make_float4(1.f, 1.f, 1.f, 1.f);
    if constexpr (WF::kScaled) {
      sc[ng][0] = load_scale4<kScaleBf16>(S0, ch);
      if constexpr (kGateUp) sc[ng][1] = load_scale4<kScaleBf16>(S1, ch);
    }
  }

  // this wave's slice of the 64-wide reduction steps
  const int nsteps_all = Kd >> 6;
  const int s_base = kslice * nsteps_all / KS;
  const int nsteps = (kslice + 1) * nsteps_all / KS - s_base;

  for (int p0 = 0; p0 < nrows; p0 += 16 * RB) {
    const int prow = min(16 * RB, nrows - p0);
    const int nrb = (prow + 15) >> 4;
    const Act* ap[RB];
    bool aok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = p0 + rb * 16 + li;
      aok[rb] = r < nrows;
      long src = 0;
      if (aok[rb]) {
        if constexpr (kGateUp) {
          const int slot = ids ? select_slot(e_slots, r) : sorted_slots[row0 + r];
          src = (long)(slot / topk) * Kd;
        } else {
          src = (long)(row0 + r) * Kd;
        }
      }
      ap[rb] = X + src + WF::kActLane * lg + (long)s_base * 64;
    }

    f32x4 acc[RB][NG][NMAT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[rb][ng][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // weights are prefetched P-1 steps ahead, activations (small, mostly
    // L2 hits) PA-1 steps ahead; the loop body is unrolled over U steps so
    // both ring slots are compile-time indices. The loop is specialised on the
    // number of 16-row blocks of the pass (NRB; 0: the runtime count nrb), so
    // the common counts run without branches around the loads and MFMAs.
    constexpr int PA_WANT = RB >= 4 ? MOE_STREAM_PA_WIDE : P;
    constexpr int PA = PA_WANT < P ? PA_WANT : P;
    constexpr int U = ring_unroll(P, PA);
    auto run = [&](auto nrbc) {
      constexpr int NRB = decltype(nrbc)::value;
      const int nb = NRB > 0 ? NRB : nrb;
      uint4 bw[P][NG][NMAT][PPS];
      bf16x8 av[PA][RB][2];

      auto load_w = [&](int s, uint4 (&b)[NG][NMAT][PPS]) {
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int q = 0; q < PPS; ++q) b[ng][m][q] = load_nt16(wp[ng][m] + ((long)(s_base + s) * PPS + q) * 1024);
      };
      auto load_a = [&](int s, bf16x8 (&a)[RB][2]) {
        const long off = (long)s * 64;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (rb < nb) {
            if (aok[rb]) {
              a[rb][0] = load_act8(ap[rb] + off);
              a[rb][1] = load_act8(ap[rb] + off + WF::kActSecond);
            } else {
              a[rb][0] = zero_bf16x8();
              a[rb][1] = zero_bf16x8();
            }
          }
        }
      };
      // Each accumulator takes its two MFMAs (elements 0-7, then 8-15 of each
      // lane's piece) in that order. The second MFMAs of channel group ng are
      // issued after the first ones of group ng+1 (of both matrices, for all
      // row blocks), so consecutive MFMAs do not wait for each other's results
      // while only two groups' operands are live.
      auto compute_step = [&](const uint4 (&b)[NG][NMAT][PPS], const bf16x8 (&a)[RB][2]) {
        bf16x8 w_hi[NG][NMAT];
        auto second = [&](int ng) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              if (rb < nb) acc[rb][ng][m] = mfma_bf16(w_hi[ng][m], a[rb][1], acc[rb][ng][m]);
        };
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          bf16x8 w_lo[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) WF::operands(b[ng][m], w_lo[m], w_hi[ng][m]);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              if (rb < nb) acc[rb][ng][m] = mfma_bf16(w_lo[m], a[rb][0], acc[rb][ng][m]);
          if (ng > 0) second(ng - 1);
        }
        second(NG - 1);
      };

#pragma unroll
      for (int j = 0; j < P - 1; ++j)
        if (j < nsteps) load_w(j, bw[j]);
#pragma unroll
      for (int j = 0; j < PA - 1; ++j)
        if (j < nsteps) load_a(j, av[j]);
      for (int s0 = 0; s0 < nsteps; s0 += U) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const int s = s0 + j;
          if (s + P - 1 < nsteps) load_w(s + P - 1, bw[(j + P - 1) % P]);
          if (s + PA - 1 < nsteps) load_a(s + PA - 1, av[(j + PA - 1) % PA]);
          if (s < nsteps) compute_step(bw[j % P], av[j % PA]);
        }
      }
    };
    if constexpr (KS > 1) {
      run(int_constant<0>{});   // one copy: the split's LDS reduction leaves no registers for more
    } else if (nrb == RB) {
      run(int_constant<RB>{});
    } else if (RB == 2 || nrb == 1) {   // RB == 2: the only other count is 1
      run(int_constant<1>{});
    } else {
      run(int_constant<0>{});
    }

    if constexpr (KS > 1) {
      // slice 0 adds slices 1..KS-1 in order, one 16-row block at a time
      // (nrb is the same for every wave of the workgroup)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb < nrb) {
          if (kslice > 0) {
#pragma unroll
            for (int ng = 0; ng < NG; ++ng)
#pragma unroll
              for (int m = 0; m < NMAT; ++m) red[kslice - 1][ng][m][lane] = acc[rb][ng][m];
          }
          __syncthreads();
          if (kslice == 0) {
            for (int j = 0; j < KS - 1; ++j)
#pragma unroll
              for (int ng = 0; ng < NG; ++ng)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[rb][ng][m] += red[j][ng][m][lane];
          }
          __syncthreads();
        }
      }
      if (kslice > 0) continue;
    }
    // ---- epilogue: lane holds channels ch_base + ng*16 + 4*lg + r, row p0 + rb*16 + li
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = p0 + rb * 16 + li;
      if (rb < nrb && r < nrows) {
        const long orow = (long)(row0 + r) * N;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          const int ch = ch_base + ng * 16 + 4 * lg;
          if constexpr (kGateUp) {
            const float sgv[4] = {sc[ng][0].x, sc[ng][0].y, sc[ng][0].z, sc[ng][0].w};
            const float suv[4] = {sc[ng][1].x, sc[ng][1].y, sc[ng][1].z, sc[ng][1].w};
            bf16x4 hv;
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[q] = (__bf16)(silu(acc[rb][ng][0][q] * sgv[q]) * (acc[rb][ng][1][q] * suv[q]));
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + orow + ch) = hv;
          } else {
            const float4 yv = make_float4(acc[rb][ng][0][0] * sc[ng][0].x, acc[rb][ng][0][1] * sc[ng][0].y,
                                          acc[rb][ng][0][2] * sc[ng][0].z, acc[rb][ng][0][3] * sc[ng][0].w);
            *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + ch) = yv;
          }
        }
      }
    }
  }
}

// Gate/up pass of the 64-row variant with the activations shared through LDS.
// With many rows per expert (a dense MLP layer at decode) every wave of
// ffn_stream_kernel re-reads the rows' activations from L2 for each step,
// which costs more vector-memory traffic than the weights it streams. Here a
// workgroup of WI*KS waves holds WI consecutive items of one expert, each
// item's reduction cut into KS equal slices streamed by KS waves (slice-major
// wave order): per 64-wide step the WI waves of a slice copy that slice's
// 64-row activation tile (8 KiB bf16) once into the slice's P-deep LDS ring
// with direct-to-LDS loads, while each wave streams its own weight blocks into
// a P-deep register ring; one barrier per step. The tile lands XOR-swizzled by
// row as in the tiled kernel. Without a split (KS = 1) each item's MFMAs run
// in the same order as in ffn_stream_kernel without a split; with one, slices
// 1..KS-1 hand their fp32 sums to slice 0 through LDS, which adds them in
// ascending slice order before the epilogue. The split lets a dense layer,
// whose items would leave a SIMD of every CU idle, spread the same MFMA and
// conversion work over all four.
// Loads per step and wave: NG*2*PPS weight loads, then its share of the 8
// activation DMAs. Before step s the activations of step s must have landed
// while the loads of steps s+1..s+P-2 may still be in flight.
template <bool kScaleBf16, int F, int NG, int WI, int KS, int P>
__global__ __launch_bounds__(WI * KS * kWave) void ffn_stream_shared_gu_kernel(
    const __bf16* __restrict__ X, const int32_t* __restrict__ sorted_slots, int topk,
    const int8_t* __restrict__ W0, const int8_t* __restrict__ W1, const void* __restrict__ S0,
    const void* __restrict__ S1, const int32_t* __restrict__ offsets, int E, int N, int Kd,
    __bf16* __restrict__ out) {
  constexpr int NMAT = 2;
  constexpr int RB = 4;                      // 16-row blocks per pass
  constexpr int ROWS = 16 * RB;
  using WF = WFormat<F>;
  constexpr int PPS = WF::kPieces;
  constexpr int STAGE = ROWS * 128;          // one step's activation tile
  constexpr int A_TOT = STAGE / 1024;        // its 1 KiB DMA instructions, dealt round-robin to the waves
  constexpr int A_MAX = (A_TOT + WI - 1) / WI;
  constexpr int A_MIN = A_TOT / WI;
  constexpr int NWI = NG * NMAT * PPS;       // weight loads per wave and step
  static_assert((P - 2) * (NWI + A_MAX) <= 63, "the vmcnt field holds at most 63");
  // slices 1..KS-1 pass their sums through the (then idle) rings
  static_assert((KS - 1) * WI * RB * NG * NMAT * kWave * 16 <= KS * P * STAGE, "reduction fits the rings");
  __shared__ __attribute__((aligned(1024))) uint8_t act[KS][P][STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slice = wave / WI;               // uniform
  const int witem = wave - slice * WI;
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- workgroup -> (expert among the touched ones, WI consecutive items)
  const int gpe = N / (16 * NG);
  const int wg_per_e = gpe / WI;
  const int te = blockIdx.x / wg_per_e;
  const int grp = (blockIdx.x - te * wg_per_e) * WI + witem;
  int e, row0, nrows;
  if (!find_touched_expert(offsets, E, te, e, row0, nrows)) return;   // the same for every wave of the workgroup

  const int ch_base = grp * 16 * NG;
  const int8_t* wp[NG][NMAT];
  float4 sc[NG][NMAT];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const long group = ((long)e * N + ch_base + ng * 16) >> 4;
    const long off = group * (long)(Kd >> 6) * (1024 * PPS) + 16 * lane;
    wp[ng][0] = W0 + off;
    wp[ng][1] = W1 + off;
    const long ch = (long)e * N + ch_base + ng * 16 + 4 * lg;
    sc[ng][0] = make_float4(1.f, 1.f, 1.f, 1.f);
    sc[ng][1] = sc[ng][0];
    if constexpr (WF::kScaled) {
      sc[ng][0] = load_scale4<kScaleBf16>(S0, ch);
      sc[ng][1] = load_scale4<kScaleBf16>(S1, ch);
    }
  }
  const int nsteps = (Kd >> 6) / KS;         // the launch checks that KS divides the steps
  const int s_base = slice * nsteps;

  for (int p0 = 0; p0 < nrows; p0 += ROWS) {
    const int prow = min(ROWS, nrows - p0);
    const int nrb = (prow + 15) >> 4;
    // this wave's activation DMAs: tile instruction c = witem + WI*j of its
    // slice covers rows 8c..8c+7; lane l writes row 8c + l/8, chunk slot l%8,
    // fetched from the logical chunk slot ^ (row % 8); rows past the pass
    // re-read row 0
    uint32_t a_off[A_MAX];
#pragma unroll
    for (int j = 0; j < A_MAX; ++j) {
      const int c = min(witem + WI * j, A_TOT - 1);
      const int r = 8 * c + (lane >> 3);
      const int rr = (r < prow) ? r : 0;
      const uint32_t src_row = (uint32_t)(sorted_slots[row0 + p0 + rr] / topk);
      const int chunk = (lane & 7) ^ (r & 7);
      a_off[j] = (src_row * (uint32_t)Kd + (uint32_t)(s_base * 64 + chunk * 8)) * 2u;
    }

    f32x4 acc[RB][NG][NMAT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[rb][ng][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 bw[P][NG][NMAT][PPS];

    auto issue = [&](int t, int st) {
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int q = 0; q < PPS; ++q) bw[st][ng][m][q] = load_nt16(wp[ng][m] + ((long)(s_base + t) * PPS + q) * 1024);
#pragma unroll
      for (int j = 0; j < A_MAX; ++j)
        if (witem + WI * j < A_TOT)
          dma16(X, a_off[j] + (uint32_t)t * 128u, lds_addr(&act[slice][st][0]) + (witem + WI * j) * 1024);
    };
    // One step's MFMAs. A full pass (kFull: all RB row blocks present) has no
    // branches, so the conversions of one weight piece can overlap the MFMAs of
    // the previous one. Each accumulator takes its two MFMAs (elements 0-7,
    // then 8-15 of each lane's piece) in that order, but the first MFMAs of all
    // row blocks are issued before the second ones, so consecutive MFMAs do not
    // wait for each other's results.
    auto compute = [&](int st, auto full) {
      constexpr bool kFull = decltype(full)::value;
      bf16x8 xf[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (kFull || rb < nrb) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int row = rb * 16 + li;
            const int chunk = ((WF::kActLane * lg + WF::kActSecond * ks) >> 3) ^ (row & 7);
            xf[rb][ks] = *reinterpret_cast<const bf16x8*>(&act[slice][st][row * 128 + chunk * 16]);
          }
        }
      }
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          bf16x8 w_lo, w_hi;
          WF::operands(bw[st][ng][m], w_lo, w_hi);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (kFull || rb < nrb) acc[rb][ng][m] = mfma_bf16(w_lo, xf[rb][0], acc[rb][ng][m]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (kFull || rb < nrb) acc[rb][ng][m] = mfma_bf16(w_hi, xf[rb][1], acc[rb][ng][m]);
        }
      }
    };
    auto main_loop = [&](auto full) {
#pragma unroll
      for (int t = 0; t < P - 1; ++t) issue(min(t, nsteps - 1), t);
      for (int s0 = 0; s0 < nsteps; s0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (s0 + j < nsteps) {   // the same for every wave
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((P - 2) * (NWI + A_MIN)));
            __builtin_amdgcn_s_barrier();
            issue(min(s0 + j + P - 1, nsteps - 1), (j + P - 1) % P);
            compute(j, full);
          }
        }
      }
    };
    if (nrb == RB) {
      main_loop(bool_constant<true>{});
    } else {
      main_loop(bool_constant<false>{});
    }
    // no load may still be writing the ring when it is reused or the waves exit
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    if constexpr (KS > 1) {
      // slices 1..KS-1 park their sums in the rings; slice 0 adds them in
      // ascending slice order (nrb is the same for the whole workgroup)
      f32x4* red = reinterpret_cast<f32x4*>(&act[0][0][0]);
      auto red_at = [&](int sl, int rb, int ng, int m) {
        return red + ((((sl - 1) * WI + witem) * RB + rb) * NG * NMAT + ng * NMAT + m) * kWave + lane;
      };
      if (slice > 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (rb < nrb)
#pragma unroll
            for (int ng = 0; ng < NG; ++ng)
#pragma unroll
              for (int m = 0; m < NMAT; ++m) *red_at(slice, rb, ng, m) = acc[rb][ng][m];
      }
      __syncthreads();
      if (slice == 0) {
        for (int sl = 1; sl < KS; ++sl)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (rb < nrb)
#pragma unroll
              for (int ng = 0; ng < NG; ++ng)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[rb][ng][m] += *red_at(sl, rb, ng, m);
      }
      __syncthreads();   // the next pass's copies overwrite the rings
    }

    // ---- epilogue (as ffn_stream_kernel's gate/up pass), by slice 0
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = p0 + rb * 16 + li;
      if (slice == 0 && rb < nrb && r < nrows) {
        const long orow = (long)(row0 + r) * N;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng) {
          const int ch = ch_base + ng * 16 + 4 * lg;
          const float sgv[4] = {sc[ng][0].x, sc[ng][0].y, sc[ng][0].z, sc[ng][0].w};
          const float suv[4] = {sc[ng][1].x, sc[ng][1].y, sc[ng][1].z, sc[ng][1].w};
          bf16x4 hv;
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = (__bf16)(silu(acc[rb][ng][0][q] * sgv[q]) * (acc[rb][ng][1][q] * suv[q]));
          *reinterpret_cast<bf16x4*>(out + orow + ch) = hv;
        }
      }
    }
  }
}

// Down pass of the 64-row variant with the reduction split over workgroups.
// Workgroup (channel block, slice ks) holds W consecutive items of one expert
// (no split inside the workgroup) and streams reduction slice ks, the same
// slice boundaries as the in-workgroup split of ffn_stream_kernel; per
// 64-wide step its waves copy the 64-row tile of h (8 KiB) once into a P-deep
// LDS ring with direct-to-LDS loads, and each wave streams its own weight
// blocks into a P-deep register ring. The slice's fp32 sums (unscaled) go to
// plane ks of `part` ([KS, S, N]); split_down_reduce adds the planes in
// ascending slice order and applies the scale. Every MFMA, the sum order and
// the scaling are those of ffn_stream_kernel with the same split, so y_rows
// is the same bit for bit.
template <int F, int NG, int W, int P>
__global__ __launch_bounds__(W * kWave) void ffn_stream_shared_dn_kernel(
    const __bf16* __restrict__ H, const int8_t* __restrict__ W0, const int32_t* __restrict__ offsets, int E, int N,
    int Kd, int S, int KS, float* __restrict__ part) {
  constexpr int RB = 4;
  constexpr int ROWS = 16 * RB;
  using WF = WFormat<F>;
  constexpr int PPS = WF::kPieces;
  constexpr int STAGE = ROWS * 128;
  constexpr int A_TOT = STAGE / 1024;
  constexpr int A_MAX = (A_TOT + W - 1) / W;
  constexpr int A_MIN = A_TOT / W;
  constexpr int NWI = NG * PPS;              // weight loads per wave and step
  static_assert((P - 2) * (NWI + A_MAX) <= 63, "the vmcnt field holds at most 63");
  __shared__ __attribute__((aligned(1024))) uint8_t act[P][STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- workgroup -> (slice, expert among the touched ones, W consecutive items)
  const int gpe = N / (16 * NG);
  const int wg_per_e = gpe / W;
  const int ks = blockIdx.x % KS;
  const int rest = blockIdx.x / KS;
  const int te = rest / wg_per_e;
  const int grp = (rest - te * wg_per_e) * W + wave;
  int e, row0, nrows;
  if (!find_touched_expert(offsets, E, te, e, row0, nrows)) return;   // the same for the whole workgroup

  const int ch_base = grp * 16 * NG;
  const int8_t* wp[NG];
#pragma unroll
  for (int ng = 0; ng < NG; ++ng) {
    const long group = ((long)e * N + ch_base + ng * 16) >> 4;
    wp[ng] = W0 + group * (long)(Kd >> 6) * (1024 * PPS) + 16 * lane;
  }
  const int nsteps_all = Kd >> 6;
  const int s_base = ks * nsteps_all / KS;
  const int nsteps = (ks + 1) * nsteps_all / KS - s_base;
  float* plane = part + (long)ks * S * N;

  for (int p0 = 0; p0 < nrows; p0 += ROWS) {
    const int prow = min(ROWS, nrows - p0);
    const int nrb = (prow + 15) >> 4;
    // this wave's activation DMAs: tile instruction c = wave + W*j covers rows
    // 8c..8c+7; lane l writes row 8c + l/8, chunk slot l%8, fetched from the
    // logical chunk slot ^ (row % 8); rows past the pass re-read row 0
    uint32_t a_off[A_MAX];
#pragma unroll
    for (int j = 0; j < A_MAX; ++j) {
      const int c = min(wave + W * j, A_TOT - 1);
      const int r = 8 * c + (lane >> 3);
      const int rr = (r < prow) ? r : 0;
      const int chunk = (lane & 7) ^ (r & 7);
      a_off[j] = ((uint32_t)(row0 + p0 + rr) * (uint32_t)Kd + (uint32_t)(s_base * 64 + chunk * 8)) * 2u;
    }

    f32x4 acc[RB][NG];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) acc[rb][ng] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 bw[P][NG][PPS];

    auto issue = [&](int t, int st) {
#pragma unroll
      for (int ng = 0; ng < NG; ++ng)
#pragma unroll
        for (int q = 0; q < PPS; ++q) bw[st][ng][q] = load_nt16(wp[ng] + ((long)(s_base + t) * PPS + q) * 1024);
#pragma unroll
      for (int j = 0; j < A_MAX; ++j)
        if (wave + W * j < A_TOT)
          dma16(H, a_off[j] + (uint32_t)t * 128u, lds_addr(&act[st][0]) + (wave + W * j) * 1024);
    };
    // one step's MFMAs, ordered and specialised as in the shared gate/up kernel
    auto compute = [&](int st, auto full) {
      constexpr bool kFull = decltype(full)::value;
      bf16x8 xf[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (kFull || rb < nrb) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int row = rb * 16 + li;
            const int chunk = ((WF::kActLane * lg + WF::kActSecond * h2) >> 3) ^ (row & 7);
            xf[rb][h2] = *reinterpret_cast<const bf16x8*>(&act[st][row * 128 + chunk * 16]);
          }
        }
      }
#pragma unroll
      for (int ng = 0; ng < NG; ++ng) {
        bf16x8 w_lo, w_hi;
        WF::operands(bw[st][ng], w_lo, w_hi);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (kFull || rb < nrb) acc[rb][ng] = mfma_bf16(w_lo, xf[rb][0], acc[rb][ng]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (kFull || rb < nrb) acc[rb][ng] = mfma_bf16(w_hi, xf[rb][1], acc[rb][ng]);
      }
    };
    auto main_loop = [&](auto full) {
#pragma unroll
      for (int t = 0; t < P - 1; ++t) issue(min(t, nsteps - 1), t);
      for (int s0 = 0; s0 < nsteps; s0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (s0 + j < nsteps) {   // the same for every wave
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((P - 2) * (NWI + A_MIN)));
            __builtin_amdgcn_s_barrier();
            issue(min(s0 + j + P - 1, nsteps - 1), (j + P - 1) % P);
            compute(j, full);
          }
        }
      }
    };
    if (nrb == RB) {
      main_loop(bool_constant<true>{});
    } else {
      main_loop(bool_constant<false>{});
    }
    // no load may still be writing the ring when it is reused or the waves exit
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    // ---- this slice's sums: lane holds channels ch_base + ng*16 + 4*lg + q, row p0 + rb*16 + li
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = p0 + rb * 16 + li;
      if (rb < nrb && r < nrows) {
        const long orow = (long)(row0 + r) * N;
#pragma unroll
        for (int ng = 0; ng < NG; ++ng)
          *reinterpret_cast<f32x4*>(plane + orow + ch_base + ng * 16 + 4 * lg) = acc[rb][ng];
      }
    }
  }
}

// y_rows[r, c] = ((part[0] + part[1]) + ...) + part[KS-1], times the channel
// scale of row r's expert (unscaled encodings: 1); rows of no expert are left
// as they are. One workgroup per (row, 1024 channels), four channels a thread;
// rows run along the grid's x axis (up to 2^26 of them), channel blocks along y.
// kOut 0: the sums go to y_rows (fp32). kOut 1 (bf16) or 2 (fp32): a dense
// layer's output y, written as the combine writes a token with one expert of
// weight 1 (0 + 1 * v, then the act dtype), so the result is the same bit for bit.
template <bool kScaleBf16, bool kScaled, int kOut>
__global__ __launch_bounds__(256) void split_down_reduce_kernel(const float* __restrict__ part, int KS, int S, int N,
                                                                const int32_t* __restrict__ offsets, int E,
                                                                const void* __restrict__ S0,
                                                                void* __restrict__ out) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63;
  int o0 = 0, o1 = 0;
  if (lane < E) {
    o0 = offsets[lane];
    o1 = offsets[lane + 1];
  }
  const uint64_t hit = __ballot(lane < E && r >= o0 && r < o1);
  if (hit == 0) return;   // the same for the whole workgroup
  const int e = __ffsll((unsigned long long)hit) - 1;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= N) return;
  const long o = (long)r * N + c;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + o);
  for (int j = 1; j < KS; ++j) v += *reinterpret_cast<const f32x4*>(part + (long)j * S * N + o);
  if constexpr (kScaled) {
    const float4 sc = load_scale4<kScaleBf16>(S0, (long)e * N + c);
    v = f32x4{v[0] * sc.x, v[1] * sc.y, v[2] * sc.z, v[3] * sc.w};
  }
  if constexpr (kOut == 0) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = v;
  } else {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += 1.0f * v[q];
    if constexpr (kOut == 1) {
      bf16x4 b;
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = (__bf16)acc[q];
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + o) = b;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = acc;
    }
  }
}

template <bool kGateUp, typename Act, bool kScaleBf16, int F, int RB, int KS>
hipError_t launch_stream_pass_ks(const FfnArgs& a, long items, hipStream_t stream) {
  constexpr int NG = kGateUp ? (RB >= 4 ? MOE_STREAM_NG_GU_WIDE : MOE_STREAM_NG_GU)
                             : (RB >= 4 ? MOE_STREAM_NG_DN_WIDE : MOE_STREAM_NG_DN);
  constexpr int P = kGateUp ? ((KS == 1 && RB < 4) ? MOE_STREAM_P_GU_LONG : MOE_STREAM_P_GU) : MOE_STREAM_P_DN;
  const int N = kGateUp ? a.f : a.d;
  const int Kd = kGateUp ? a.d : a.f;
  const dim3 grid((unsigned)(KS > 1 ? items : (items + kStreamWaves - 1) / kStreamWaves));
  const dim3 block(stream_block_waves(KS) * kWave);
  if constexpr (kGateUp) {
    hipLaunchKernelGGL((ffn_stream_kernel<true, Act, kScaleBf16, F, NG, RB, P, KS>), grid, block, 0, stream,
                       static_cast<const Act*>(a.x), a.sorted_slots, a.K, a.w_gate, a.w_up, a.s_gate, a.s_up,
                       a.offsets, a.E, N, Kd, static_cast<void*>(a.h), a.ids, a.S, a.perm_offsets, a.perm_sorted,
                       a.perm_s2r);
  } else {
    hipLaunchKernelGGL((ffn_stream_kernel<false, __bf16, kScaleBf16, F, NG, RB, P, KS>), grid, block, 0, stream,
                       static_cast<const __bf16*>(a.h), a.sorted_slots, a.K, a.w_down, nullptr, a.s_down,
                       nullptr, a.offsets, a.E, N, Kd, static_cast<void*>(a.y_rows), nullptr, a.S, nullptr, nullptr,
                       nullptr);
  }
  return hipGetLastError();
}

template <bool kGateUp, typename Act, bool kScaleBf16, int F, int RB>
hipError_t launch_stream_pass_rb(const FfnArgs& a, hipStream_t stream) {
  constexpr int NG = kGateUp ? (RB >= 4 ? MOE_STREAM_NG_GU_WIDE : MOE_STREAM_NG_GU)
                             : (RB >= 4 ? MOE_STREAM_NG_DN_WIDE : MOE_STREAM_NG_DN);
  const int N = kGateUp ? a.f : a.d;
  const long items = (long)a.E * (N / (16 * NG));
  switch (choose_split(items, RB, kGateUp)) {
    case 1: return launch_stream_pass_ks<kGateUp, Act, kScaleBf16, F, RB, 1>(a, items, stream);
    case 2: return launch_stream_pass_ks<kGateUp, Act, kScaleBf16, F, RB, 2>(a, items, stream);
    case 4: return launch_stream_pass_ks<kGateUp, Act, kScaleBf16, F, RB, 4>(a, items, stream);
    default: return launch_stream_pass_ks<kGateUp, Act, kScaleBf16, F, RB, 8>(a, items, stream);
  }
}

template <bool kScaleBf16, int F, int NG, int WI, int KS, int P>
hipError_t launch_stream_shared_gu_w(const FfnArgs& a, hipStream_t stream) {
  const int gpe = a.f / (16 * NG);
  const dim3 grid((unsigned)((long)a.E * (gpe / WI)));
  hipLaunchKernelGGL((ffn_stream_shared_gu_kernel<kScaleBf16, F, NG, WI, KS, P>), grid,
                     dim3(WI * KS * kWave), 0, stream, static_cast<const __bf16*>(a.x), a.sorted_slots, a.K,
                     a.w_gate, a.w_up, a.s_gate, a.s_up, a.offsets, a.E, a.f, a.d, a.h);
  return hipGetLastError();
}

// Workgroup shape of the shared-activation gate/up pass (ng 16-channel groups
// per item, wi items, reductions cut in ks slices).
//   - Enough items for two 4-wave workgroups per CU: WI = 4 items, no split.
//   - Else, with 48-channel items (f a multiple of 96) of which two per
//     workgroup give every CU a workgroup: WI = 2 items cut in two (KS = 2),
//     four waves, one per SIMD (the dense MLP layer: gate/up 82-84 -> 72-73 us,
//     A/B on one box, where the six-wave shape below leaves two SIMDs with
//     two waves and two with one, and every step waits for the busier ones).
//   - Else, with a third of an expert's 32-channel items giving every CU a
//     workgroup: WI = 3 items with their reductions cut in two, six waves on
//     the four SIMDs, where three unsplit items would leave one SIMD of every
//     CU idle (the dense MLP layer: gate/up 90-96 -> 82-84 us).
//   - Else the most of 4, 3, 2 items that divides an expert's items and still
//     gives every CU a workgroup; 2 always divides (f is a multiple of 64).
// The split shapes need an even number of 64-wide reduction steps and weights
// of one piece per step (int8, fp8); bf16 weights, whose ring of two-piece
// steps does not fit two waves per SIMD, take the three items unsplit.
struct SharedGuShape {
  int ng, wi, ks;
};
SharedGuShape shared_gu_shape(int E, int f, int d, bool one_piece) {
  const int gpe = f / (16 * MOE_STREAM_NG_GU_WIDE);
  const long cus = MOE_STREAM_SHARED_MIN_WGS;
  const bool even = ((d >> 6) % 2) == 0;
  if (gpe % 4 == 0 && (long)E * (gpe / 4) >= 2 * cus) return {MOE_STREAM_NG_GU_WIDE, 4, 1};
  if (one_piece && even && f % 96 == 0 && (long)E * (f / 96) >= cus) return {3, 2, 2};
  if (even && gpe % 3 == 0 && (long)E * (gpe / 3) >= cus) return {MOE_STREAM_NG_GU_WIDE, 3, one_piece ? 2 : 1};
  for (int w = 4; w >= 2; --w)
    if (gpe % w == 0 && (long)E * (gpe / w) >= cus) return {MOE_STREAM_NG_GU_WIDE, w, 1};
  return {MOE_STREAM_NG_GU_WIDE, 2, 1};
}

template <bool kScaleBf16, int F>
hipError_t launch_stream_shared_gu(const FfnArgs& a, hipStream_t stream) {
  constexpr int NG = MOE_STREAM_NG_GU_WIDE;
  constexpr bool kOnePiece = WFormat<F>::kPieces == 1;
  const SharedGuShape sh = shared_gu_shape(a.E, a.f, a.d, kOnePiece);
  if constexpr (kOnePiece) {
    if (sh.ks == 2 && sh.ng == 3)
      return launch_stream_shared_gu_w<kScaleBf16, F, 3, 2, 2, MOE_STREAM_P_SHARED_SPLIT>(a, stream);
    if (sh.ks == 2) return launch_stream_shared_gu_w<kScaleBf16, F, NG, 3, 2, MOE_STREAM_P_SHARED_SPLIT>(a, stream);
  }
  switch (sh.wi) {
    case 4: return launch_stream_shared_gu_w<kScaleBf16, F, NG, 4, 1, MOE_STREAM_P_SHARED>(a, stream);
    case 3: return launch_stream_shared_gu_w<kScaleBf16, F, NG, 3, 1, MOE_STREAM_P_SHARED>(a, stream);
    default: return launch_stream_shared_gu_w<kScaleBf16, F, NG, 2, 1, MOE_STREAM_P_SHARED>(a, stream);
  }
}

// Partial-sum planes the 64-row down pass with a reduction split across
// workgroups needs ([planes, S, d] fp32), or 0 when it is not taken: fewer
// than 33 rows per expert on average, no split, a slice without a step, h
// offsets past 32 bits, or channel groups of an expert that do not fill
// whole workgroups. The split is the one the in-workgroup split of the
// 64-row down pass takes (from its item count), so the two agree bit for bit.
int shared_down_planes(long S, int d, int f, int E) {
  constexpr int NG = MOE_STREAM_NG_SHARED_DN, W = MOE_STREAM_SHARED_DN_WAVES;
  if (!MOE_STREAM_SHARED_DN || S <= 32L * E) return 0;
  if ((uint64_t)S * f * 2 >= (1ull << 32)) return 0;
  if ((d / (16 * NG)) % W || d % (16 * NG)) return 0;
  const int ks = choose_split((long)E * (d / (16 * MOE_STREAM_NG_DN_WIDE)), 4);
  if (ks <= 1 || (f >> 6) < ks) return 0;
  return ks;
}

template <int F, int kOut>
hipError_t launch_split_down_reduce(const FfnArgs& a, int KS, void* out, hipStream_t stream) {
  const dim3 rgrid((unsigned)a.S, (unsigned)((a.d + 1023) / 1024));
  if (!WFormat<F>::kScaled) {
    hipLaunchKernelGGL((split_down_reduce_kernel<true, false, kOut>), rgrid, dim3(256), 0, stream, a.part, KS, a.S,
                       a.d, a.offsets, a.E, a.s_down, out);
  } else if (a.scale_bf16) {
    hipLaunchKernelGGL((split_down_reduce_kernel<true, true, kOut>), rgrid, dim3(256), 0, stream, a.part, KS, a.S,
                       a.d, a.offsets, a.E, a.s_down, out);
  } else {
    hipLaunchKernelGGL((split_down_reduce_kernel<false, true, kOut>), rgrid, dim3(256), 0, stream, a.part, KS, a.S,
                       a.d, a.offsets, a.E, a.s_down, out);
  }
  return hipGetLastError();
}

template <int F>
hipError_t launch_stream_shared_dn(const FfnArgs& a, int KS, hipStream_t stream) {
  constexpr int NG = MOE_STREAM_NG_SHARED_DN, W = MOE_STREAM_SHARED_DN_WAVES;
  const int gpe = a.d / (16 * NG);
  const dim3 grid((unsigned)((long)a.E * (gpe / W) * KS));
  hipLaunchKernelGGL((ffn_stream_shared_dn_kernel<F, NG, W, MOE_STREAM_P_SHARED_DN>), grid, dim3(W * kWave), 0,
                     stream, static_cast<const __bf16*>(a.h), a.w_down, a.offsets, a.E, a.d, a.f, a.S, KS, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.y_dense) return launch_split_down_reduce<F, 0>(a, KS, a.y_rows, stream);
  return a.act_bf16 ? launch_split_down_reduce<F, 1>(a, KS, a.y_dense, stream)
                    : launch_split_down_reduce<F, 2>(a, KS, a.y_dense, stream);
}

// Rows per pass: 16*RB. More than 32 rows per expert on average (a dense MLP
// layer, or a hot expert at decode) takes the 64-row variant so the weights
// are streamed once; otherwise the 32-row variant keeps more waves resident.
// The 64-row gate/up pass with bf16 activations shares them through LDS when
// their byte offsets fit 32 bits; so does the 64-row down pass with a
// reduction split when the caller gives it the partial-sum planes.
template <bool kGateUp, typename Act, bool kScaleBf16, int F>
hipError_t launch_stream_pass(const FfnArgs& a, hipStream_t stream) {
  if (a.ids && !(kGateUp && stream_gate_up_takes_ids(a.S, a.E))) return hipErrorInvalidValue;
  if (!kGateUp && a.y_dense && (a.E != 1 || a.K != 1 || (long)a.S <= 32L * a.E)) return hipErrorInvalidValue;
  if ((long)a.S > 32L * a.E) {
    if constexpr (kGateUp && sizeof(Act) == 2) {
      if (MOE_STREAM_SHARED_GU && (uint64_t)a.T * a.d * 2 < (1ull << 32))
        return launch_stream_shared_gu<kScaleBf16, F>(a, stream);
    }
    if constexpr (!kGateUp) {
      const int planes = shared_down_planes(a.S, a.d, a.f, a.E);
      if (a.part && planes > 0) return launch_stream_shared_dn<F>(a, planes, stream);
      if (a.y_dense) return hipErrorInvalidValue;
    }
    return launch_stream_pass_rb<kGateUp, Act, kScaleBf16, F, 4>(a, stream);
  }
  return launch_stream_pass_rb<kGateUp, Act, kScaleBf16, F, MOE_STREAM_RB>(a, stream);
}

// int8 weights: fp32 or bf16 activations and scales. bf16 and fp8 weights
// (comparators): bf16 activations; fp8 takes either scale dtype.
template <bool kGateUp>
hipError_t dispatch_stream(const FfnArgs& a, hipStream_t stream) {
  switch (a.wfmt) {
    case kWInt8:
      if (a.act_bf16) {
        return a.scale_bf16 ? launch_stream_pass<kGateUp, __bf16, true, kWInt8>(a, stream)
                            : launch_stream_pass<kGateUp, __bf16, false, kWInt8>(a, stream);
      }
      return a.scale_bf16 ? launch_stream_pass<kGateUp, float, true, kWInt8>(a, stream)
                          : launch_stream_pass<kGateUp, float, false, kWInt8>(a, stream);
    case kWBf16:
      if (!a.act_bf16) return hipErrorInvalidValue;
      return launch_stream_pass<kGateUp, __bf16, true, kWBf16>(a, stream);
    case kWFp8:
      if (!a.act_bf16) return hipErrorInvalidValue;
      return a.scale_bf16 ? launch_stream_pass<kGateUp, __bf16, true, kWFp8>(a, stream)
                          : launch_stream_pass<kGateUp, __bf16, false, kWFp8>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

int stream_down_planes(long S, int d, int f, int E) { return shared_down_planes(S, d, f, E); }

bool stream_gate_up_takes_ids(long S, int E) { return S <= (long)kWave * kIdChunks && S <= 32L * E; }

hipError_t launch_stream_gate_up(const FfnArgs& a, hipStream_t stream) { return dispatch_stream<true>(a, stream); }
hipError_t launch_stream_down(const FfnArgs& a, hipStream_t stream) { return dispatch_stream<false>(a, stream); }

}  // namespace moe
