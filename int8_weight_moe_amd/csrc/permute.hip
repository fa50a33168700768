// Expert permutation: histogram of the slot -> expert assignments, exclusive
// scan, and a stable scatter of the slots into contiguous per-expert segments,
// with the inverse map. Grouping the rows of each expert lets the expert FFN
// read each expert's weights once for all of its rows (the paper's serving
// note: batching and fusing the two chosen experts is what saves time, since
// the MoE layer is I/O-bound).
//
// One workgroup of 16 waves. Wave w owns a contiguous range of slots, walked
// in 64-slot chunks (the ids of 8 chunks loaded together). Pass 1 counts, per
// chunk and expert, the lanes whose id matches (a ballot and a popcount),
// accumulated by the lane that owns that expert. The 16 x E counts are scanned
// in a fixed order (expert-major, then wave) by the whole workgroup, one count
// per thread. Pass 2 walks the same chunks again and gives each slot its
// position: the expert's running base plus the number of matching lanes below
// it in the ballot. Slots therefore keep ascending order inside an expert, and
// the result is bit-exact and independent of scheduling.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kPermWaves = 16;
constexpr int kMaxExperts = 64;
constexpr int kBatch = 8;   // 64-slot chunks whose ids a wave loads at once

__global__ __launch_bounds__(kPermWaves * kWave) void permute_kernel(const int32_t* __restrict__ ids, int S, int E,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_slots,
                                                                     int32_t* __restrict__ slot_to_row) {
  __shared__ int cnt[kPermWaves][kMaxExperts];
  __shared__ int base[kPermWaves][kMaxExperts];
  __shared__ int wave_total[kPermWaves];
  __shared__ int total_valid;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // contiguous slot range of this wave, a whole number of 64-slot chunks
  const int chunks_total = (S + 63) >> 6;
  const int chunks_per_wave = (chunks_total + kPermWaves - 1) / kPermWaves;
  const int s_begin = wave * chunks_per_wave * 64;
  const int s_end = min(S, s_begin + chunks_per_wave * 64);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  int my_count = 0;  // lane e counts expert e
  for (int s0 = s_begin; s0 < s_end; s0 += 64 * kBatch) {
    int idv[kBatch];   // the batch's ids are loaded together: one memory latency per batch
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = s0 + 64 * b + lane;
      idv[b] = (s < s_end) ? ids[s] : -1;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (s0 + 64 * b >= s_end) break;   // past this wave's range (the same for the whole wave)
      for (int e = 0; e < E; ++e) {
        const uint64_t m = __ballot(idv[b] == e);
        if (lane == e) my_count += __popcll(m);
      }
    }
  }
  cnt[wave][lane] = my_count;
  __syncthreads();

  // Exclusive scan of the counts in (expert, wave) order, one value per
  // thread: thread t holds cnt[t % 16][t / 16]. A shuffle scan inside each
  // wave, then the wave totals through LDS.
  {
    const int t = threadIdx.x;
    const int se = t >> 4, sw = t & 15;
    const int v = (se < E) ? cnt[sw][se] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int n = __shfl_up(incl, off);
      if (lane >= off) incl += n;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int woff = 0;
    for (int j = 0; j < wave; ++j) woff += wave_total[j];
    const int excl = woff + incl - v;
    if (se < E) {
      base[sw][se] = excl;
      if (sw == 0) offsets[se] = excl;
    }
    if (t == kPermWaves * kWave - 1) {   // holds the grand total (values past E are 0)
      offsets[E] = woff + incl;
      total_valid = woff + incl;
    }
  }
  __syncthreads();

  int my_base = (lane < E) ? base[wave][lane] : 0;
  for (int s0 = s_begin; s0 < s_end; s0 += 64 * kBatch) {
    int idv[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = s0 + 64 * b + lane;
      idv[b] = (s < s_end) ? ids[s] : -1;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (s0 + 64 * b >= s_end) break;   // past this wave's range (the same for the whole wave)
      const int s = s0 + 64 * b + lane;
      const int id = idv[b];
      int pos = -1;
      for (int e = 0; e < E; ++e) {
        const uint64_t m = __ballot(id == e);
        const int bs = __builtin_amdgcn_readlane(my_base, e);   // e is uniform: a scalar read of lane e
        if (id == e) pos = bs + __popcll(m & below);
        if (lane == e) my_base += __popcll(m);
      }
      if (s < s_end) {
        slot_to_row[s] = pos;
        if (pos >= 0) sorted_slots[pos] = s;
      }
    }
  }
  // rows past the placed slots (only when some id was out of range)
  for (int r = total_valid + threadIdx.x; r < S; r += blockDim.x) sorted_slots[r] = -1;
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int S, int E, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_to_row, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermWaves * kWave), 0, stream, ids, S, E, offsets,
                     sorted_slots, slot_to_row);
  return hipGetLastError();
}

}  // namespace moe
