// Expert permutation: histogram of the slot -> expert assignments, exclusive
// scan, and a stable scatter of the slots into contiguous per-expert segments,
// with the inverse map. Grouping the rows of each expert lets the expert FFN
// read each expert's weights once for all of its rows (the paper's serving
// note: batching and fusing the two chosen experts is what saves time, since
// the MoE layer is I/O-bound).
//
// Fewer than 4 chunks of 2048 slots (decode, small batches): one workgroup of
// 16 waves. Wave w owns a contiguous range of slots, walked in 64-slot chunks
// (the ids of 8 chunks loaded together). Pass 1 counts, per chunk and expert,
// the lanes whose id matches (a ballot and a popcount), accumulated by the
// lane that owns that expert. The 16 x E counts are scanned
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

// ---------------------------------------------------------------------------
// Many slots (prefill): the same permutation from three short kernels over
// chunks of kChunkSlots slots, so that every CU can take part instead of one.
//   1. count: block b counts the slots of chunk b per expert (the 4 waves of
//      the block each take a quarter of the chunk) and stores the counts in
//      the tail of sorted_slots, cnt[b][e] at sorted_slots[S - B*E + b*E + e]
//      (sorted_slots is rewritten in full by step 3);
//   2. place: block b sums the counts of every chunk: expert e starts at the
//      total of the experts before it, chunk b's slots of expert e after those
//      of the chunks before b; inside the chunk, wave by wave and lane by lane
//      as in the one-workgroup kernel. It writes slot_to_row (block 0 also
//      offsets);
//   3. invert: sorted_slots[slot_to_row[s]] = s, and -1 for the rows past the
//      placed slots.
// The positions are the ones the one-workgroup kernel gives (experts in index
// order, slots ascending inside an expert), bit for bit.
constexpr int kChunkWaves = 4;
constexpr int kChunkSlots = 2048;   // 8 64-slot groups per wave
constexpr int kChunkGroups = kChunkSlots / kWave / kChunkWaves;

// per-wave counts of chunk b: lane e of wave w ends with the count of expert e
// in the wave's quarter of the chunk
__device__ __forceinline__ int chunk_wave_count(const int32_t* __restrict__ ids, int S, int E, int s_begin,
                                                int lane) {
  int idv[kChunkGroups];
#pragma unroll
  for (int g = 0; g < kChunkGroups; ++g) {
    const int s = s_begin + 64 * g + lane;
    idv[g] = (s < S) ? ids[s] : -1;
  }
  int my_count = 0;
#pragma unroll
  for (int g = 0; g < kChunkGroups; ++g) {
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(idv[g] == e);
      if (lane == e) my_count += __popcll(m);
    }
  }
  return my_count;
}

__global__ __launch_bounds__(kChunkWaves * kWave) void permute_count_kernel(const int32_t* __restrict__ ids, int S,
                                                                            int E, int32_t* __restrict__ sorted_slots) {
  __shared__ int wc[kChunkWaves][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int B = gridDim.x;
  const int s_begin = blockIdx.x * kChunkSlots + wave * (kChunkSlots / kChunkWaves);
  wc[wave][lane] = chunk_wave_count(ids, S, E, s_begin, lane);
  __syncthreads();
  if (threadIdx.x < E) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) c += wc[w][threadIdx.x];
    sorted_slots[(long)S - (long)B * E + (long)blockIdx.x * E + threadIdx.x] = c;
  }
}

__global__ __launch_bounds__(kChunkWaves * kWave) void permute_place_kernel(const int32_t* __restrict__ ids, int S,
                                                                            int E, const int32_t* __restrict__ cnt,
                                                                            int32_t* __restrict__ offsets,
                                                                            int32_t* __restrict__ slot_to_row) {
  __shared__ int wc[kChunkWaves][kMaxExperts];
  __shared__ int chunk_base[kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int B = gridDim.x, b = blockIdx.x;
  const int s_begin = b * kChunkSlots + wave * (kChunkSlots / kChunkWaves);
  wc[wave][lane] = chunk_wave_count(ids, S, E, s_begin, lane);
  if (wave == 0) {
    // lane e: the total of expert e over all chunks and over the chunks before b
    int tot = 0, before = 0;
    if (lane < E) {
      for (int c = 0; c < B; ++c) {
        const int v = cnt[(long)c * E + lane];
        tot += v;
        if (c < b) before += v;
      }
    }
    int incl = tot;   // exclusive scan of the totals over the experts
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int n = __shfl_up(incl, off);
      if (lane >= off) incl += n;
    }
    if (lane < E) {
      chunk_base[lane] = incl - tot + before;
      if (b == 0) offsets[lane] = incl - tot;
    }
    if (b == 0 && lane == 63) offsets[E] = incl;   // lanes past E add nothing
  }
  __syncthreads();
  // this wave's base per expert: the chunk's base plus the earlier waves' counts
  int my_base = 0;
  if (lane < E) {
    my_base = chunk_base[lane];
    for (int w = 0; w < wave; ++w) my_base += wc[w][lane];
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int idv[kChunkGroups];
#pragma unroll
  for (int g = 0; g < kChunkGroups; ++g) {
    const int s = s_begin + 64 * g + lane;
    idv[g] = (s < S) ? ids[s] : -1;
  }
#pragma unroll
  for (int g = 0; g < kChunkGroups; ++g) {
    const int s = s_begin + 64 * g + lane;
    const int id = idv[g];
    int pos = -1;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(id == e);
      const int bs = __builtin_amdgcn_readlane(my_base, e);
      if (id == e) pos = bs + __popcll(m & below);
      if (lane == e) my_base += __popcll(m);
    }
    if (s < S) slot_to_row[s] = pos;
  }
}

__global__ void permute_invert_kernel(int S, int E, const int32_t* __restrict__ offsets,
                                      const int32_t* __restrict__ slot_to_row, int32_t* __restrict__ sorted_slots) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  const int r = slot_to_row[s];
  if (r >= 0) sorted_slots[r] = s;
  if (s >= offsets[E]) sorted_slots[s] = -1;   // rows past the placed slots (ids out of range)
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int S, int E, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_to_row, hipStream_t stream) {
  const int B = (S + kChunkSlots - 1) / kChunkSlots;
  if (B < 4 || (long)B * E > S) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermWaves * kWave), 0, stream, ids, S, E, offsets,
                       sorted_slots, slot_to_row);
    return hipGetLastError();
  }
  const int32_t* cnt = sorted_slots + ((long)S - (long)B * E);
  hipLaunchKernelGGL(permute_count_kernel, dim3(B), dim3(kChunkWaves * kWave), 0, stream, ids, S, E, sorted_slots);
  hipLaunchKernelGGL(permute_place_kernel, dim3(B), dim3(kChunkWaves * kWave), 0, stream, ids, S, E, cnt, offsets,
                     slot_to_row);
  hipLaunchKernelGGL(permute_invert_kernel, dim3((S + 255) / 256), dim3(256), 0, stream, S, E, offsets, slot_to_row,
                     sorted_slots);
  return hipGetLastError();
}

}  // namespace moe
