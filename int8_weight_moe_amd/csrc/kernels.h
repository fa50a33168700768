// Launchers of the gfx950 kernels (host side). Arguments are validated by the
// C ABI layer before any of these is called; each returns the HIP status of
// its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

hipError_t launch_router(const void* x, const void* router_w, const float* bias, int T, int d, int E, int K,
                         bool act_bf16, int32_t* topk_ids, float* topk_w, hipStream_t stream);

hipError_t launch_permute(const int32_t* ids, int S, int E, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_to_row, hipStream_t stream);

// Arguments of the expert FFN (both schedules).
struct FfnArgs {
  const void* x;              // [T, d] activations
  bool act_bf16;              // x dtype
  bool scale_bf16;            // scale dtype
  const int32_t* offsets;     // [E + 1]
  const int32_t* sorted_slots;  // [S]
  int wfmt;                   // weight encoding (WFmt: int8, bf16 or fp8)
  const int8_t* w_gate;       // [E, f, d], tiled layout of the weight bytes
  const int8_t* w_up;         // [E, f, d], tiled layout of the weight bytes
  const int8_t* w_down;       // [E, d, f], tiled layout of the weight bytes
  const void* s_gate;         // [E, f] (unused for bf16 weights)
  const void* s_up;           // [E, f]
  const void* s_down;         // [E, d]
  __bf16* h;                  // [S, f] scratch
  float* y_rows;              // [S, d] out
  float* part;                // [planes, S, d] scratch of a down pass split over workgroups, or null
  // A dense layer (E = K = 1, every token its own row with weight 1) whose
  // down pass splits its reduction over workgroups: the sum of the slices goes
  // straight to y ([T, d], act dtype), as the combine would write it, and
  // y_rows is not written. Null otherwise.
  void* y_dense;
  // gate/up from the expert ids (S <= 256, 32-row stream pass): ids [S] in,
  // the permutation (offsets, sorted_slots, slot_to_row) out; null otherwise
  const int32_t* ids;
  int32_t* perm_offsets;
  int32_t* perm_sorted;
  int32_t* perm_s2r;
  // tile claim words of the tiled gate/up and down passes ([8] each, zeroed by
  // the pass before use), or null: the static tile order throughout
  unsigned long long* claims_gate_up;
  unsigned long long* claims_down;
  int T, d, f, E, K, S;
};

// Bytes of one tiled pass's tile claim words (eight 64-bit words, padded).
constexpr size_t kTileClaimBytes = 256;

// Weight-streaming schedule for few rows per expert (decode): gate/up pass
// (x -> h) and down pass (h -> y_rows).
hipError_t launch_stream_gate_up(const FfnArgs& a, hipStream_t stream);
hipError_t launch_stream_down(const FfnArgs& a, hipStream_t stream);
// Partial-sum planes ([planes, S, d] fp32, in FfnArgs::part) with which the
// stream down pass splits its reduction over workgroups; 0: it does not. With
// part null the pass keeps the split inside one workgroup, with the same result.
int stream_down_planes(long S, int d, int f, int E);
// Whether the stream gate/up pass can take the expert ids instead of a
// permutation (FfnArgs::ids): at most 256 slots on the 32-row variant.
bool stream_gate_up_takes_ids(long S, int E);
// Tiled MFMA schedule for many rows per expert (prefill). bf16 and fp8
// weights need bf16 activations and dma_offsets_fit(T, S, d, f, bytes per
// weight); int8 weights take any shape.
bool dma_offsets_fit(long T, long S, long d, long f, int wbytes);
hipError_t launch_tiled_gate_up(const FfnArgs& a, hipStream_t stream);
hipError_t launch_tiled_down(const FfnArgs& a, hipStream_t stream);

hipError_t launch_combine(const float* y_rows, const int32_t* slot_to_row, const float* topk_w, int T, int d,
                          int K, bool act_bf16, void* y, hipStream_t stream);

hipError_t launch_dense_init(int T, int32_t* offsets, int32_t* sorted_slots, int32_t* slot_to_row, float* w,
                             hipStream_t stream);

hipError_t launch_pack_rows(long rows, int cols, const int8_t* src, int8_t* dst, hipStream_t stream);

// int8 codes (fp8 = false) or OCP e4m3 code bytes (fp8 = true), row-major or
// in the tiled layout (tiled = true: rows % 16 == 0, cols % 64 == 0)
hipError_t launch_quantize_rows(int64_t rows, int cols, bool src_bf16, const void* w, bool scale_bf16, int8_t* q,
                                void* s, bool fp8, bool tiled, hipStream_t stream);

}  // namespace moe
