// C ABI of libmoe_int8: argument validation, workspace layout and the
// enqueueing of the kernels. Nothing here allocates device memory or
// synchronises, except the checks that MOE_DEBUG turns on.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_int8.h"
#include "debug_checks.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- MOE_DEBUG: permutation checks on the host (debug runs only)

// Set and not "0" at the time of the call.
bool debug_on() {
  const char* v = getenv("MOE_DEBUG");
  return v && v[0] && strcmp(v, "0") != 0;
}

// n int32 values from the device, after the work already enqueued on `stream`.
moe_status fetch_ints(const int32_t* dev, long n, std::vector<int32_t>& out, hipStream_t stream) {
  out.assign((size_t)n, 0);
  if (n <= 0) return MOE_OK;
  hipError_t e = hipMemcpyAsync(out.data(), dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "MOE_DEBUG copy to the host");
}

moe_status debug_verdict(const std::string& m, const char* what) {
  return m.empty() ? MOE_OK : fail(MOE_ERR_CHECK, "MOE_DEBUG %s: %s", what, m.c_str());
}

// A caller's segment offsets and, when `sorted` is given, the slots of the
// rows they cover.
moe_status debug_inputs(const moe_shape* s, const int32_t* offsets, const int32_t* sorted, hipStream_t stream) {
  const long S = (long)s->T * s->K;
  std::vector<int32_t> off, srt;
  moe_status st = fetch_ints(offsets, s->E + 1, off, stream);
  if (st != MOE_OK) return st;
  st = debug_verdict(moe_debug::check_offsets(off.data(), s->E, S), "expert_offsets");
  if (st != MOE_OK || !sorted) return st;
  if ((st = fetch_ints(sorted, off[s->E], srt, stream)) != MOE_OK) return st;
  return debug_verdict(moe_debug::check_sorted(srt.data(), off[s->E], S), "sorted_slots");
}

// A caller's slot_to_row.
moe_status debug_rows(const moe_shape* s, const int32_t* s2r, hipStream_t stream) {
  const long S = (long)s->T * s->K;
  std::vector<int32_t> rows;
  moe_status st = fetch_ints(s2r, S, rows, stream);
  if (st != MOE_OK) return st;
  return debug_verdict(moe_debug::check_rows(rows.data(), S), "slot_to_row");
}

// The permutation the library produced from the expert ids.
moe_status debug_permutation(const moe_shape* s, const int32_t* ids, const int32_t* offsets, const int32_t* sorted,
                             const int32_t* s2r, hipStream_t stream) {
  const long S = (long)s->T * s->K;
  std::vector<int32_t> i, off, srt, rows;
  moe_status st;
  if ((st = fetch_ints(ids, S, i, stream)) != MOE_OK) return st;
  if ((st = fetch_ints(offsets, s->E + 1, off, stream)) != MOE_OK) return st;
  if ((st = fetch_ints(sorted, S, srt, stream)) != MOE_OK) return st;
  if ((st = fetch_ints(s2r, S, rows, stream)) != MOE_OK) return st;
  return debug_verdict(moe_debug::check_permutation(i.data(), off.data(), srt.data(), rows.data(), s->E, S),
                       "permutation");
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Rows at or below this many per expert (on average) go to the weight-streaming schedule.
constexpr long kStreamRowsPerExpert = 64;

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_NULL, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_SHAPE, "T=%d must be >= 0", s->T);
  if (s->d < 64 || s->d > 65536 || s->d % 64) return fail(MOE_ERR_SHAPE, "d=%d must be a multiple of 64 in [64, 65536]", s->d);
  if (s->f < 64 || s->f > 131072 || s->f % 64) return fail(MOE_ERR_SHAPE, "f=%d must be a multiple of 64 in [64, 131072]", s->f);
  if (s->E < 1 || s->E > 64) return fail(MOE_ERR_SHAPE, "E=%d must be in [1, 64]", s->E);
  if (s->K < 1 || s->K > s->E || s->K > 8) return fail(MOE_ERR_SHAPE, "K=%d must be in [1, min(E, 8)]", s->K);
  if ((long)s->T * s->K > (1L << 26)) return fail(MOE_ERR_SHAPE, "T*K=%ld exceeds 2^26", (long)s->T * s->K);
  if (s->act_dtype != MOE_F32 && s->act_dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "act_dtype=%d", s->act_dtype);
  if (s->scale_dtype != MOE_F32 && s->scale_dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "scale_dtype=%d", s->scale_dtype);
  if (s->ffn_path < MOE_PATH_AUTO || s->ffn_path > MOE_PATH_TILED) return fail(MOE_ERR_SHAPE, "ffn_path=%d", s->ffn_path);
  if (s->weight_fmt < MOE_W_INT8 || s->weight_fmt > MOE_W_FP8) return fail(MOE_ERR_DTYPE, "weight_fmt=%d", s->weight_fmt);
  return MOE_OK;
}

#define REQUIRE_PTR(p)                                                         \
  do {                                                                         \
    if (!(p)) return fail(MOE_ERR_NULL, "%s is NULL", #p);                     \
    if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

// Scales are read for the scaled weight encodings (int8, fp8) only.
#define REQUIRE_SCALE(s, p)                                                    \
  do {                                                                         \
    if ((s)->weight_fmt != MOE_W_BF16) REQUIRE_PTR(p);                         \
  } while (0)

struct WsLayout {
  size_t ids, w, offsets, sorted, s2r, h, y_rows, part, part_bytes, claims, total;
};

bool use_stream(const moe_shape* s);
size_t down_ws_bytes(const moe_shape* s);

WsLayout forward_layout(const moe_shape* s) {
  const size_t S = (size_t)s->T * s->K;
  WsLayout L;
  size_t o = 0;
  L.ids = o;     o += round_up(S * 4);
  L.w = o;       o += round_up(S * 4);
  L.offsets = o; o += round_up((s->E + 1) * 4);
  L.sorted = o;  o += round_up(S * 4);
  L.s2r = o;     o += round_up(S * 4);
  L.h = o;       o += round_up(S * (size_t)s->f * 2);
  L.y_rows = o;  o += round_up(S * (size_t)s->d * 4);
  // partial sums of a stream down pass split over workgroups (none otherwise)
  L.part_bytes = use_stream(s) ? down_ws_bytes(s) : 0;
  L.part = o;    o += round_up(L.part_bytes);
  // tile claim words of the tiled gate/up and down passes (none for the stream schedule)
  L.claims = o;  o += use_stream(s) ? 0 : 2 * moe::kTileClaimBytes;
  L.total = o;
  return L;
}

// Workspace of the down pass: the stream schedule's fp32 partial sums of a
// reduction split over workgroups ([planes, S, d]; 0 bytes if it does not
// split), or the tiled schedule's tile claim words.
size_t down_ws_bytes(const moe_shape* s) {
  if (!use_stream(s)) return moe::kTileClaimBytes;
  const long S = (long)s->T * s->K;
  const int planes = moe::stream_down_planes(S, s->d, s->f, s->E);
  return (size_t)planes * (size_t)S * (size_t)s->d * 4;
}

// Workspace of the gate/up pass: the tiled schedule's tile claim words.
size_t gate_up_ws_bytes(const moe_shape* s) { return use_stream(s) ? 0 : moe::kTileClaimBytes; }

// moe_expert_ffn: h, then the down pass's workspace, then the gate/up pass's
size_t ffn_h_bytes(const moe_shape* s) { return round_up((size_t)s->T * s->K * (size_t)s->f * 2); }
size_t ffn_ws_bytes(const moe_shape* s) {
  return ffn_h_bytes(s) + round_up(down_ws_bytes(s)) + round_up(gate_up_ws_bytes(s));
}

bool use_stream(const moe_shape* s) {
  if (s->ffn_path == MOE_PATH_STREAM) return true;
  if (s->ffn_path == MOE_PATH_TILED) return false;
  return (long)s->T * s->K <= kStreamRowsPerExpert * s->E;
}

// What the FFN kernels accept beyond check_shape: the bf16 and fp8 weight
// encodings run with bf16 activations, and their tiled schedule addresses
// with 32-bit offsets.
moe_status check_ffn(const moe_shape* s) {
  if (s->weight_fmt == MOE_W_INT8) return MOE_OK;
  if (s->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "weight_fmt=%d needs bf16 activations", s->weight_fmt);
  const int wbytes = s->weight_fmt == MOE_W_BF16 ? 2 : 1;
  if (!use_stream(s) && !moe::dma_offsets_fit(s->T, (long)s->T * s->K, s->d, s->f, wbytes))
    return fail(MOE_ERR_UNSUPPORTED, "weight_fmt=%d: tensors too large for the tiled schedule", s->weight_fmt);
  return MOE_OK;
}

moe::FfnArgs ffn_args(const moe_shape* s, const void* x, const int32_t* offsets, const int32_t* sorted_slots,
                      const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                      const void* s_up, const void* s_down, float* y_rows, __bf16* h) {
  moe::FfnArgs a;
  a.x = x;
  a.act_bf16 = s->act_dtype == MOE_BF16;
  a.scale_bf16 = s->scale_dtype == MOE_BF16;
  a.offsets = offsets;
  a.sorted_slots = sorted_slots;
  a.wfmt = s->weight_fmt;
  a.w_gate = static_cast<const int8_t*>(w_gate);
  a.w_up = static_cast<const int8_t*>(w_up);
  a.w_down = static_cast<const int8_t*>(w_down);
  a.s_gate = s_gate;
  a.s_up = s_up;
  a.s_down = s_down;
  a.h = h;
  a.y_rows = y_rows;
  a.part = nullptr;
  a.y_dense = nullptr;
  a.ids = nullptr;
  a.perm_offsets = a.perm_sorted = a.perm_s2r = nullptr;
  a.claims_gate_up = a.claims_down = nullptr;
  a.T = s->T;
  a.d = s->d;
  a.f = s->f;
  a.E = s->E;
  a.K = s->K;
  a.S = s->T * s->K;
  return a;
}

// ---- MOE_LOG: one line per FFN pass on stderr, naming the schedule it takes

// Set and not "0" at the time of the call.
bool log_on() {
  const char* v = getenv("MOE_LOG");
  return v && v[0] && strcmp(v, "0") != 0;
}

void log_pass(const char* call, bool gate_up, const moe_shape* s, const moe::FfnArgs& a) {
  const long S = (long)s->T * s->K;
  char how[192];
  if (!use_stream(s)) {
    snprintf(how, sizeof(how), "tiled schedule, %s",
             (gate_up ? a.claims_gate_up : a.claims_down) ? "the last tiles of each XCD queue claimed"
                                                          : "static tile order");
  } else if (gate_up) {
    snprintf(how, sizeof(how), "stream schedule, %d-row passes, expert segments %s", S > 32L * s->E ? 64 : 32,
             a.ids ? "derived from the expert ids (permutation written by the pass)" : "read from the permutation");
  } else {
    const int planes = moe::stream_down_planes(S, s->d, s->f, s->E);
    if (a.part && planes > 0) {
      snprintf(how, sizeof(how), "stream schedule, reduction split over workgroups in %d slices%s", planes,
               a.y_dense ? ", their sum written to y (combine folded in)" : "");
    } else {
      snprintf(how, sizeof(how), "stream schedule, %d-row passes, reduction inside the workgroup",
               S > 32L * s->E ? 64 : 32);
    }
  }
  static const char* const kFmt[] = {"int8", "bf16", "fp8"};
  fprintf(stderr, "[moe] %s %s: T=%d d=%d f=%d E=%d K=%d act=%s scale=%s weights=%s; %s\n", call,
          gate_up ? "gate/up" : "down", s->T, s->d, s->f, s->E, s->K, s->act_dtype == MOE_BF16 ? "bf16" : "f32",
          s->scale_dtype == MOE_BF16 ? "bf16" : "f32", kFmt[s->weight_fmt], how);
}

moe_status run_gate_up(const char* call, const moe_shape* s, const moe::FfnArgs& a, hipStream_t stream) {
  if (log_on()) log_pass(call, true, s, a);
  const hipError_t e = use_stream(s) ? moe::launch_stream_gate_up(a, stream) : moe::launch_tiled_gate_up(a, stream);
  if (e != hipSuccess) return hip_fail(e, "gate/up launch");
  return MOE_OK;
}

moe_status run_down(const char* call, const moe_shape* s, const moe::FfnArgs& a, hipStream_t stream) {
  if (log_on()) log_pass(call, false, s, a);
  const hipError_t e = use_stream(s) ? moe::launch_stream_down(a, stream) : moe::launch_tiled_down(a, stream);
  if (e != hipSuccess) return hip_fail(e, "down launch");
  return MOE_OK;
}

moe_status check_quantize(int64_t rows, int32_t cols, int32_t src_dtype, const void* w, int32_t scale_dtype,
                          const void* q, const void* s) {
  if (rows < 0 || rows > 0x7fffffffL) return fail(MOE_ERR_SHAPE, "rows=%ld must be in [0, 2^31)", (long)rows);
  if (cols < 16 || cols > (1 << 20) || cols % 16) return fail(MOE_ERR_SHAPE, "cols=%d must be a multiple of 16 in [16, 2^20]", cols);
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "src_dtype=%d", src_dtype);
  if (scale_dtype != MOE_F32 && scale_dtype != MOE_BF16) return fail(MOE_ERR_DTYPE, "scale_dtype=%d", scale_dtype);
  REQUIRE_PTR(w);
  REQUIRE_PTR(q);
  if (!s) return fail(MOE_ERR_NULL, "s is NULL");
  if ((reinterpret_cast<uintptr_t>(s) & 3u) != 0) return fail(MOE_ERR_ALIGN, "s is not 4-byte aligned");
  return MOE_OK;
}

// ---------------------------------------------------------------- fixed scratch of moe_forward_noalloc
// The allocation-free entry point keeps its workspace in this file-scope
// device array. Each GPU the library runs on holds its own copy until the
// process ends. In host code the name stands for a host-side shadow, not a
// device address: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB: the decode-sized layers
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

moe_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the library's %d", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

moe_status forward_impl(const char* call, const moe_shape* s, const void* x, const void* router_w,
                       const float* router_bias, const void* w_gate, const void* w_up, const void* w_down,
                       const void* s_gate, const void* s_up, const void* s_down, void* y, int32_t* topk_ids_out,
                       float* topk_w_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_ffn(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(x);
  REQUIRE_PTR(router_w);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_down);
  REQUIRE_SCALE(s, s_gate);
  REQUIRE_SCALE(s, s_up);
  REQUIRE_SCALE(s, s_down);
  REQUIRE_PTR(y);
  REQUIRE_PTR(workspace);
  if (router_bias && !aligned16(router_bias)) return fail(MOE_ERR_ALIGN, "router_bias is not 16-byte aligned");
  if (topk_ids_out && !aligned16(topk_ids_out)) return fail(MOE_ERR_ALIGN, "topk_ids_out is not 16-byte aligned");
  if (topk_w_out && !aligned16(topk_w_out)) return fail(MOE_ERR_ALIGN, "topk_w_out is not 16-byte aligned");
  const WsLayout L = forward_layout(s);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* s2r = reinterpret_cast<int32_t*>(ws + L.s2r);
  __bf16* h = reinterpret_cast<__bf16*>(ws + L.h);
  float* y_rows = reinterpret_cast<float*>(ws + L.y_rows);

  hipError_t e = moe::launch_router(x, router_w, router_bias, s->T, s->d, s->E, s->K, s->act_dtype == MOE_BF16,
                                    ids, wts, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  moe::FfnArgs a = ffn_args(s, x, offsets, sorted, w_gate, w_up, w_down, s_gate, s_up, s_down, y_rows, h);
  if (L.part_bytes) a.part = reinterpret_cast<float*>(ws + L.part);
  if (!use_stream(s)) {
    a.claims_gate_up = reinterpret_cast<unsigned long long*>(ws + L.claims);
    a.claims_down = reinterpret_cast<unsigned long long*>(ws + L.claims + moe::kTileClaimBytes);
  }
  if (use_stream(s) && moe::stream_gate_up_takes_ids((long)s->T * s->K, s->E)) {
    // at most 256 slots: the gate/up pass derives the permutation from the ids
    // and writes it for the down pass and the combine (one launch fewer)
    a.ids = ids;
    a.perm_offsets = offsets;
    a.perm_sorted = sorted;
    a.perm_s2r = s2r;
    st = run_gate_up(call, s, a, stream);
    a.ids = nullptr;
    if (st == MOE_OK && debug_on()) st = debug_permutation(s, ids, offsets, sorted, s2r, stream);
  } else {
    e = moe::launch_permute(ids, s->T * s->K, s->E, offsets, sorted, s2r, stream);
    if (e != hipSuccess) return hip_fail(e, "permute launch");
    if (debug_on()) {
      st = debug_permutation(s, ids, offsets, sorted, s2r, stream);
      if (st != MOE_OK) return st;
    }
    st = run_gate_up(call, s, a, stream);
  }
  if (st != MOE_OK) return st;
  st = run_down(call, s, a, stream);
  if (st != MOE_OK) return st;
  e = moe::launch_combine(y_rows, s2r, wts, s->T, s->d, s->K, s->act_dtype == MOE_BF16, y, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported request";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_CHECK: return "MOE_DEBUG check failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = forward_layout(shape).total;
  return MOE_OK;
}

moe_status moe_ffn_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = ffn_ws_bytes(shape);
  return MOE_OK;
}

moe_status moe_route(const moe_shape* s, const void* x, const void* router_w, const float* router_bias,
                     int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(x);
  REQUIRE_PTR(router_w);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_w);
  if (router_bias && !aligned16(router_bias)) return fail(MOE_ERR_ALIGN, "router_bias is not 16-byte aligned");
  const hipError_t e = moe::launch_router(x, router_w, router_bias, s->T, s->d, s->E, s->K,
                                          s->act_dtype == MOE_BF16, topk_ids, topk_w, stream);
  if (e != hipSuccess) return hip_fail(e, "router launch");
  return MOE_OK;
}

moe_status moe_permute(const moe_shape* s, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* sorted_slots, int32_t* slot_to_row, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots);
  REQUIRE_PTR(slot_to_row);
  const hipError_t e = moe::launch_permute(topk_ids, s->T * s->K, s->E, expert_offsets, sorted_slots,
                                           slot_to_row, stream);
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  if (debug_on()) return debug_permutation(s, topk_ids, expert_offsets, sorted_slots, slot_to_row, stream);
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_shape* s, const void* x, const int32_t* expert_offsets,
                          const int32_t* sorted_slots, const void* w_gate, const void* w_up,
                          const void* w_down, const void* s_gate, const void* s_up, const void* s_down,
                          float* y_rows, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_ffn(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(x);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_down);
  REQUIRE_SCALE(s, s_gate);
  REQUIRE_SCALE(s, s_up);
  REQUIRE_SCALE(s, s_down);
  REQUIRE_PTR(y_rows);
  REQUIRE_PTR(workspace);
  const size_t need = ffn_ws_bytes(s);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, need);
  if (debug_on() && (st = debug_inputs(s, expert_offsets, sorted_slots, stream)) != MOE_OK) return st;
  moe::FfnArgs a = ffn_args(s, x, expert_offsets, sorted_slots, w_gate, w_up, w_down, s_gate, s_up, s_down, y_rows,
                            static_cast<__bf16*>(workspace));
  char* dws = static_cast<char*>(workspace) + ffn_h_bytes(s);
  if (use_stream(s)) {
    if (down_ws_bytes(s)) a.part = reinterpret_cast<float*>(dws);
  } else {
    a.claims_down = reinterpret_cast<unsigned long long*>(dws);
    a.claims_gate_up = reinterpret_cast<unsigned long long*>(dws + round_up(down_ws_bytes(s)));
  }
  st = run_gate_up("moe_expert_ffn", s, a, stream);
  if (st != MOE_OK) return st;
  return run_down("moe_expert_ffn", s, a, stream);
}

moe_status moe_expert_gate_up(const moe_shape* s, const void* x, const int32_t* expert_offsets,
                              const int32_t* sorted_slots, const void* w_gate, const void* w_up,
                              const void* s_gate, const void* s_up, void* h, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_ffn(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(x);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(sorted_slots);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_up);
  REQUIRE_SCALE(s, s_gate);
  REQUIRE_SCALE(s, s_up);
  REQUIRE_PTR(h);
  const size_t need = gate_up_ws_bytes(s);
  if (workspace) {
    if (!aligned16(workspace)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, need);
  }
  if (debug_on() && (st = debug_inputs(s, expert_offsets, sorted_slots, stream)) != MOE_OK) return st;
  moe::FfnArgs a = ffn_args(s, x, expert_offsets, sorted_slots, w_gate, w_up, nullptr, s_gate, s_up, nullptr,
                            nullptr, static_cast<__bf16*>(h));
  if (workspace && need) a.claims_gate_up = static_cast<unsigned long long*>(workspace);
  return run_gate_up("moe_expert_gate_up", s, a, stream);
}

moe_status moe_expert_down(const moe_shape* s, const void* h, const int32_t* expert_offsets, const void* w_down,
                           const void* s_down, float* y_rows, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_ffn(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(h);
  REQUIRE_PTR(expert_offsets);
  REQUIRE_PTR(w_down);
  REQUIRE_SCALE(s, s_down);
  REQUIRE_PTR(y_rows);
  const size_t need = down_ws_bytes(s);
  if (workspace) {
    if (!aligned16(workspace)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, need);
  }
  if (debug_on() && (st = debug_inputs(s, expert_offsets, nullptr, stream)) != MOE_OK) return st;
  moe::FfnArgs a = ffn_args(s, nullptr, expert_offsets, nullptr, nullptr, nullptr, w_down, nullptr, nullptr, s_down,
                            y_rows, static_cast<__bf16*>(const_cast<void*>(h)));
  if (workspace && need) {
    if (use_stream(s)) {
      a.part = static_cast<float*>(workspace);
    } else {
      a.claims_down = static_cast<unsigned long long*>(workspace);
    }
  }
  return run_down("moe_expert_down", s, a, stream);
}

moe_status moe_down_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = down_ws_bytes(shape);
  return MOE_OK;
}

moe_status moe_gate_up_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = gate_up_ws_bytes(shape);
  return MOE_OK;
}

moe_status moe_combine(const moe_shape* s, const float* y_rows, const int32_t* slot_to_row,
                       const float* topk_w, void* y, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(y_rows);
  REQUIRE_PTR(slot_to_row);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(y);
  if (debug_on() && (st = debug_rows(s, slot_to_row, stream)) != MOE_OK) return st;
  const hipError_t e = moe::launch_combine(y_rows, slot_to_row, topk_w, s->T, s->d, s->K,
                                           s->act_dtype == MOE_BF16, y, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

moe_status moe_forward(const moe_shape* s, const void* x, const void* router_w, const float* router_bias,
                       const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                       const void* s_up, const void* s_down, void* y, int32_t* topk_ids_out, float* topk_w_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return forward_impl("moe_forward", s, x, router_w, router_bias, w_gate, w_up, w_down, s_gate, s_up, s_down, y,
                      topk_ids_out, topk_w_out, workspace, workspace_bytes, stream);
}

moe_status moe_forward_noalloc(const moe_shape* s, const void* x, const void* router_w, const float* router_bias,
                               const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                               const void* s_up, const void* s_down, void* y, int32_t* topk_ids_out,
                               float* topk_w_out, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const size_t need = forward_layout(s).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc: this shape needs %zu bytes of scratch, more than the "
                "library's fixed %zu (use moe_forward with a caller workspace)", need, kScratchBytes);
  if (s->T == 0) return MOE_OK;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MOE_OK) return st;
  return forward_impl("moe_forward_noalloc", s, x, router_w, router_bias, w_gate, w_up, w_down, s_gate, s_up,
                      s_down, y, topk_ids_out, topk_w_out, ws, kScratchBytes, stream);
}

moe_status moe_mlp_workspace_size(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  if (shape->E != 1 || shape->K != 1) return fail(MOE_ERR_SHAPE, "the dense MLP needs E = K = 1");
  *bytes = forward_layout(shape).total;
  return MOE_OK;
}

moe_status moe_mlp_forward(const moe_shape* s, const void* x, const void* w_gate, const void* w_up,
                           const void* w_down, const void* s_gate, const void* s_up, const void* s_down, void* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_ffn(s);
  if (st != MOE_OK) return st;
  if (s->E != 1 || s->K != 1) return fail(MOE_ERR_SHAPE, "the dense MLP needs E = K = 1 (E=%d, K=%d)", s->E, s->K);
  if (s->T == 0) return MOE_OK;   // nothing is read or written
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_down);
  REQUIRE_SCALE(s, s_gate);
  REQUIRE_SCALE(s, s_up);
  REQUIRE_SCALE(s, s_down);
  REQUIRE_PTR(y);
  REQUIRE_PTR(workspace);
  const WsLayout L = forward_layout(s);
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  float* wts = reinterpret_cast<float*>(ws + L.w);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* s2r = reinterpret_cast<int32_t*>(ws + L.s2r);
  __bf16* h = reinterpret_cast<__bf16*>(ws + L.h);
  float* y_rows = reinterpret_cast<float*>(ws + L.y_rows);
  hipError_t e = moe::launch_dense_init(s->T, offsets, sorted, s2r, wts, stream);
  if (e != hipSuccess) return hip_fail(e, "dense init launch");
  moe::FfnArgs a = ffn_args(s, x, offsets, sorted, w_gate, w_up, w_down, s_gate, s_up, s_down, y_rows, h);
  if (L.part_bytes) a.part = reinterpret_cast<float*>(ws + L.part);
  if (!use_stream(s)) {
    a.claims_gate_up = reinterpret_cast<unsigned long long*>(ws + L.claims);
    a.claims_down = reinterpret_cast<unsigned long long*>(ws + L.claims + moe::kTileClaimBytes);
  }
  // with the down pass's reduction split over workgroups, the sum of its slices
  // is written to y directly (the combine of one expert of weight 1)
  if (L.part_bytes) a.y_dense = y;
  st = run_gate_up("moe_mlp_forward", s, a, stream);
  if (st != MOE_OK) return st;
  st = run_down("moe_mlp_forward", s, a, stream);
  if (st != MOE_OK || a.y_dense) return st;
  e = moe::launch_combine(y_rows, s2r, wts, s->T, s->d, 1, s->act_dtype == MOE_BF16, y, stream);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

moe_status moe_quantize_rows(int64_t rows, int32_t cols, int32_t src_dtype, const void* w, int32_t scale_dtype,
                             int8_t* q, void* s, hipStream_t stream) {
  const moe_status st = check_quantize(rows, cols, src_dtype, w, scale_dtype, q, s);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  const hipError_t e = moe::launch_quantize_rows(rows, cols, src_dtype == MOE_BF16, w, scale_dtype == MOE_BF16, q,
                                                 s, false, false, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return MOE_OK;
}

moe_status moe_quantize_rows_fp8(int64_t rows, int32_t cols, int32_t src_dtype, const void* w, int32_t scale_dtype,
                                 uint8_t* q, void* s, hipStream_t stream) {
  const moe_status st = check_quantize(rows, cols, src_dtype, w, scale_dtype, q, s);
  if (st != MOE_OK) return st;
  if (rows == 0) return MOE_OK;
  const hipError_t e = moe::launch_quantize_rows(rows, cols, src_dtype == MOE_BF16, w, scale_dtype == MOE_BF16,
                                                 reinterpret_cast<int8_t*>(q), s, true, false, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return MOE_OK;
}

moe_status moe_quantize_pack_rows(int64_t rows, int32_t cols, int32_t src_dtype, const void* w,
                                  int32_t scale_dtype, int32_t weight_fmt, void* q_tiled, void* s,
                                  hipStream_t stream) {
  moe_status st = check_quantize(rows, cols, src_dtype, w, scale_dtype, q_tiled, s);
  if (st != MOE_OK) return st;
  if (rows % 16 || cols % 64) return fail(MOE_ERR_SHAPE, "rows=%ld must be a multiple of 16 and cols=%d of 64", (long)rows, cols);
  if (weight_fmt != MOE_W_INT8 && weight_fmt != MOE_W_FP8)
    return fail(MOE_ERR_DTYPE, "weight_fmt=%d: only the int8 and fp8 encodings are quantized", weight_fmt);
  if (rows == 0) return MOE_OK;
  const hipError_t e = moe::launch_quantize_rows(rows, cols, src_dtype == MOE_BF16, w, scale_dtype == MOE_BF16,
                                                 static_cast<int8_t*>(q_tiled), s, weight_fmt == MOE_W_FP8, true,
                                                 stream);
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return MOE_OK;
}

moe_status moe_pack_rows(int64_t rows, int32_t cols, const int8_t* q, int8_t* packed, hipStream_t stream) {
  if (rows < 0 || rows % 16) return fail(MOE_ERR_SHAPE, "rows=%ld must be a non-negative multiple of 16", (long)rows);
  if (cols < 64 || cols > (1 << 20) || cols % 64) return fail(MOE_ERR_SHAPE, "cols=%d must be a multiple of 64 in [64, 2^20]", cols);
  if (rows * (int64_t)cols / 16 > 0x7fffffffL * 256L) return fail(MOE_ERR_SHAPE, "matrix too large");
  REQUIRE_PTR(q);
  REQUIRE_PTR(packed);
  if (q == packed) return fail(MOE_ERR_UNSUPPORTED, "packing cannot be done in place");
  if (rows == 0) return MOE_OK;
  const hipError_t e = moe::launch_pack_rows(rows, cols, q, packed, stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return MOE_OK;
}

}  // extern "C"
