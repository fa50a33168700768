/*
 * moe_int8.h -- C ABI of libmoe_int8.so: the forward pass of a mixture-of-experts
 * feed-forward layer whose expert weights are stored as int8 (MI355X / gfx950).
 *
 * What the layer computes (Jamba-1.5 paper, "Model Architecture"): an MoE module
 * stands in for the MLP; a router scores n experts per token and the top K are
 * used (n=16, K=2 in Jamba). "Serving Considerations and Improvements" (the
 * ExpertsInt8 scheme): expert weights live in memory as INT8, are turned back
 * into BF16 values inside the fused MoE kernel, and activations stay BF16.
 *
 * Readings of what the paper leaves open, implemented by every call below:
 *   gate    p = softmax(l) over all E logits l = x . router_w[e] (+ bias[e]);
 *           the K largest logits, descending, exact ties to the lower index;
 *           w_k = p_k / sum of p over the K chosen experts.
 *   expert  SwiGLU: o = s_d * (q_d . h), h = silu(g) * u,
 *           g = s_g * (q_g . x), u = s_u * (q_u . x); no biases.
 *   int8    symmetric, one scale per output channel (row of an (out, in)
 *           matrix); moe_quantize_rows below produces the codes and scales.
 *   combine y_t = sum_k w_k * o_{t,k}; no capacity limit, no residual.
 * The contractions run on bf16 MFMA with fp32 accumulation: int8 codes become
 * bf16 exactly, activations given as fp32 are rounded to bf16 at the MFMA input,
 * the per-channel scale is applied to the fp32 sum, h is held as bf16, the
 * per-slot expert outputs (y_rows) as fp32.
 *
 * Conventions (all calls):
 *   - Pointers named x, router_w, y, w_*, s_*, topk_*, expert_offsets,
 *     sorted_slots, slot_to_row, y_rows and workspace are DEVICE pointers on
 *     the current HIP device, row-major, 16-byte aligned. The caller owns
 *     every buffer; the library allocates nothing and keeps no state between
 *     calls, so calls on different streams may run concurrently.
 *   - Work is enqueued on `stream` and is asynchronous; no call synchronises.
 *   - Arguments are validated before anything is enqueued. On error nothing is
 *     launched and a moe_status other than MOE_OK is returned; the message is
 *     available from moe_last_error() on the calling thread. A launch failure
 *     reported by HIP maps to MOE_ERR_HIP. Device-side faults surface at the
 *     caller's next synchronisation.
 *   - Expert weights are (out, in) matrices w_gate, w_up [E, f, d] and
 *     w_down [E, d, f] in the encoding shape->weight_fmt names (int8 unless
 *     stated), held by the FFN calls in the TILED LAYOUT that moe_pack_rows
 *     produces (see there). router_w [E, d] is row-major; scales
 *     s_gate, s_up [E, f], s_down [E, d] are row-major.
 *   - Slots: token t's k-th choice is slot s = t*K + k.
 *   - T = 0 is valid and enqueues nothing; once the shape is valid, no
 *     pointer is then checked (empty tensors may be NULL).
 *   - Debug checks: while the environment variable MOE_DEBUG is set (to a
 *     value other than "0"), the calls that take or produce a permutation
 *     also check it, on the host:
 *       moe_expert_ffn, moe_expert_gate_up, moe_expert_down: expert_offsets
 *         starts at 0, never decreases and ends at most at T*K; for the first
 *         two, the sorted rows below off[E] hold distinct slots in [0, T*K);
 *       moe_combine: every slot_to_row entry is -1 or in [0, T*K);
 *       these run BEFORE anything is launched, so bad caller arrays are
 *       reported instead of being read out of bounds by a kernel;
 *       moe_permute, moe_forward, moe_forward_noalloc: after the permutation
 *         is computed, also that every id is in [0, E) (all slots placed),
 *         that each expert's rows hold its own slots in ascending order and
 *         that slot_to_row inverts sorted_slots.
 *     A failed check returns MOE_ERR_CHECK (moe_forward: before the down
 *     pass). The checks copy the arrays to the host and synchronise `stream`:
 *     they are for debugging, not for timed runs or graph capture.
 *   - Logging: while the environment variable MOE_LOG is set (to a value
 *     other than "0"), every call that runs an expert-FFN pass writes one line
 *     per pass to stderr ("[moe] <call> gate/up|down: <shape>; <schedule>"):
 *     the schedule (stream or tiled), and for the stream schedule the rows per
 *     pass, where the expert segments come from, and whether the down pass
 *     splits its reduction over workgroups. Nothing else changes.
 */
#ifndef MOE_INT8_H
#define MOE_INT8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or not a supported multiple */
  MOE_ERR_DTYPE = 3,       /* unknown dtype code */
  MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  MOE_ERR_UNSUPPORTED = 6, /* valid request the library does not support */
  MOE_ERR_HIP = 7,         /* a HIP runtime call failed */
  MOE_ERR_CHECK = 8        /* a MOE_DEBUG consistency check failed */
};

/* dtype codes */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* Expert weight encodings (moe_shape.weight_fmt). MOE_W_INT8 is the layer
 * itself (ExpertsInt8). The other two are comparators for the paper's claims
 * ("Serving Considerations and Improvements": in-kernel INT8 dequantization is
 * faster than BF16 weights and as fast as FP8):
 *   MOE_W_INT8  int8 codes + per-output-channel scales (moe_quantize_rows);
 *   MOE_W_BF16  the bf16 weights themselves, no scales (s_* unused, may be NULL);
 *   MOE_W_FP8   OCP fp8 e4m3 codes + per-output-channel scales
 *               (moe_quantize_rows_fp8); every e4m3 value is exact in bf16.
 * All three are held in the tiled layout of their bytes (moe_pack_rows; a
 * bf16 matrix [rows, cols] is packed as int8 [rows, 2*cols]). The bf16 and
 * fp8 encodings need bf16 activations; on the TILED schedule their tensors
 * must also fit 32-bit byte offsets (x and h below 4 GiB, one expert's matrix
 * below 4 GiB), else MOE_ERR_UNSUPPORTED. */
enum { MOE_W_INT8 = 0, MOE_W_BF16 = 1, MOE_W_FP8 = 2 };

/* expert-FFN schedule: AUTO picks STREAM when at most 64 rows fall on each
 * expert on average (T*K <= 64*E: decode) and TILED otherwise (prefill).
 * Both give results within the same tolerance of the exact layer; they are
 * not bit-identical to each other. Each is deterministic. */
enum { MOE_PATH_AUTO = 0, MOE_PATH_STREAM = 1, MOE_PATH_TILED = 2 };

typedef struct moe_shape {
  int32_t T;           /* tokens, >= 0                                     */
  int32_t d;           /* hidden size, multiple of 64, 64..65536            */
  int32_t f;           /* expert FFN width, multiple of 64, 64..131072      */
  int32_t E;           /* experts, 1..64                                    */
  int32_t K;           /* experts per token, 1..min(E, 8)                   */
  int32_t act_dtype;   /* x, router_w, y: MOE_F32 or MOE_BF16               */
  int32_t scale_dtype; /* s_gate, s_up, s_down: MOE_F32 or MOE_BF16         */
  int32_t ffn_path;    /* MOE_PATH_*                                        */
  int32_t weight_fmt;  /* MOE_W_*: encoding of w_gate, w_up, w_down        */
} moe_shape;

/* ABI version of this header (bumped on any signature change). */
#define MOE_ABI_VERSION 6
int32_t moe_abi_version(void);

/* Static description of a status code. */
const char* moe_status_str(moe_status status);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Workspace, in bytes, that moe_forward needs for this shape (includes the
 * routing buffers, the permutation, h, y_rows and the FFN passes' own
 * workspaces, see moe_gate_up_workspace_size and moe_down_workspace_size). */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/* Workspace, in bytes, that moe_expert_ffn needs: h (T*K*f bf16), then the
 * down pass's workspace (moe_down_workspace_size), then the gate/up pass's
 * (moe_gate_up_workspace_size), each padded to 256. */
moe_status moe_ffn_workspace_size(const moe_shape* shape, size_t* bytes);

/* Workspace, in bytes, that the down pass can use:
 *   - STREAM schedule: fp32 partial sums [planes, T*K, d] for shapes whose
 *     weight-streaming down pass splits its reduction over workgroups (33 to
 *     64 rows per expert on average and too few output-channel groups to fill
 *     the GPU, e.g. a dense MLP at decode); 0 for every other stream shape;
 *   - TILED schedule: 256 bytes of tile claim words (see moe_expert_down). */
moe_status moe_down_workspace_size(const moe_shape* shape, size_t* bytes);

/* Workspace, in bytes, that the gate/up pass can use: 256 bytes of tile claim
 * words on the TILED schedule, 0 on the STREAM schedule (see moe_expert_gate_up). */
moe_status moe_gate_up_workspace_size(const moe_shape* shape, size_t* bytes);

/* Router and gate (paper: "Model Architecture", top K of n experts per token).
 *   x           [T, d]  act_dtype
 *   router_w    [E, d]  act_dtype
 *   router_bias [E] fp32 added to the logits, or NULL
 *   topk_ids    [T, K] int32 out: chosen experts, descending logit
 *   topk_w      [T, K] fp32  out: renormalised gate weights (sum to 1 per token)
 * Logits are fp32 dot products of the exact inputs. */
moe_status moe_route(const moe_shape* shape, const void* x, const void* router_w,
                     const float* router_bias, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream);

/* Group the T*K slots by expert (stable: ascending slot inside an expert).
 * Source: Jamba-1.5 paper, "Model Architecture": each token is sent to the
 * top K of n experts, so every expert sees its own subset of the tokens; this
 * call gathers each expert's slots into one contiguous segment.
 *   topk_ids       [T*K] int32 in, values in [0, E)
 *   expert_offsets [E+1] int32 out: expert e owns sorted rows [off[e], off[e+1])
 *   sorted_slots   [T*K] int32 out: slot held by each sorted row
 *   slot_to_row    [T*K] int32 out: sorted row of each slot
 * An id outside [0, E) is not placed: its slot_to_row entry is -1 and the
 * sorted rows past off[E] hold -1. Bit-exact and deterministic. */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* sorted_slots,
                       int32_t* slot_to_row, hipStream_t stream);

/* Expert SwiGLU FFNs on the permuted rows (the ExpertsInt8 contraction).
 * Source: Jamba-1.5 paper, "Serving Considerations and Improvements": the
 * expert weights stay INT8 in memory and become BF16 values inside the fused
 * MoE kernel, right before the contraction; activations stay BF16.
 *   x              [T, d] act_dtype (row of sorted row r is token sorted_slots[r] / K)
 *   expert_offsets [E+1], sorted_slots [T*K] from moe_permute
 *   w_gate, w_up   [E, f, d];  w_down [E, d, f] -- shape->weight_fmt encoding, tiled layout (moe_pack_rows)
 *   s_gate, s_up   [E, f] scale_dtype;  s_down [E, d] scale_dtype (unused for MOE_W_BF16)
 *   y_rows         [T*K, d] fp32 out: row r = output of sorted row r's expert
 *   workspace      >= moe_ffn_workspace_size bytes (holds h and the down pass's partial sums)
 * Rows past off[E] are left untouched. */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x,
                          const int32_t* expert_offsets, const int32_t* sorted_slots,
                          const void* w_gate, const void* w_up, const void* w_down,
                          const void* s_gate, const void* s_up, const void* s_down,
                          float* y_rows, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* The two passes of moe_expert_ffn, callable on their own (same kernels;
 * source as moe_expert_ffn: Jamba-1.5 paper, "Serving Considerations and
 * Improvements"):
 * gate/up  h[r] = silu(s_g * (q_g . x_r)) * (s_u * (q_u . x_r))  for every sorted row r,
 *          h [T*K, f] bf16 out (rows past off[E] untouched).
 * down     y_rows[r] = s_d * (q_d . h[r]),  h [T*K, f] bf16 in, y_rows [T*K, d] fp32 out.
 * workspace (both passes): NULL, or 16-byte aligned and at least
 *          moe_gate_up_workspace_size / moe_down_workspace_size bytes (else
 *          MOE_ERR_ALIGN / MOE_ERR_WORKSPACE). Its contents need not be
 *          initialised. With it:
 *          - on the TILED schedule, the last tiles of each XCD's share are
 *            claimed through atomic counters in the workspace (cleared by the
 *            pass itself) by the workgroups of any XCD, so XCDs that run
 *            faster take more tiles; without it every workgroup's tile is
 *            fixed by its id;
 *          - on the STREAM schedule, a down pass that splits its reduction
 *            may spread the slices over workgroups (partial sums in the
 *            workspace, added in slice order by a second kernel); without it
 *            the slices stay inside one workgroup.
 *          The results are the same bit for bit either way.
 * moe_expert_ffn is moe_expert_gate_up followed by moe_expert_down on the same
 * stream, with the parts of its workspace after h as their workspaces. */
moe_status moe_expert_gate_up(const moe_shape* shape, const void* x, const int32_t* expert_offsets,
                              const int32_t* sorted_slots, const void* w_gate, const void* w_up,
                              const void* s_gate, const void* s_up, void* h, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);
moe_status moe_expert_down(const moe_shape* shape, const void* h, const int32_t* expert_offsets,
                           const void* w_down, const void* s_down, float* y_rows, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Weighted combine back to token order: y[t] = sum_k topk_w[t,k] * y_rows[slot_to_row[t*K+k]]
 * Source: Jamba-1.5 paper, "Model Architecture": the MoE module takes the
 * place of the MLP, so its output is the gate-weighted sum of the K chosen
 * experts' outputs, one [d] vector per token.
 * (k ascending, fp32, no atomics); a slot with row -1 contributes nothing.
 *   y [T, d] act_dtype out. */
moe_status moe_combine(const moe_shape* shape, const float* y_rows, const int32_t* slot_to_row,
                       const float* topk_w, void* y, hipStream_t stream);

/* The whole layer: route, permute, expert FFN, combine, enqueued on `stream`.
 * Sources: Jamba-1.5 paper, "Model Architecture" (an MoE module with n
 * experts, top K per token, in place of the MLP) and "Serving Considerations
 * and Improvements" (ExpertsInt8: int8 expert weights dequantized to BF16
 * inside the fused kernel).
 * Bit-identical to the four staged calls above with the same ffn_path.
 *   topk_ids_out [T, K] / topk_w_out [T, K]: optional copies of the routing (NULL to skip)
 *   workspace    >= moe_workspace_size bytes */
moe_status moe_forward(const moe_shape* shape, const void* x, const void* router_w,
                       const float* router_bias,
                       const void* w_gate, const void* w_up, const void* w_down,
                       const void* s_gate, const void* s_up, const void* s_down,
                       void* y, int32_t* topk_ids_out, float* topk_w_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments and results as moe_forward (bit for
 * bit), minus the workspace: the library keeps a fixed 32 MiB scratch array in
 * device memory on each GPU it runs on (held until the process ends) and uses
 * it as the workspace. A shape whose moe_workspace_size exceeds 32 MiB is
 * rejected with MOE_ERR_WORKSPACE before anything is enqueued (every
 * decode-sized layer fits: Jamba-1.5-Large at T=64 needs about 11 MiB). The
 * call allocates nothing. All calls on one GPU share that GPU's scratch, which
 * keeps the last call's contents: calls that overlap on one GPU (concurrent
 * streams, or host threads) race and must be serialised by the caller. */
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const void* router_w,
                               const float* router_bias,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const void* s_gate, const void* s_up, const void* s_down,
                               void* y, int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream);

/* Dense int8-weight MLP (Jamba-1.5 paper, "Serving Considerations and
 * Improvements": ExpertsInt8 quantizes the MoE *and* the MLP weights). An MLP
 * layer is the MoE layer with one expert used by every token with weight 1:
 *   y = s_d * (q_d . h),  h = silu(s_g * (q_g . x)) * (s_u * (q_u . x)).
 * shape->E and shape->K must be 1; no router. Same kernels, weight encodings
 * and layouts as the MoE calls, same tolerance; the result is bitwise that of
 * moe_expert_ffn followed by moe_combine with weight 1 (when the down pass
 * splits its reduction over workgroups, the kernel that adds the slices
 * writes y itself).
 *   y [T, d] act_dtype out; workspace >= moe_mlp_workspace_size bytes. */
moe_status moe_mlp_workspace_size(const moe_shape* shape, size_t* bytes);
moe_status moe_mlp_forward(const moe_shape* shape, const void* x,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down, void* y,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ExpertsInt8 quantizer (paper: "Serving Considerations and Improvements":
 * quantized at load time in seconds, no calibration). Row-wise symmetric int8:
 *   a = max_i |w[r, i]|,  s[r] = a / 127 rounded once (nearest-even) to scale_dtype,
 *   q[r, i] = round-half-even(w[r, i] / s[r]) clamped to [-127, 127];
 *   an all-zero row gives s = 0 and q = 0.
 *   w [rows, cols] src_dtype (MOE_F32 or MOE_BF16), q [rows, cols] int8, s [rows].
 * Quantizing an (out, in) weight [E, out, in] is rows = E*out, cols = in.
 * cols must be a multiple of 16, 16..1048576. Non-finite inputs give
 * unspecified codes. Bit-exact (the rounding decisions are exact). */
moe_status moe_quantize_rows(int64_t rows, int32_t cols, int32_t src_dtype, const void* w,
                             int32_t scale_dtype, int8_t* q, void* s, hipStream_t stream);

/* FP8 comparator quantizer: as moe_quantize_rows with OCP e4m3 codes (the
 * paper compares ExpertsInt8 with FP8 weights, "Serving Considerations and
 * Improvements"). Row-wise symmetric, one scale per output channel:
 *   s[r] = max_i |w[r, i]| / 448 rounded once (nearest-even) to scale_dtype,
 *   q[r, i] = byte of the e4m3 value nearest to w[r, i] / s[r] (ties to the
 *   even mantissa), saturated to +-448; a zero value is byte 0x00;
 *   an all-zero row gives s = 0 and q = 0.
 * e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals m*2^-9,
 * largest finite 448, bytes 0x7F/0xFF NaN (never produced).
 * Same sizes, dtypes and errors as moe_quantize_rows. Bit-exact. */
moe_status moe_quantize_rows_fp8(int64_t rows, int32_t cols, int32_t src_dtype, const void* w,
                                 int32_t scale_dtype, uint8_t* q, void* s, hipStream_t stream);

/* Quantizer and packer in one pass (load time: "Serving Considerations and
 * Improvements", quantized in seconds when the model is loaded): the codes of
 * moe_quantize_rows (weight_fmt MOE_W_INT8) or moe_quantize_rows_fp8
 * (MOE_W_FP8), written straight into the tiled layout of moe_pack_rows, so
 * the weights are read and the codes written once. Same scales, same codes
 * bit for bit as quantizing then packing.
 *   w [rows, cols] src_dtype in (rows % 16 == 0, cols % 64 == 0),
 *   q_tiled [rows*cols] bytes out (tiled layout), s [rows] scale_dtype out.
 * Errors as moe_quantize_rows; other weight_fmt values: MOE_ERR_DTYPE. */
moe_status moe_quantize_pack_rows(int64_t rows, int32_t cols, int32_t src_dtype, const void* w,
                                  int32_t scale_dtype, int32_t weight_fmt, void* q_tiled, void* s,
                                  hipStream_t stream);

/* Tiled int8 layout of the expert weights (load time, next to the quantizer).
 * The kernels read a wavefront's MFMA operands as whole 1 KiB blocks: a
 * row-major int8 matrix q [rows, cols] (rows % 16 == 0, cols % 64 == 0) is
 * stored as blocks of 16 rows x 64 columns; block (rg, ks) covers rows
 * 16*rg..+16 and columns 64*ks..+64 and sits at block index rg*(cols/64) + ks;
 * inside it, element (r, c) is byte 256*(c/16) + 16*r + (c%16). An expert
 * tensor [E, out, in] is packed as rows = E*out, cols = in.
 *   q [rows, cols] int8 row-major in, packed [rows*cols] int8 out (not in place).
 * A byte permutation: bit-exact. */
moe_status moe_pack_rows(int64_t rows, int32_t cols, const int8_t* q, int8_t* packed, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_INT8_H */
