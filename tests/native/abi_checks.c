/* Host-side checks of the C ABI's argument validation, built with the address
 * and undefined-behaviour sanitizers on the host code (no GPU: every call here
 * returns before anything is enqueued). Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_int8.h"

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static moe_shape shape(int T, int d, int f, int E, int K, int path) {
  moe_shape s;
  s.T = T; s.d = d; s.f = f; s.E = E; s.K = K;
  s.act_dtype = MOE_BF16; s.scale_dtype = MOE_BF16; s.ffn_path = path; s.weight_fmt = MOE_W_INT8;
  return s;
}

int main(void) {
  /* fake, 256-aligned device addresses: validation never dereferences them */
  void* A = (void*)(uintptr_t)0x10000;
  void* MIS = (void*)(uintptr_t)0x10008;
  size_t n = 0;

  CHECK(moe_abi_version() == MOE_ABI_VERSION);
  for (int st = -3; st < 12; ++st) CHECK(moe_status_str(st) != NULL && strlen(moe_status_str(st)) > 0);

  /* shapes out of range, every size query */
  const int bad[][5] = {{-1, 256, 512, 16, 2}, {8, 100, 512, 16, 2}, {8, 256, 96, 16, 2}, {8, 256, 512, 0, 2},
                        {8, 256, 512, 65, 2}, {8, 256, 512, 4, 5}, {8, 256, 512, 16, 9}, {8, 131072, 512, 16, 2},
                        {1 << 30, 256, 512, 16, 2}};
  for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
    moe_shape s = shape(bad[i][0], bad[i][1], bad[i][2], bad[i][3], bad[i][4], MOE_PATH_AUTO);
    CHECK(moe_workspace_size(&s, &n) == MOE_ERR_SHAPE);
    CHECK(moe_ffn_workspace_size(&s, &n) == MOE_ERR_SHAPE);
    CHECK(moe_down_workspace_size(&s, &n) == MOE_ERR_SHAPE);
    CHECK(moe_gate_up_workspace_size(&s, &n) == MOE_ERR_SHAPE);
    CHECK(strlen(moe_last_error()) > 0);
    CHECK(moe_forward(&s, A, A, NULL, A, A, A, A, A, A, A, NULL, NULL, A, (size_t)1 << 40, NULL) == MOE_ERR_SHAPE);
  }
  moe_shape s = shape(64, 256, 512, 16, 2, MOE_PATH_AUTO);
  CHECK(moe_workspace_size(NULL, &n) == MOE_ERR_NULL);
  CHECK(moe_workspace_size(&s, NULL) == MOE_ERR_NULL);
  s.act_dtype = 7;
  CHECK(moe_route(&s, A, A, NULL, A, A, NULL) == MOE_ERR_DTYPE);
  s.act_dtype = MOE_BF16;
  s.weight_fmt = 9;
  CHECK(moe_expert_ffn(&s, A, A, A, A, A, A, A, A, A, A, A, (size_t)1 << 30, NULL) == MOE_ERR_DTYPE);
  s.weight_fmt = MOE_W_INT8;

  /* null and misaligned pointers, short workspaces */
  CHECK(moe_route(&s, NULL, A, NULL, A, A, NULL) == MOE_ERR_NULL);
  CHECK(moe_route(&s, MIS, A, NULL, A, A, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_route(&s, A, A, (const float*)MIS, A, A, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_permute(&s, A, NULL, A, A, NULL) == MOE_ERR_NULL);
  CHECK(moe_combine(&s, A, A, A, MIS, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_workspace_size(&s, &n) == MOE_OK && n > 0);
  CHECK(moe_forward(&s, A, A, NULL, A, A, A, A, A, A, A, NULL, NULL, A, n - 1, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_forward(&s, A, A, NULL, A, A, A, A, A, MIS, A, NULL, NULL, A, n, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_ffn_workspace_size(&s, &n) == MOE_OK);
  CHECK(moe_expert_ffn(&s, A, A, A, A, A, A, A, A, A, A, A, n - 1, NULL) == MOE_ERR_WORKSPACE);
  moe_shape t = shape(512, 256, 512, 4, 2, MOE_PATH_TILED);
  CHECK(moe_gate_up_workspace_size(&t, &n) == MOE_OK && n == 256);
  CHECK(moe_expert_gate_up(&t, A, A, A, A, A, A, A, A, A, 255, NULL) == MOE_ERR_WORKSPACE);
  CHECK(moe_expert_gate_up(&t, A, A, A, A, A, A, A, A, MIS, 256, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_down_workspace_size(&t, &n) == MOE_OK && n == 256);
  CHECK(moe_expert_down(&t, A, A, A, A, A, A, 255, NULL) == MOE_ERR_WORKSPACE);
  moe_shape mlp = shape(8, 256, 512, 2, 1, MOE_PATH_AUTO);
  CHECK(moe_mlp_workspace_size(&mlp, &n) == MOE_ERR_SHAPE);
  CHECK(moe_mlp_forward(&mlp, A, A, A, A, A, A, A, A, A, (size_t)1 << 30, NULL) == MOE_ERR_SHAPE);

  /* the comparator encodings need bf16 activations */
  moe_shape c = shape(8, 256, 512, 16, 2, MOE_PATH_AUTO);
  c.act_dtype = MOE_F32;
  c.weight_fmt = MOE_W_FP8;
  CHECK(moe_forward(&c, A, A, NULL, A, A, A, A, A, A, A, NULL, NULL, A, (size_t)1 << 30, NULL) == MOE_ERR_UNSUPPORTED);

  /* the allocation-free forward: oversized shapes rejected, T = 0 accepted */
  moe_shape big = shape(40000, 128, 192, 4, 2, MOE_PATH_AUTO);
  CHECK(moe_forward_noalloc(&big, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
        MOE_ERR_WORKSPACE);
  moe_shape zero = shape(0, 256, 512, 16, 2, MOE_PATH_AUTO);
  CHECK(moe_forward_noalloc(&zero, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
        MOE_OK);

  /* T = 0: every call returns MOE_OK and reads no pointer */
  CHECK(moe_route(&zero, NULL, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_permute(&zero, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_expert_ffn(&zero, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);
  CHECK(moe_expert_gate_up(&zero, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);
  CHECK(moe_expert_down(&zero, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);
  CHECK(moe_combine(&zero, NULL, NULL, NULL, NULL, NULL) == MOE_OK);
  CHECK(moe_forward(&zero, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        MOE_OK);

  /* quantizer and packing arguments */
  CHECK(moe_quantize_rows(-1, 64, MOE_BF16, A, MOE_BF16, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_quantize_rows(16, 24, MOE_BF16, A, MOE_BF16, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_quantize_rows(16, 64, 5, A, MOE_BF16, A, A, NULL) == MOE_ERR_DTYPE);
  CHECK(moe_quantize_rows(16, 64, MOE_BF16, NULL, MOE_BF16, A, A, NULL) == MOE_ERR_NULL);
  CHECK(moe_quantize_rows(16, 64, MOE_BF16, A, MOE_BF16, A, (char*)A + 2, NULL) == MOE_ERR_ALIGN);
  CHECK(moe_quantize_rows_fp8(16, 64, MOE_BF16, A, MOE_BF16, NULL, A, NULL) == MOE_ERR_NULL);
  CHECK(moe_quantize_rows(0, 64, MOE_BF16, A, MOE_BF16, A, A, NULL) == MOE_OK);
  CHECK(moe_quantize_pack_rows(24, 64, MOE_BF16, A, MOE_BF16, MOE_W_INT8, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_quantize_pack_rows(32, 80, MOE_BF16, A, MOE_BF16, MOE_W_INT8, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_quantize_pack_rows(32, 64, MOE_BF16, A, MOE_BF16, MOE_W_BF16, A, A, NULL) == MOE_ERR_DTYPE);
  CHECK(moe_quantize_pack_rows(32, 64, MOE_BF16, A, MOE_BF16, MOE_W_FP8, NULL, A, NULL) == MOE_ERR_NULL);
  CHECK(moe_quantize_pack_rows(0, 64, MOE_BF16, A, MOE_BF16, MOE_W_FP8, A, A, NULL) == MOE_OK);
  CHECK(moe_pack_rows(17, 64, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_pack_rows(16, 96, A, A, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_pack_rows(16, 64, A, A, NULL) == MOE_ERR_UNSUPPORTED);   /* in place */
  CHECK(moe_pack_rows(0, 64, A, (int8_t*)A + 1024, NULL) == MOE_OK);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi checks ok\n");
  return 0;
}
