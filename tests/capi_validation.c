/* Host-only driver of the C ABI's argument validation, built and run with
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_capi_asan.py.
 *
 * Every call below either fails validation or has nothing to do (M = 0), so
 * no call reaches the GPU: device pointers are aligned fake addresses that
 * are never dereferenced.  The size queries and the validation code run on
 * the host, where the sanitizers watch them.  Exit status 0 when every
 * status matches; the first mismatch is printed and exits with 1. */
#include <stdint.h>
#include <stdio.h>
#include <math.h>
#include <stdlib.h>

#include "../include/qlora.h"

static int failures = 0;

static void expect(int got, int want, const char *what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)
#define EXPECT_TRUE(cond) expect(!!(cond), 1, #cond, __LINE__)

static qlora_nf4_weight fake_weight(int64_t rows, int64_t cols, int32_t qtype) {
  qlora_nf4_weight w;
  w.packed = (uint8_t *)(uintptr_t)0x10000;
  w.code8 = (uint8_t *)(uintptr_t)0x11000;
  w.c2 = (float *)(uintptr_t)0x12000;
  w.mean = (float *)(uintptr_t)0x13000;
  w.rows = rows;
  w.cols = cols;
  w.qtype = qtype;
  return w;
}

int main(void) {
  void *P = (void *)(uintptr_t)0x20000;          /* aligned, never dereferenced */
  const float *PF = (const float *)P;
  const uint16_t *PH = (const uint16_t *)P;
  uint16_t *OH = (uint16_t *)P;
  const size_t BIG = (size_t)1 << 30;
  qlora_nf4_weight w = fake_weight(64, 64, QLORA_Q4_NF4);
  qlora_nf4_weight wk = fake_weight(64, 100, QLORA_Q4_NF4);     /* K % 64 != 0 */
  qlora_nf4_weight wn = fake_weight(60, 64, QLORA_Q4_NF4);      /* N % 8 != 0 */
  qlora_nf4_weight wbig = fake_weight((int64_t)1 << 20, (int64_t)1 << 20, QLORA_Q4_NF4);
  qlora_nf4_weight wbad = fake_weight(64, 64, 3);
  qlora_nf4_weight wmis = w;
  wmis.packed = (uint8_t *)(uintptr_t)0x10008;

  /* status strings and sizes */
  for (int s = -6; s <= 2; ++s) EXPECT_TRUE(qlora_status_string(s) != NULL);
  EXPECT(qlora_version(), 10000);
  int64_t pb = 0, nb = 0, nb2 = 0;
  EXPECT(qlora_nf4_sizes(64 * 257 + 3, &pb, &nb, &nb2), QLORA_OK);
  EXPECT_TRUE(pb == (64 * 257 + 4) / 2 && nb == 258 && nb2 == 2);
  EXPECT(qlora_nf4_sizes(0, &pb, &nb, &nb2), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_sizes(5, NULL, NULL, NULL), QLORA_OK);
  EXPECT_TRUE(qlora_quantize_workspace_bytes(0) == 0);
  EXPECT_TRUE(qlora_quantize_workspace_bytes((int64_t)22016 * 8192) > 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(8192, 11008, 4096, 64, 1) > 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(64, 11008, 4096, 64, 0) > 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(1, 4096, 4096, 64, 0) > 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(8, 4096, 4000, 64, 0) == 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(8, 4099, 4096, 64, 0) == 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(8, 4096, 4096, 129, 1) == 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes(-1, 4096, 4096, 64, 1) == 0);
  EXPECT_TRUE(qlora_linear_workspace_bytes((int64_t)1 << 40, 4096, 4096, 64, 1) == 0);
  EXPECT_TRUE(qlora_lora_grad_in_workspace_bytes(11008, 65) > 0);
  EXPECT_TRUE(qlora_lora_grads_workspace_bytes(8192, 11008, 4096, 100) > 0);
  EXPECT_TRUE(qlora_linear_dropout_workspace_bytes(8192, 4096, 4096, 64, 1) > 0);

  /* codec */
  EXPECT(qlora_quantize_nf4(NULL, &w, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_quantize_nf4(PF, NULL, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_quantize_nf4(PF, &w, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_quantize_nf4(PF, &w, P, 1, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_quantize_nf4(PF, &wbad, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_quantize_nf4(PF, &wbig, P, BIG, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_quantize_nf4_16(PH, 0, &w, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_quantize_nf4_16(PH, QLORA_IN_FP16, &w, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_dequantize_nf4(NULL, OH, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dequantize_nf4(&wmis, OH, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dequantize_nf4(&w, (uint16_t *)(uintptr_t)0x20002, NULL), QLORA_ERR_INVALID_ARG);

  /* linear layer */
  EXPECT(qlora_linear_fwd(PH, 8, &wk, PH, PH, 8, 1.0f, OH, OH, P, BIG, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_linear_fwd(PH, 8, &wn, PH, PH, 8, 1.0f, OH, OH, P, BIG, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_linear_fwd(PH, 8, &w, PH, PH, 0, 1.0f, OH, OH, P, BIG, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_linear_fwd(PH, -3, &w, PH, PH, 8, 1.0f, OH, OH, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_fwd(PH, 8, &w, PH, PH, 8, INFINITY, OH, OH, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_fwd(PH, 8, &w, PH, PH, 8, 1.0f, OH, NULL, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_linear_fwd(PH, 0, &w, PH, PH, 8, 1.0f, OH, OH, NULL, 0, NULL), QLORA_OK);
  EXPECT(qlora_linear_bwd(PH, PH, PH, 8, &w, PH, PH, 8, 1.0f, OH, OH, OH, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_linear_bwd(NULL, PH, PH, 8, &w, PH, PH, 8, 1.0f, OH, OH, OH, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_bwd(PH, PH, NULL, 0, &w, PH, PH, 8, 1.0f, NULL, NULL, NULL, P, BIG, NULL), QLORA_OK);
  EXPECT(qlora_lora_down(PH, 4, 60, PH, 8, 1.0f, OH, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_lora_down(PH, 0, 64, PH, 8, 1.0f, OH, NULL), QLORA_OK);
  EXPECT(qlora_nf4_matmul_fwd(PH, 8, &wk, PH, PH, 8, OH, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_nf4_matmul_dx(PH, 0, &w, PH, PH, 8, OH, NULL), QLORA_OK);
  EXPECT(qlora_lora_grad_in(PH, 4, 64, PH, 8, 1.0f, OH, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_lora_grads(PH, PH, PH, PH, 4, 64, 64, 8, OH, OH, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_lora_grads(PH, PH, PH, PH, 0, 64, 64, 8, OH, OH, P, BIG, NULL), QLORA_OK);
  /* M = 0: tensors with M rows may be NULL (empty storage), workspace-free forward */
  EXPECT(qlora_linear_fwd(NULL, 0, &w, PH, PH, 8, 1.0f, NULL, NULL, NULL, 0, NULL), QLORA_OK);
  EXPECT(qlora_linear_bwd(NULL, NULL, NULL, 0, &w, PH, PH, 8, 1.0f, NULL, OH, OH, P, BIG, NULL), QLORA_OK);
  EXPECT(qlora_lora_grads(NULL, NULL, NULL, NULL, 0, 64, 64, 8, OH, OH, P, BIG, NULL), QLORA_OK);
  EXPECT(qlora_lora_down(NULL, 0, 64, PH, 8, 1.0f, NULL, NULL), QLORA_OK);
  EXPECT(qlora_nf4_matmul_fwd(NULL, 0, &w, NULL, PH, 8, NULL, NULL), QLORA_OK);
  EXPECT(qlora_dropout_mask(NULL, 0, 64, 0.1f, 1, NULL, NULL, NULL), QLORA_OK);
  EXPECT(qlora_linear_fwd(NULL, 8, &w, PH, PH, 8, 1.0f, OH, OH, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_bwd(PH, PH, NULL, 0, &w, NULL, PH, 8, 1.0f, NULL, OH, OH, P, BIG, NULL),
         QLORA_ERR_INVALID_ARG);   /* A has r rows, not M: never NULL */

  /* the static-scratch forward: rejections and M = 0 happen before any HIP call */
  qlora_nf4_weight w64 = fake_weight(64, 64, QLORA_Q4_NF4);
  EXPECT(qlora_linear_fwd_noalloc(PH, 70000, &w64, PH, PH, 128, 1.0f, OH, NULL, NULL), QLORA_ERR_SCRATCH_LIMIT);
  EXPECT(qlora_linear_fwd_noalloc(PH, 8, &wk, PH, PH, 8, 1.0f, OH, NULL, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_linear_fwd_noalloc(NULL, 0, &w64, PH, PH, 8, 1.0f, NULL, NULL, NULL), QLORA_OK);
  EXPECT_TRUE(qlora_status_string(QLORA_ERR_SCRATCH_LIMIT)[0] != 0);

  /* grouped forward: descriptors read on the host */
  qlora_linear_desc d[9];
  for (int i = 0; i < 9; ++i) {
    d[i].X = PH;
    d[i].W = &w;
    d[i].A = PH;
    d[i].B = PH;
    d[i].r = 8;
    d[i].scale = 1.0f;
    d[i].Y = OH;
    d[i].T_out = NULL;
  }
  EXPECT_TRUE(qlora_linear_group_workspace_bytes(8, d, 16) > 0);
  EXPECT_TRUE(qlora_linear_group_workspace_bytes(9, d, 16) == 0);
  EXPECT(qlora_linear_fwd_group(9, d, 16, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_fwd_group(8, d, 16, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  EXPECT(qlora_linear_fwd_group(8, d, 0, P, BIG, NULL), QLORA_OK);
  d[3].W = NULL;
  EXPECT(qlora_linear_fwd_group(8, d, 16, P, BIG, NULL), QLORA_ERR_INVALID_ARG);
  d[3].W = &wk;
  EXPECT(qlora_linear_fwd_group(8, d, 16, P, BIG, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);

  /* shared-input products: member arrays read on the host */
  const uint16_t *As[8] = {PH, PH, PH, PH, PH, PH, PH, PH};
  uint16_t *Ts[8] = {OH, OH, OH, OH, OH, OH, OH, OH};
  int32_t rs[8] = {64, 64, 64, 8, 16, 24, 32, 128};
  float sc[8] = {1, 1, 1, 1, 1, 1, 1, 1};
  EXPECT_TRUE(qlora_lora_dA_shared_workspace_bytes(8192, 4096, 8, rs) > 0);
  EXPECT(qlora_lora_down_shared(PH, 8, 64, 9, As, rs, sc, Ts, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_lora_down_shared(PH, 0, 64, 8, As, rs, sc, Ts, NULL), QLORA_OK);
  EXPECT(qlora_lora_dA_shared(PH, 8, 64, 8, As, rs, Ts, NULL, 0, NULL), QLORA_ERR_WORKSPACE);
  rs[5] = 129;
  EXPECT(qlora_lora_down_shared(PH, 8, 64, 8, As, rs, sc, Ts, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);

  /* dropout */
  EXPECT(qlora_dropout_mask(PH, 8, 64, 1.0f, 1, OH, (uint32_t *)P, NULL), QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dropout_mask(PH, 8, 48, 0.1f, 1, OH, (uint32_t *)P, NULL), QLORA_ERR_UNSUPPORTED_SHAPE);
  EXPECT(qlora_dropout_apply(PH, 0, 64, (const uint32_t *)P, OH, NULL), QLORA_OK);
  EXPECT(qlora_linear_fwd_dropout(PH, 8, &w, PH, PH, 8, 1.0f, 0.1f, 1, OH, NULL, (uint32_t *)P, NULL, 0, NULL),
         QLORA_ERR_WORKSPACE);
  EXPECT(qlora_linear_bwd_dropout(PH, PH, NULL, 8, &w, PH, PH, 8, 1.0f, 0.1f, NULL, OH, OH, OH, P, BIG, NULL),
         QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_matmul_dx_dropout(PH, 8, &wn, PH, PH, 8, (const uint32_t *)P, OH, NULL),
         QLORA_ERR_UNSUPPORTED_SHAPE);

  if (failures) {
    fprintf(stderr, "%d validation mismatches\n", failures);
    return 1;
  }
  printf("capi validation ok\n");
  return 0;
}
